"""GPU parity of the bias-update variants beside Quantile Balancing, through
the C ABI: the margin form of QB (lmoe_qb_margin_update: histograms and solved
bias bit-exact against the oracle on identical fp32 scores and bias) and the
K2-style fixed-step update (lmoe_bias_signsgd: bias bit-exact against the
oracle on identical top-k lists).

Sources: "Kimi K3 Architecture Deep Dive" §3; LeiPhone report "Keeping the
numbers in range"; "Inside K3", section Quantile Balancing."""
import numpy as np
import pytest
import torch

import sparse_moe_layer_down_amd as lmoe
import synth
from oracle import ref

pytestmark = pytest.mark.gpu


def host_scores(T, n, seed, skew=0.0):
    z = synth.host_fill(T * n, seed, synth.TID["scores"], 0, 1.5).astype(np.float64).reshape(T, n)
    if skew:
        z = z + skew * (1.0 + np.arange(n))[None, :] ** -1.1
    return ref.sigmoid(z).astype(np.float32)


def same_bits(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


def gpu_margin(s, k, nbins, bias, hist=None, accumulate=False, solve=True):
    dev = torch.device("cuda:0")
    n = s.shape[1]
    h = torch.empty((n, nbins), dtype=torch.int32, device=dev) if hist is None else \
        torch.from_numpy(np.ascontiguousarray(hist, dtype=np.int32)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).to(dev)
    lmoe.qb_margin_update(torch.from_numpy(s).to(dev), k, h, b, accumulate=accumulate, solve=solve)
    torch.cuda.synchronize()
    return h.cpu().numpy().astype(np.int64), b.cpu().numpy()


@pytest.mark.parametrize("T,n,k,nbins,bias_scale", [
    (64, 16, 4, 1000, 0.0), (4096, 128, 8, 1000, 0.05), (777, 100, 3, 37, 0.1),   # n % 4 != 0: scalar path
    (300, 896, 16, 10000, 0.02), (513, 896, 16, 1000, 0.0), (40, 24, 24, 1000, 0.1),  # k == n: tau_k1 = -inf
    (5, 3, 1, 1, 0.0), (200, 1024, 64, 1000, 0.01),
])
def test_margin_update_bit_exact(T, n, k, nbins, bias_scale):
    s = host_scores(T, n, seed=T + 7 * n, skew=1.0)
    s[0, 0] = 1.0
    s[min(1, T - 1), min(1, n - 1)] = 0.0
    b = (np.random.default_rng(n).standard_normal(n) * bias_scale).astype(np.float32)
    h, bn = gpu_margin(s, k, nbins, b)
    H, B = ref.margin_update(s, nbins, k, b)
    assert np.array_equal(h, H)
    assert same_bits(bn, B)


def test_margin_update_with_exact_ties():
    """Scores and bias on a 2^-8 grid: many keys tie with the k-th and (k+1)-th."""
    rng = np.random.default_rng(3)
    T, n, k, nbins = 1000, 64, 6, 1000
    s = (rng.integers(1, 256, (T, n)) / 256.0).astype(np.float32)
    b = (rng.integers(-4, 4, n) / 256.0).astype(np.float32)
    h, bn = gpu_margin(s, k, nbins, b)
    H, B = ref.margin_update(s, nbins, k, b)
    assert np.array_equal(h, H)
    assert same_bits(bn, B)


def test_margin_accumulate_is_the_cross_batch_sum():
    n, k, nbins = 896, 16, 1000
    a = host_scores(3000, n, seed=1, skew=2.0)
    c = host_scores(5000, n, seed=2, skew=2.0)
    b = (np.random.default_rng(5).standard_normal(n) * 0.02).astype(np.float32)
    ha, _ = gpu_margin(a, k, nbins, b, solve=False)
    hac, bn = gpu_margin(c, k, nbins, b, hist=ha, accumulate=True)
    H, B = ref.margin_update(np.concatenate([a, c]), nbins, k, b)
    assert np.array_equal(hac, H)
    assert same_bits(bn, B)


def test_margin_empty_batch():
    n, nbins = 8, 100
    b0 = np.arange(n, dtype=np.float32) * 0.01
    h, b = gpu_margin(np.zeros((0, n), np.float32), 2, nbins, b0, hist=np.full((n, nbins), 7))
    assert not h.any() and same_bits(b, b0)


def gpu_signsgd(idx, n, step, bias):
    dev = torch.device("cuda:0")
    b = torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).to(dev)
    lmoe.bias_signsgd(torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(dev), n, step, b)
    torch.cuda.synchronize()
    return b.cpu().numpy()


@pytest.mark.parametrize("T,n,k,step", [(64, 16, 4, 0.01), (32768, 896, 16, 1e-3), (1000, 300, 7, 0.125),
                                        (10, 1024, 64, 0.5), (0, 16, 4, 0.01)])
def test_signsgd_bit_exact(T, n, k, step):
    rng = np.random.default_rng(T + n)
    s = rng.random((T, n)) + (1.0 + np.arange(n))[None, :] ** -1.1
    idx, _ = ref.biased_topk(s, np.zeros(n), k)
    b = (rng.standard_normal(n) * 0.1).astype(np.float32)
    got = gpu_signsgd(idx, n, step, b)
    want = ref.signsgd_update(ref.expert_loads(idx, n), T, k, b, step)
    assert same_bits(got, want)


def test_signsgd_at_the_share_keeps_the_bias():
    # every expert exactly at its share T k / n: no move
    n, k = 8, 2
    idx = np.array([[2 * i % n, (2 * i + 1) % n] for i in range(4 * n)])
    b = np.linspace(-1, 1, n).astype(np.float32)
    assert same_bits(gpu_signsgd(idx, n, 0.25, b), b)
