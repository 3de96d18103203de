"""GPU parity of lmoe_qb_update against the oracle (bit-exact histograms and bias
on identical fp32 scores), including accumulation across batches (the
single-device form of the cross-device histogram sum) and the edge cases."""
import numpy as np
import pytest
import torch

import sparse_moe_layer_down_amd as lmoe
import synth
from oracle import ref

pytestmark = pytest.mark.gpu


def host_scores(T, n, seed, skew=0.0):
    """Synthetic fp32 router-like scores: logistic of generated normals plus an expert skew."""
    z = synth.host_fill(T * n, seed, synth.TID["scores"], 0, 1.5).astype(np.float64).reshape(T, n)
    if skew:
        z = z + skew * (1.0 + np.arange(n))[None, :] ** -1.1
    return ref.sigmoid(z).astype(np.float32)


def gpu_qb(s, k, nbins, hist=None, bias=None, accumulate=False, solve=True):
    dev = torch.device("cuda:0")
    n = s.shape[1]
    st = torch.from_numpy(s).to(dev)
    h = torch.empty((n, nbins), dtype=torch.int32, device=dev) if hist is None else \
        torch.from_numpy(np.ascontiguousarray(hist, dtype=np.int32)).to(dev)
    b = torch.zeros(n, dtype=torch.float32, device=dev) if bias is None else torch.from_numpy(bias.copy()).to(dev)
    lmoe.qb_update(st, k, h, b if solve else None, accumulate=accumulate, solve=solve)
    torch.cuda.synchronize()
    return h.cpu().numpy().astype(np.int64), b.cpu().numpy()


def same_bits(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("T,n,k,nbins", [(64, 16, 4, 1000), (4096, 128, 8, 1000), (777, 100, 3, 37),
                                         (300, 896, 16, 10000), (5, 3, 1, 1),
                                         # wide histograms: tau read once, bins staged in LDS; n not a
                                         # multiple of 4 (per-expert loads), the widest histogram
                                         (513, 6, 2, 4099), (700, 40, 5, 16384), (2000, 12, 3, 8192),
                                         # group geometry edges: 4 experts in exactly 160 KB of LDS, one bin
                                         # more (one expert per group), 32-expert groups with n % 4 != 0
                                         (3000, 12, 3, 10240), (3000, 12, 3, 10241), (5000, 70, 7, 1000)])
def test_hist_and_bias_bit_exact(T, n, k, nbins):
    s = host_scores(T, n, seed=T + n, skew=1.0)
    s[0, 0] = 1.0
    s[min(1, T - 1), min(1, n - 1)] = 0.0
    h, b = gpu_qb(s, k, nbins)
    H, B = ref.qb_update(s, nbins, k)
    assert np.array_equal(h, H)
    assert same_bits(b, B)


@pytest.mark.parametrize("T", [16 * 65535, 1_100_000])
def test_run_counts_at_the_16_bit_limit(T):
    """Every score equal, so each token run's counts all land in one bin: with 16
    runs of 65535 tokens that bin holds 65535 in every run (the most a 16-bit slab
    takes); with 68750 tokens per run the runs' slabs are 32-bit."""
    n, k, nbins = 8, 2, 1000
    s = np.full((T, n), 0.5, dtype=np.float32)
    s[::3, 1] = 0.25
    h, b = gpu_qb(s, k, nbins)
    H, B = ref.qb_update(s, nbins, k)
    assert np.array_equal(h, H)
    assert same_bits(b, B)
    assert h[0, 500] == T


def test_special_scores_bins():
    s = np.array([[0.0, 0.0005, 0.001, 0.9995, 0.999, 1.0, 1.5, -0.1, np.nan] * 2], dtype=np.float32).reshape(2, 9)
    h, _ = gpu_qb(s, 1, 1000, solve=False)
    assert np.array_equal(h, ref.qb_histogram(s, 1000))


def test_accumulate_is_the_cross_batch_sum():
    n, k, nbins = 896, 16, 1000
    a = host_scores(3000, n, seed=1, skew=2.0)
    bb = host_scores(5000, n, seed=2, skew=2.0)
    ha, _ = gpu_qb(a, k, nbins, solve=False)
    hab, bias = gpu_qb(bb, k, nbins, hist=ha, accumulate=True, solve=True)
    H, B = ref.qb_update(np.concatenate([a, bb]), nbins, k)
    assert np.array_equal(hab, H)
    assert same_bits(bias, B)
    # a batch of at most 256 tokens is one run, added in place rather than through the slabs
    c = host_scores(200, n, seed=3, skew=2.0)
    habc, bias = gpu_qb(c, k, nbins, hist=hab, accumulate=True, solve=True)
    H, B = ref.qb_update(np.concatenate([a, bb, c]), nbins, k)
    assert np.array_equal(habc, H)
    assert same_bits(bias, B)


def test_c4_shaped_batch():
    cfg = synth.get_config("C4")
    s = host_scores(cfg.T, cfg.n, seed=44, skew=2.0)
    h, b = gpu_qb(s, cfg.k, cfg.nbins)
    H, B = ref.qb_update(s, cfg.nbins, cfg.k)
    assert np.array_equal(h, H)
    assert same_bits(b, B)
    assert h.sum() == cfg.T * cfg.n


def test_empty_batch_and_empty_histogram():
    n, nbins = 8, 100
    s = np.zeros((0, n), dtype=np.float32)
    b0 = np.arange(n, dtype=np.float32)
    h, b = gpu_qb(s, 2, nbins, hist=np.full((n, nbins), 7), bias=b0, accumulate=False, solve=True)
    assert not h.any()
    assert same_bits(b, b0)
    # accumulate with no tokens leaves the histogram as it was and solves from it
    h0 = np.zeros((n, nbins), np.int64)
    h0[:, 50] = 3
    h, b = gpu_qb(s, 2, nbins, hist=h0, bias=b0, accumulate=True, solve=True)
    assert np.array_equal(h, h0)
    assert same_bits(b, ref.qb_solve(h0, 2, n, b0))
