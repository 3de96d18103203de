"""Pins of the oracle's Quantile Balancing estimator.

Sources: "Kimi K3 Architecture Deep Dive" §3 (scores mapped into [0,1], a
B-bin histogram, histograms summed across devices, the quantile read from the
sum; 1000 bins); "Inside K3" section Quantile Balancing; LeiPhone report
"Keeping the numbers in range" (read the score distribution against the top-k
threshold to give each expert its target share).
"""
import numpy as np
import pytest

from oracle import ref


def test_bins_rule():
    s = np.array([[0.0, 0.0005, 0.001, 0.9995, 0.999, 1.0, 1.5, -0.1, np.nan]], dtype=np.float32)
    b = ref.qb_bins(s, 1000)
    assert b.tolist() == [[0, 0, 1, 999, 999, 999, 999, 0, 0]]


def test_histogram_matches_numpy_histogram_away_from_edges():
    rng = np.random.default_rng(0)
    s = rng.random((3000, 7)).astype(np.float32)
    H = ref.qb_histogram(s, 1000)
    sb = s.astype(np.float64) * 1000
    near = np.abs(sb - np.round(sb)) < 1e-3
    for e in range(7):
        keep = ~near[:, e]
        h_np, _ = np.histogram(s[keep, e].astype(np.float64), bins=1000, range=(0.0, 1.0))
        h_me = np.bincount(ref.qb_bins(s[keep, e:e + 1], 1000)[:, 0], minlength=1000)
        assert np.array_equal(h_np, h_me)
    assert H.sum() == 3000 * 7 and np.all(H.sum(1) == 3000)


def test_histograms_are_additive():
    rng = np.random.default_rng(1)
    a = rng.random((500, 5)).astype(np.float32)
    b = rng.random((700, 5)).astype(np.float32)
    assert np.array_equal(ref.qb_histogram(a, 1000) + ref.qb_histogram(b, 1000),
                          ref.qb_histogram(np.concatenate([a, b]), 1000))
    H, _ = ref.qb_update(b, 1000, 2, hist=ref.qb_histogram(a, 1000), accumulate=True, solve=False)
    assert np.array_equal(H, ref.qb_histogram(np.concatenate([a, b]), 1000))


def test_read_hand_example():
    # B = 10, half the mass in bin 8 and half in bin 9 (counts 5, 5)
    h = np.zeros(10, dtype=np.int64)
    h[8] = 5
    h[9] = 5
    assert ref.qb_read(h, 3) == pytest.approx(0.94, abs=1e-15)   # inside bin 9: 10 - 3/5
    assert ref.qb_read(h, 5) == pytest.approx(0.90, abs=1e-15)   # exactly the bin-9 mass
    assert ref.qb_read(h, 7) == pytest.approx(0.86, abs=1e-15)   # 9 - 2/5
    assert ref.qb_read(h, 10) == pytest.approx(0.80, abs=1e-15)  # all mass


def test_read_within_one_bin_of_exact_sort():
    rng = np.random.default_rng(2)
    for dist in ("uniform", "beta", "sigmoid"):
        if dist == "uniform":
            s = rng.random(20000)
        elif dist == "beta":
            s = rng.beta(2, 9, 20000)
        else:
            s = 1 / (1 + np.exp(-rng.standard_normal(20000) * 2))
        s = s.astype(np.float32)
        h = ref.qb_histogram(s[:, None], 1000)[0]
        for c in (1.0, 146.29, 585.14, 5000.0, 20000.0):
            q = ref.qb_read(h, c)
            exact = np.sort(s.astype(np.float64))[::-1][int(np.ceil(c)) - 1]
            assert abs(q - exact) <= 1.0 / 1000 + 1e-12


def test_uniform_scores_give_complement_share():
    rng = np.random.default_rng(3)
    n, k, T = 64, 4, 50000
    s = rng.random((T, n)).astype(np.float32)
    H = ref.qb_histogram(s, 1000)
    for e in range(4):
        assert abs(ref.qb_read(H[e], T * k / n) - (1 - k / n)) < 0.01


def test_solved_bias_gives_target_share_per_expert():
    rng = np.random.default_rng(4)
    n, k, T, B = 32, 4, 20000, 1000
    logits = rng.standard_normal((T, n)) + np.linspace(2, -2, n)[None, :]
    s = (1 / (1 + np.exp(-logits))).astype(np.float32)
    H = ref.qb_histogram(s, B)
    b = ref.qb_solve(H, k, n, np.zeros(n, np.float32))
    pooled = H.sum(0)
    tau = ref.qb_read(pooled, T * n * k / n)
    for e in range(n):
        q = tau - float(b[e])
        # the count of scores at or above the expert's threshold brackets the target count
        jstar = min(int(q * B), B - 1)
        cnt = np.sum(s[:, e].astype(np.float64) >= q)
        assert abs(cnt - T * k / n) <= H[e, jstar] + 1
    # every expert's threshold moved to the common level: s + b >= tau at share k/n
    loads = np.sum(s.astype(np.float64) + b.astype(np.float64)[None, :] >= tau, axis=0)
    assert loads.max() / loads.mean() < 1.15


def test_qb_reduces_top_k_load_skew():
    rng = np.random.default_rng(5)
    n, k, T = 128, 8, 8000
    skew = 2.0 * (1 + rng.permutation(n)) ** -1.1
    logits = rng.standard_normal((T, n)) * 0.5 + skew[None, :]
    s = 1 / (1 + np.exp(-logits))
    idx0, _ = ref.biased_topk(s, np.zeros(n), k)
    H, b = ref.qb_update(s.astype(np.float32), 1000, k)
    idx1, _ = ref.biased_topk(s, b.astype(np.float64), k)
    l0 = ref.expert_loads(idx0, n)
    l1 = ref.expert_loads(idx1, n)
    assert l0.max() / l0.mean() > 5
    assert l1.max() / l1.mean() < 2


def test_empty_histogram_leaves_bias():
    b0 = np.arange(4, dtype=np.float32)
    assert np.array_equal(ref.qb_solve(np.zeros((4, 10), np.int64), 1, 4, b0), b0)
