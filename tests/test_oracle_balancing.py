"""Pins of the oracle's bias-update baselines and variants next to Quantile
Balancing: the K2-style SignSGD step and the margin reading of QB.

Sources: "Kimi K3 Architecture Deep Dive" §3 (K2's SignSGD-style update,
unstable at 896 experts, replaced by QB with no hyper-parameters); LeiPhone
report "Keeping the numbers in range" (K2 nudged selection by a fixed step; QB
reads the scores against the top-k threshold and solves where each expert's
threshold should move); "Inside K3", section Quantile Balancing.
"""
import numpy as np

from oracle import ref


def test_signsgd_hand_example():
    # T k = 18 over n = 3 experts: target 6 each; expert 0 over, 1 under, 2 at its share
    b = ref.signsgd_update([10, 2, 6], T=9, k=2, bias=[0.0, 0.25, -0.5], step=0.125)
    assert b.dtype == np.float32 and b.tolist() == [-0.125, 0.375, -0.5]
    # the comparison with the share is exact: 7 * 3 = 21 = T k sits at the share
    assert ref.signsgd_update([7, 7, 7], T=7, k=3, bias=[1.0, 2.0, 3.0], step=1.0).tolist() == [1.0, 2.0, 3.0]


def test_signsgd_step_is_fixed_whatever_the_imbalance():
    # the step does not grow with the imbalance (the pages: a fixed step cannot be both fast and stable)
    b1 = ref.signsgd_update([1000, 0], T=500, k=2, bias=[0.0, 0.0], step=0.01)
    b2 = ref.signsgd_update([501, 499], T=500, k=2, bias=[0.0, 0.0], step=0.01)
    assert np.array_equal(b1, b2) and b1[0] == np.float32(-0.01) and b1[1] == np.float32(0.01)


def test_thresholds_hand_example():
    sel = np.array([[0.9, 0.3, 0.7, 0.1], [0.2, 0.2, 0.5, 0.2]], dtype=np.float32)
    tk, tk1 = ref.margin_thresholds(sel, 2)
    assert tk.tolist() == [np.float32(0.7), np.float32(0.2)] and tk1.tolist() == [np.float32(0.3), np.float32(0.2)]
    tk, tk1 = ref.margin_thresholds(sel, 4)
    assert np.all(np.isneginf(tk1))


def _grid_case(seed, T=60, n=12):
    """Scores and bias on a grid of 2^-10, so every fp32 key and margin is exact."""
    rng = np.random.default_rng(seed)
    s = (rng.integers(1, 1024, (T, n)) / 1024.0).astype(np.float32)
    b = (rng.integers(-64, 64, n) / 1024.0).astype(np.float32)
    return s, b


def test_margin_is_the_shift_that_flips_membership():
    """Away from exact ties at the crossing, shifting expert e's bias alone by
    delta keeps it in (or brings it into) token i's top-k exactly when
    m_ie + delta > 0; checked by brute force with the oracle's top-k (ties to the
    lower index) for every expert and shifts of both signs that avoid the grid."""
    for seed, k in ((0, 3), (1, 1), (2, 11)):
        s, b = _grid_case(seed)
        m = ref.margins(s, b, k)
        n = s.shape[1]
        for e in range(n):
            for delta in (-0.3 - 2 ** -11, -3 * 2 ** -11, -2 ** -11, 2 ** -11, 5 * 2 ** -11, 0.2 + 2 ** -11):
                bb = b.astype(np.float64).copy()
                bb[e] += delta
                idx, _ = ref.biased_topk(s.astype(np.float64), bb, k)
                member = (idx == e).any(axis=1)
                assert np.array_equal(member, m[:, e] + delta > 0), (seed, k, e, delta)


def test_margins_of_chosen_experts_are_non_negative():
    s, b = _grid_case(3)
    k = 4
    m = ref.margins(s, b, k)
    idx, gap = ref.biased_topk(s.astype(np.float64), b.astype(np.float64), k)
    chosen = np.zeros_like(m, dtype=bool)
    np.put_along_axis(chosen, idx, True, axis=1)
    assert np.all(m[chosen] >= 0)
    clear = gap > 0
    assert np.all(m[~chosen & clear[:, None]] < 0)


def test_margin_bins_closed_forms():
    m = np.array([[0.0, -1.0, 0.999, 1.5, -0.5, -2.0, np.nan, 0.25]], dtype=np.float32)
    assert ref.margin_bins(m, 1000).tolist() == [[500, 0, 999, 999, 250, 0, 0, 625]]


def test_margin_solve_brackets_each_experts_target_count():
    """After the solve, the tokens of expert e whose margin clears the shift
    (u >= q_e in bin units) number between the tail counts around the crossing
    bin, i.e. its target N k / n within one bin; and moved alone, the expert
    gets that many tokens in its top-k (the membership property above)."""
    rng = np.random.default_rng(9)
    T, n, k, B = 4000, 32, 4, 1000
    s = ref.sigmoid(rng.standard_normal((T, n)) + 1.5 * (1 + np.arange(n)) ** -1.1).astype(np.float32)
    b0 = np.zeros(n, np.float32)
    H, b1 = ref.margin_update(s, B, k, b0)
    m = ref.margins(s, b0, k)
    u = (((m + np.float32(1)).astype(np.float32)) * np.float32(0.5)).astype(np.float32)
    c = T * k / n
    for e in range(n):
        q = (1.0 - float(b1[e] - b0[e])) / 2.0   # b1 - b0 = -(2 q - 1)
        G = np.concatenate([np.cumsum(H[e][::-1])[::-1], [0]])
        j = int(np.nonzero(G[:B] >= c)[0].max())
        cnt = int((u[:, e] >= q - 1e-7).sum())
        assert G[j + 1] <= cnt <= G[j] + 1, e
        bb = b0.astype(np.float64).copy()
        bb[e] = float(b1[e])
        idx, _ = ref.biased_topk(s.astype(np.float64), bb, k)
        got = int((idx == e).sum())
        assert abs(got - c) <= H[e][j] + 1, e


def test_iterated_updates_reduce_skew():
    """On a skewed router (logit offset 2 r^-1.1, as in the skewed workload) ten
    batches of margin-QB, of QB and of SignSGD with a small fixed step: both QB
    forms bring the max/mean load near 1 (250 tokens per expert, so sampling
    noise alone keeps it above 1), the fixed step does not get there."""
    rng = np.random.default_rng(11)
    T, n, k, B = 4000, 64, 4, 1000
    off = 2.0 * (1 + rng.permutation(n)) ** -1.1

    def batch():
        return ref.sigmoid(rng.standard_normal((T, n)) + off[None, :]).astype(np.float32)

    def skew(s, b):
        idx, _ = ref.biased_topk(s.astype(np.float64), b.astype(np.float64), k)
        load = ref.expert_loads(idx, n)
        return load.max() / load.mean(), load

    start, _ = skew(batch(), np.zeros(n, np.float32))
    bm = np.zeros(n, np.float32)
    bq = np.zeros(n, np.float32)
    bs = np.zeros(n, np.float32)
    for _ in range(10):
        s = batch()
        _, bm = ref.margin_update(s, B, k, bm)
        _, bq = ref.qb_update(s, B, k, bias=bq)
        _, load = skew(s, bs)
        bs = ref.signsgd_update(load, T, k, bs, 1e-3)
    s = batch()
    end_m, _ = skew(s, bm)
    end_q, _ = skew(s, bq)
    end_s, _ = skew(s, bs)
    assert start > 2.5
    assert end_m < 1.4 and end_q < 1.6
    assert end_s > 2.0
