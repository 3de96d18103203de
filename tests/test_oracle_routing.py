"""Pins of the router, top-k, routing weights and dispatch of the oracle.

Sources: "Kimi K3 Architecture Deep Dive" §3 (896-choose-16 selection with a
loss-free bias), §2 (route in the latent); LeiPhone report "Keeping the numbers
in range" (bias steers selection).
"""
import itertools

import numpy as np
import pytest

from oracle import ref


def test_topk_brute_force_tiny():
    rng = np.random.default_rng(0)
    n, k, T = 16, 4, 40
    s = rng.random((T, n))
    b = rng.standard_normal(n) * 0.1
    idx, gap = ref.biased_topk(s, b, k)
    sel = s + b
    for t in range(T):
        best = max(itertools.combinations(range(n), k), key=lambda c: sum(sel[t, list(c)]))
        assert set(idx[t]) == set(best)
        # ordered by decreasing biased score
        assert np.all(np.diff(sel[t, idx[t]]) <= 0)
        rest = sorted(set(range(n)) - set(best), key=lambda e: -sel[t, e])
        assert gap[t] == pytest.approx(sel[t, idx[t, -1]] - sel[t, rest[0]])


def test_topk_ties_go_to_lower_index():
    s = np.array([[0.5, 0.7, 0.7, 0.7, 0.1, 0.7]])
    idx, gap = ref.biased_topk(s, np.zeros(6), 2)
    assert idx.tolist() == [[1, 2]]
    assert gap[0] == 0.0
    idx, _ = ref.biased_topk(s, np.array([0, 0, 0, 0, 0, 1e-9]), 2)
    assert idx.tolist() == [[5, 1]]


def test_topk_nan_is_lowest():
    s = np.array([[np.nan, 0.2, np.nan, 0.1]])
    idx, _ = ref.biased_topk(s, np.zeros(4), 3)
    assert idx.tolist() == [[1, 3, 0]]
    s = np.full((1, 4), np.nan)
    idx, _ = ref.biased_topk(s, np.zeros(4), 2)
    assert idx.tolist() == [[0, 1]]


def test_topk_k_equals_n():
    s = np.array([[0.3, 0.9, 0.1]])
    idx, gap = ref.biased_topk(s, np.zeros(3), 3)
    assert idx.tolist() == [[1, 0, 2]] and np.isinf(gap[0])


def test_routing_weights_use_unbiased_scores():
    s = np.array([[0.75, 0.5, 0.25]])
    idx = np.array([[0, 1]])
    g = ref.routing_weights(s, idx)
    assert g.tolist() == [[0.6, 0.4]]
    # a selection bias changes which experts are chosen, never the weights' formula
    idx2, _ = ref.biased_topk(s, np.array([0.0, 0.0, 0.6]), 2)
    assert idx2.tolist() == [[2, 0]]
    assert ref.routing_weights(s, idx2).tolist() == [[0.25, 0.75]]


def test_bias_shift_invariance():
    rng = np.random.default_rng(3)
    s = rng.random((50, 32))
    b = rng.standard_normal(32) * 0.05
    i1, _ = ref.biased_topk(s, b, 5)
    i2, _ = ref.biased_topk(s, b + 0.125, 5)
    assert np.array_equal(i1, i2)


def test_dispatch_brute_force():
    rng = np.random.default_rng(4)
    T, n, k = 37, 11, 3
    idx = np.stack([rng.choice(n, k, replace=False) for _ in range(T)])
    counts, offs, row_token, row_slot = ref.dispatch(idx, n)
    exp_tok, exp_slot = [], []
    for e in range(n):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    exp_tok.append(t)
                    exp_slot.append(j)
    assert row_token.tolist() == exp_tok and row_slot.tolist() == exp_slot
    assert counts.sum() == T * k and offs[0] == 0 and offs[-1] == T * k
    assert np.array_equal(np.diff(offs), counts)
    for e in range(n):
        seg = row_token[offs[e]:offs[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(idx[seg, row_slot[offs[e]:offs[e + 1]]] == e)


def test_logit_offset_enters_before_the_sigmoid():
    """router_scores with a per-expert logit offset o: s = sigmoid(z W_r^T + o).

    With W_r = 0 the scores are exactly sigmoid(o); with logits (ln 3, 0) and
    o = (-ln 3, ln 3) they are (1/2, 3/4).  An offset added after the sigmoid
    would give 3/4 - ln 3 and 1/2 + ln 3 instead, and a dropped offset (3/4, 1/2)."""
    import math
    o = np.array([-2.0, -0.5, 0.0, 0.75, 3.0])
    s = ref.router_scores(np.ones((3, 4)), np.zeros((5, 4)), o)
    want = 1.0 / (1.0 + np.exp(-o))
    assert np.array_equal(s, np.broadcast_to(want, (3, 5)))
    z = np.array([[math.log(3), 0.0]])
    w_r = np.array([[1.0, 0.0], [0.0, 1.0]])
    s = ref.router_scores(z, w_r, np.array([-math.log(3), math.log(3)]))
    assert s == pytest.approx(np.array([[0.5, 0.75]]), rel=1e-15)
    assert ref.router_scores(z, w_r) == pytest.approx(np.array([[0.75, 0.5]]), rel=1e-15)
