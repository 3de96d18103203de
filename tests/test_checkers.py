"""CPU tests of the parity checkers the GPU tests use: each must accept what
the oracle produces and reject a planted mistake."""
import numpy as np

from oracle import ref
from test_gpu_forward import check_topk_valid


def _case():
    rng = np.random.default_rng(5)
    s = rng.random((50, 40)).astype(np.float32)
    s[:, 7] = s[:, 3]    # exact ties between experts 3 and 7
    s[:, 30] = s[:, 12]  # and between 12 and 30
    b = (np.arange(40) % 4 * 0.125).astype(np.float32)
    sel = (s + b).astype(np.float64)  # the fp32 keys, exactly
    idx, _ = ref.biased_topk(sel, np.zeros(40), 6)
    return s, b, idx


def test_topk_checker_accepts_the_oracle_selection():
    s, b, idx = _case()
    assert check_topk_valid(s, b, idx) >= 0


def test_topk_checker_rejects_planted_mistakes():
    import pytest
    s, b, idx = _case()
    sel = s + b
    t = 0
    unchosen = np.setdiff1d(np.arange(40), idx[t])
    # a lower key than one left out
    bad = idx.copy()
    bad[t, -1] = unchosen[np.argmin(sel[t, unchosen])]
    with pytest.raises(AssertionError):
        check_topk_valid(s, b, bad)
    # a repeated expert
    bad = idx.copy()
    bad[t, 1] = bad[t, 0]
    with pytest.raises(AssertionError):
        check_topk_valid(s, b, bad)
    # wrong order inside the list
    bad = idx.copy()
    bad[t, [0, 1]] = bad[t, [1, 0]]
    with pytest.raises(AssertionError):
        check_topk_valid(s, b, bad)
    # a tie at the threshold broken towards the higher index
    s2 = np.full((1, 10), 0.5, dtype=np.float32)
    z = np.zeros(10, dtype=np.float32)
    assert check_topk_valid(s2, z, np.array([[0, 1, 2]])) == 1
    with pytest.raises(AssertionError):
        check_topk_valid(s2, z, np.array([[0, 1, 3]]))
