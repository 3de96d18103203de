"""The C-ABI library loads, exports every declared entry point, sizes its
workspace and rejects invalid arguments before launching anything (no GPU
needed: every call here fails validation or is a no-op)."""
import ctypes
import math
import os
import re

import pytest

import sparse_moe_layer_down_amd as lmoe
from sparse_moe_layer_down_amd._abi import Dims, Weights, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_declarations_are_exported():
    hdr = open(os.path.join(ROOT, "include", "lmoe.h")).read()
    declared = set(re.findall(r"^\S[^\n(]*?\b(lmoe_\w+)\(", hdr, flags=re.M))
    assert declared == set(lmoe.EXPORTS)
    L = lib()
    for name in declared:
        assert hasattr(L, name)


def c2dims(**kw):
    d = dict(T=8192, d=7168, L=3584, n=896, k=16, n_shared=2, D=512)
    d.update(kw)
    return Dims(*[d[f] for f in ("T", "d", "L", "n", "k", "n_shared", "D")])


def test_workspace_size():
    ws = lmoe.workspace_size(c2dims(), lmoe.LMOE_BF16)
    # dominated by the staged expert rows, sized for fp32 (the uncapped ablation stages in
    # fp32; fp16 otherwise for bf16 inputs): T*(k+n_shared)*L*4 = 2.11 GB
    assert 8192 * 18 * 3584 * 4 < ws < 2.6e9
    # fp32 inputs stage them in fp32
    assert lmoe.workspace_size(c2dims(), lmoe.LMOE_F32) > 8192 * 16 * 3584 * 4
    assert lmoe.workspace_size(c2dims(L=1000), lmoe.LMOE_BF16) == 0
    assert lmoe.workspace_size(c2dims(), 7) == 0
    # regions are 256-byte aligned and inside the workspace
    for r in range(8):
        off = lib().lmoe_workspace_offset(c2dims(), 1, r)
        assert off >= 0 and off % 256 == 0 and off < ws
    assert lib().lmoe_workspace_offset(c2dims(), 1, 99) == -1


@pytest.mark.parametrize("kw", [dict(n_shared=0), dict(T=1), dict(T=0), dict(T=1, n_shared=0, n=1, k=1),
                                dict(T=64, d=256, L=128, n=16, k=4, n_shared=1, D=64), dict(T=100000)])
def test_workspace_size_edge_dims(kw):
    # host-side sizing (split-K planning included) must handle every valid shape
    for dt in (0, 1):
        ws = lmoe.workspace_size(c2dims(**kw), dt)
        assert ws > 0
        for r in range(8):
            assert 0 <= lib().lmoe_workspace_offset(c2dims(**kw), dt, r) < ws


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def fake_weights(n_shared=2, **over):
    vals = dict(w_down=FAKE, w_router=FAKE, router_bias=FAKE, router_logit_offset=None, w1=FAKE, w2=FAKE,
                w3=FAKE, ws1=FAKE if n_shared else None, ws2=FAKE if n_shared else None,
                ws3=FAKE if n_shared else None, rms_gain=FAKE, w_up=FAKE, beta1=4.0, beta2=25.0, rms_eps=1e-6,
                gate=0, norm=0)
    vals.update(over)
    return Weights(*[vals[f] for f, _ in Weights._fields_])


def call(dims, w, dtype=1, x=FAKE, y=FAKE, ws=FAKE, wsb=1 << 40):
    return lib().lmoe_forward(ctypes.byref(dims), ctypes.byref(w), dtype, x, y, None, None, None, ws, wsb, None)


@pytest.mark.parametrize("dims,code", [
    (c2dims(L=3000), -2), (c2dims(k=0), -2), (c2dims(k=897), -2), (c2dims(n=2000), -2),
    (c2dims(d=7000, L=3500), -2), (c2dims(D=500), -2), (c2dims(T=-1), -2), (c2dims(k=65, n=896), -2),
])
def test_shape_errors(dims, code):
    assert call(dims, fake_weights()) == code


def test_operand_span_limit():
    """The load-to-LDS GEMMs address each operand through 32-bit byte offsets, so
    dims whose operands would span 4 GiB or more are rejected up front: at
    T = 150000 and d = 7168, x is 4.3 GB in fp32 (rejected) and 2.15 GB in bf16
    (accepted); the backward's gathered-row transposes [L, ~T(k + n_s)] reach
    5.05 GB at T = 32768 in bf16 (rejected) and 1.88 GB at T = 8192."""
    big = c2dims(T=150000)
    assert lmoe.workspace_size(big, 0) == 0
    assert call(big, fake_weights(), dtype=0) == -2
    assert lib().lmoe_forward_static(ctypes.byref(big), ctypes.byref(fake_weights()), 0, FAKE, FAKE, None, None,
                                     None, None) == -2
    assert lmoe.workspace_size(big, 1) > 0
    bws = lib().lmoe_backward_workspace_size
    assert bws(ctypes.byref(c2dims(T=32768)), 1) == 0
    assert bws(ctypes.byref(c2dims(T=8192)), 1) > 0
    assert bws(ctypes.byref(c2dims(T=16384)), 1) > 0


def test_other_errors():
    d = c2dims()
    assert call(d, fake_weights(), dtype=5) == -3
    assert call(d, fake_weights(w1=None)) == -1
    assert call(d, fake_weights(), x=None) == -1
    assert call(d, fake_weights(ws3=None)) == -1
    assert call(c2dims(n_shared=0), fake_weights(n_shared=2)) == -2
    assert call(d, fake_weights(w3=FAKE + 8)) == -4
    assert call(d, fake_weights(), wsb=1000) == -5
    assert call(d, fake_weights(beta1=0.0)) == -7
    assert call(d, fake_weights(beta2=-math.inf)) == -7
    assert call(d, fake_weights(beta1=math.nan)) == -7
    assert call(d, fake_weights(gate=2)) == -7
    assert call(d, fake_weights(gate=-1)) == -7
    assert call(d, fake_weights(norm=3)) == -7
    assert call(d, fake_weights(rms_eps=-1.0)) == -7
    assert lib().lmoe_forward(None, ctypes.byref(fake_weights()), 1, FAKE, FAKE, None, None, None, FAKE, 1, None) == -1


def test_timed_forward_validation():
    """lmoe_forward_timed: the event array itself is required and must hold
    LMOE_N_STAGES + 1 entries; NULL entries are allowed (that boundary is not
    recorded), so an all-NULL array reaches the forward's own validation."""
    t = lib().lmoe_forward_timed
    d, w = c2dims(), fake_weights()
    arr = (ctypes.c_void_p * 9)()
    args = (ctypes.byref(d), ctypes.byref(w), 1, FAKE, FAKE, None, None, None)
    assert t(*args, FAKE, 1 << 40, None, 9, None) == -1            # no event array
    assert t(*args, FAKE, 1 << 40, arr, 8, None) == -7             # wrong count
    assert t(*args, FAKE, 1000, arr, 9, None) == -5                # NULL entries pass; workspace too small
    assert t(ctypes.byref(c2dims(T=0)), ctypes.byref(w), 1, None, None, None, None, None, None, 0, arr, 9,
             None) == 0                                           # empty batch, nothing recorded


def test_empty_batch_is_a_noop():
    assert call(c2dims(T=0), fake_weights(), x=None, y=None, ws=None, wsb=0) == 0


def test_qb_validation():
    q = lib().lmoe_qb_update
    assert q(FAKE, 10, 896, 0, 1000, FAKE, 0, FAKE, 1, FAKE, 1 << 20, None) == -2   # k = 0
    assert q(FAKE, 10, 896, 16, 0, FAKE, 0, FAKE, 1, FAKE, 1 << 20, None) == -7     # no bins
    assert q(FAKE, 10, (1 << 20) + 1, 16, 1000, FAKE, 0, FAKE, 1, FAKE, 1 << 30, None) == -2  # too many experts
    assert q(FAKE, 10, 896, 16, 1000, None, 0, FAKE, 1, FAKE, 1 << 20, None) == -1  # no histogram
    assert q(FAKE, 10, 896, 16, 1000, FAKE, 0, None, 1, FAKE, 1 << 20, None) == -1  # solve without bias
    assert q(FAKE, 10, 896, 16, 1000, FAKE + 4, 0, FAKE, 1, FAKE, 1 << 20, None) == -4
    assert q(FAKE, 10, 896, 16, 1000, FAKE, 0, FAKE, 1, FAKE, 16, None) == -5
    # the pooled histogram (int64 per bin), then one int32 [n, nbins] count slab per token run:
    # 16-expert groups of 64 KB of LDS, two resident per CU: runs = min(16, 512 // groups)
    # (56 groups at n = 896: 9 runs)
    assert lmoe.qb_workspace_size(896, 1000) == 15360 + 9 * 896 * 1000 * 4  # (1000 + 2 + 896) x 8 B, rounded to 256
    assert lmoe.qb_workspace_size(8, 1000) == 8192 + 16 * 8 * 1000 * 4
    # one expert per group at 10000 bins (40 KB, four per CU): 896 groups fill 1024 slots in one run
    assert lmoe.qb_workspace_size(896, 10000) == 87296  # (10000 + 2 + 896) x 8 B, rounded to 256
    assert lmoe.qb_workspace_size(200, 10000) == 81664 + 5 * 200 * 10000 * 4
    assert lmoe.qb_workspace_size(896, 0) == 0 and lmoe.qb_workspace_size(0, 1000) == 0


def test_strerror():
    assert lmoe.strerror(-5).startswith("workspace")
    assert lmoe.strerror(123) == "unknown status"


def test_static_forward_validation():
    """lmoe_forward_static checks its scratch bound on the host before anything
    else touches the GPU: the prefill shape needs more than the static scratch."""
    f = lib().lmoe_forward_static
    w = fake_weights()

    def call_s(d, **kw):
        return f(ctypes.byref(d), ctypes.byref(w), kw.get("dtype", 1), FAKE, FAKE, None, None, None, None)

    assert lmoe.workspace_size(c2dims(), 1) > lmoe.STATIC_SCRATCH_BYTES
    assert call_s(c2dims()) == -8
    assert call_s(c2dims(L=3000)) == -2
    assert call_s(c2dims(), dtype=9) == -3
    assert f(ctypes.byref(c2dims(T=0)), ctypes.byref(w), 1, None, None, None, None, None, None) == 0
    assert lmoe.strerror(-8).startswith("the call needs more scratch")


def test_balancing_entry_points_validation():
    """lmoe_qb_margin_update and lmoe_bias_signsgd validate before launching."""
    q = lib().lmoe_qb_margin_update
    assert q(FAKE, 10, 1025, 16, 1000, FAKE, 0, FAKE, 1, FAKE, 1 << 20, None) == -2   # n beyond the top-k kernels
    assert q(FAKE, 10, 896, 897, 1000, FAKE, 0, FAKE, 1, FAKE, 1 << 20, None) == -2   # k > n
    assert q(FAKE, 10, 896, 16, 0, FAKE, 0, FAKE, 1, FAKE, 1 << 20, None) == -7       # no bins
    assert q(FAKE, 10, 896, 16, 1000, FAKE, 0, None, 1, FAKE, 1 << 20, None) == -1    # bias is an input too
    assert q(FAKE, 10, 896, 16, 1000, FAKE, 0, FAKE, 1, None, 0, None) == -1          # thresholds need a workspace
    assert q(FAKE, 10, 896, 16, 1000, FAKE, 0, FAKE, 1, FAKE, 16, None) == -5
    assert q(FAKE, 10, 896, 16, 1000, FAKE + 4, 0, FAKE, 1, FAKE, 1 << 20, None) == -4
    assert lmoe.qb_margin_workspace_size(32768, 896, 1000) == 32768 * 8 + 9 * 896 * 1000 * 4
    assert lmoe.qb_margin_workspace_size(-1, 896, 1000) == 0 and lmoe.qb_margin_workspace_size(8, 1025, 1000) == 0
    g = lib().lmoe_bias_signsgd
    assert g(FAKE, 10, 896, 16, float("inf"), FAKE, None) == -7
    assert g(FAKE, 10, 896, 16, float("nan"), FAKE, None) == -7
    assert g(FAKE, 10, 896, 0, 0.01, FAKE, None) == -2
    assert g(FAKE, 10, 896, 16, 0.01, None, None) == -1
    assert g(None, 10, 896, 16, 0.01, FAKE, None) == -1
    assert g(FAKE, 10, 896, 16, 0.01, FAKE + 4, None) == -4
    assert g(None, 0, 896, 16, 0.01, FAKE, None) == 0                                 # empty batch: no-op


def test_backward_validation():
    """lmoe_backward validates on the host before launching anything."""
    from sparse_moe_layer_down_amd._abi import Grads
    b = lib().lmoe_backward
    w = fake_weights()
    full = Grads(*([FAKE] * 11))

    def call_b(d, grads=full, ws=FAKE, wsb=1 << 40, fwsb=1 << 40, ww=w):
        return b(ctypes.byref(d), ctypes.byref(ww), 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, fwsb, ctypes.byref(grads),
                 ws, wsb, None)

    assert lmoe.backward_workspace_size(c2dims(), 1) > lmoe.workspace_size(c2dims(), 1)
    assert lmoe.backward_workspace_size(c2dims(d=16384, L=8192), 1) == 0      # latent above 4096
    assert call_b(c2dims(d=16384, L=8192)) == -2
    assert call_b(c2dims(), ww=fake_weights(norm=2)) == -7                  # no backward of the extra norm
    assert call_b(c2dims(), grads=Grads(*([FAKE] * 10 + [None]))) == -1      # dw_up missing
    assert call_b(c2dims(n_shared=0), ww=fake_weights(n_shared=0)) == -2     # shared gradients without shared experts
    assert call_b(c2dims(), fwsb=1000) == -5
    assert call_b(c2dims(), wsb=1000) == -5
    assert call_b(c2dims(), ws=None) == -1
