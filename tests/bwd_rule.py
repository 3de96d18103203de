"""Matching rule for the layer's gradients (shared by the GPU parity tests and
the CPU test that pins its bounds to the oracle's own rounding floor).

fp32: every gradient within max|err| <= 1e-5 * sqrt(K / 1024) * RMS(ref), as
the forward's fp32 outputs.

bf16: the gradients pass through up to five chained bf16 stores (du and g du,
da, dp1 and dp2, dl, dz).  Where two correct implementations (here fp32
accumulation and fp16 staged expert rows against the fp64 oracle) round a
stored element to different neighbours, that element moves by one bf16 ulp
(2^-8 of itself) and the move propagates, so the largest single deviation
scales with the heaviest element, not with the bulk.  The rule therefore
bounds the bulk everywhere and the maximum only where it is well conditioned:

  dense gradients (dx, dW_down, dW_up, the gain, the shared experts' banks,
  whose rows come from every token):
      RMS(err) <= 1e-2 RMS(ref) and max|err| <= 1e-1 RMS(ref);
  routed expert banks (dW1, dW2, dW3: one matrix per expert, from its own
  rows only, so an expert with one token has a rank-one gradient):
      RMS(err) <= 1e-2 RMS(ref) over the bank, each expert with rows
      RMS(err_e) <= 5e-2 RMS(ref_e), each expert without rows exactly zero;
  the router weight dW_r (row e sums the logit gradients of the tokens that
      chose e; each is a difference of nearly equal routing-weight gradients):
      RMS(err) <= 1e-2 RMS(ref), rows of experts no token chose exactly zero.

A gradient whose reference is identically zero (one expert with k = 1: the
routing weight is always 1) must come back exactly zero.  A wrong term,
operand or index moves a whole gradient by O(1) of its RMS; a wrong expert
(or a lost tile of one) moves that expert by O(1) of its own RMS.
"""
import numpy as np

BF16_RMS = 1e-2
BF16_MAX = 1e-1
BF16_EXPERT_RMS = 5e-2

ROUTED = ("dw1", "dw2", "dw3")
ROUTER = ("dw_router",)


def fp32_tol(K):
    return 1e-5 * max(1.0, np.sqrt(K / 1024.0))


def _rms(a):
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def measures(got, want, kind, counts=None):
    """Dict of the rule's measures for one gradient (relative errors; a zero
    reference contributes 0 when matched exactly and inf otherwise)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = got - want
    r = _rms(want)
    m = {}
    if r == 0.0:
        bad = float(np.inf) if d.any() else 0.0
        m["rms"] = m["max"] = bad
    else:
        m["rms"] = _rms(d) / r
        m["max"] = float(np.abs(d).max()) / r
    if kind in ("routed", "router") and counts is not None:
        live = np.asarray(counts) > 0
        dead = got.reshape(got.shape[0], -1)[~live]
        m["dead"] = float(np.abs(dead).max()) if dead.size else 0.0
        if kind == "routed":
            de = d.reshape(d.shape[0], -1)[live]
            we = want.reshape(want.shape[0], -1)[live]
            ratio = [(_rms(a) / _rms(b)) if _rms(b) > 0 else (np.inf if a.any() else 0.0) for a, b in zip(de, we)]
            m["expert_rms"] = float(max(ratio, default=0.0))
    return m


def kind_of(name):
    return "routed" if name in ROUTED else ("router" if name in ROUTER else "dense")


def failures(dtype, K, name, got, want, counts=None, scale=1.0):
    """Rule violations of one gradient as text (empty: it matches).  `scale`
    multiplies every bound (the CPU pin checks the floor against a fraction)."""
    kind = kind_of(name)
    m = measures(got, want, kind, counts)
    out = []
    if dtype == "f32":
        if m["max"] > scale * fp32_tol(K):
            out.append(f"max {m['max']:.3e} > {scale * fp32_tol(K):.1e}")
    else:
        if m["rms"] > scale * BF16_RMS:
            out.append(f"rms {m['rms']:.3e} > {scale * BF16_RMS:.1e}")
        if kind == "dense" and m["max"] > scale * BF16_MAX:
            out.append(f"max {m['max']:.3e} > {scale * BF16_MAX:.1e}")
        if m.get("expert_rms", 0.0) > scale * BF16_EXPERT_RMS:
            out.append(f"expert rms {m['expert_rms']:.3e} > {scale * BF16_EXPERT_RMS:.1e}")
    if m.get("dead", 0.0) != 0.0:
        out.append(f"unrouted experts not zero ({m['dead']:.3e})")
    return m, out


def describe(m):
    return "  ".join(f"{k} {v:.2e}" for k, v in m.items())
