"""Pins of the oracle's elementwise pieces: bf16 rounding, softcap, SiTU, SiTU-GLU.

Sources: "Kimi K3 Architecture Deep Dive" §1 (softcap and SiTU definitions,
beta1 = 4, beta2 = 25, product bounded by beta1*beta2); "Inside K3" section
SiTU-GLU; LeiPhone report "Keeping the numbers in range" (soft cap preserves
small values).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from oracle import ref


# ---------------------------------------------------------------- bf16 rounding

def _bf16_nearest_exact(x):
    """Brute force: the bf16 value nearest to x (ties to even mantissa), by exact rationals."""
    fx = Fraction(x)
    f32 = np.float32(x)
    # candidates: neighbours in bf16 of the value, from a coarse truncation
    bits = int(np.array([f32], dtype=np.float32).view(np.uint32)[0]) >> 16
    cands = []
    for b in range(bits - 2, bits + 3):
        if 0 <= b < 0x7F80 or 0x8000 <= b < 0xFF80:
            v = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
            cands.append((abs(Fraction(float(v)) - fx), b & 1, float(v)))
    cands.sort()
    best = cands[0]
    ties = [c for c in cands if c[0] == best[0]]
    if len(ties) > 1:
        best = [c for c in ties if c[1] == 0][0]
    return best[2]


def test_round_bf16_matches_exact_nearest():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-20, 20, 300),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 1.0 + 2.0 ** -8 + 2.0 ** -40]])
    got = ref.round_bf16(x)
    for xi, gi in zip(x, got):
        assert gi == _bf16_nearest_exact(float(xi)), xi


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    f = (rng.standard_normal(100000) * 3).astype(np.float32)
    t = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ref.round_bf16(f.astype(np.float64)), t)


def test_round_bf16_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4e38, 1e-40])
    r = ref.round_bf16(x)
    assert r[0] == 0.0 and r[2] == np.inf and r[3] == -np.inf and np.isnan(r[4])
    assert r[5] == np.inf or r[5] == 3.3895313892515355e38
    assert abs(r[6] - 1e-40) <= 2.0 ** -134


def test_round_f32():
    x = np.array([1.0 + 2.0 ** -30, 0.1])
    assert np.array_equal(ref.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- softcap / SiTU

def test_softcap_closed_forms():
    # tanh(ln a) = (a^2 - 1)/(a^2 + 1): ln 2 -> 3/5, ln 3 -> 4/5
    assert ref.softcap(4 * math.log(2), 4.0) == pytest.approx(4 * 3 / 5, rel=1e-15)
    assert ref.softcap(25 * math.log(3), 25.0) == pytest.approx(25 * 4 / 5, rel=1e-15)
    assert ref.softcap(0.0, 4.0) == 0.0


def test_softcap_odd_bounded_and_small_x():
    x = np.linspace(-1e3, 1e3, 200001)
    for beta in (4.0, 25.0):
        s = ref.softcap(x, beta)
        assert np.array_equal(ref.softcap(-x, beta), -s)
        assert np.all(np.abs(s) <= beta)
        xs = x[np.abs(x) <= 2.0]
        err = np.abs(ref.softcap(xs, beta) - xs)
        assert np.all(err <= np.abs(xs) ** 3 / (3 * beta ** 2) + 1e-15)
    # beta -> infinity: identity; beta = +inf is that limit exactly
    assert np.allclose(ref.softcap(x, 1e30), x, rtol=1e-15, atol=0)
    assert np.array_equal(ref.softcap(x, np.inf), x)


def test_sigmoid_closed_forms():
    assert ref.sigmoid(math.log(3)) == pytest.approx(0.75, rel=1e-15)
    assert ref.sigmoid(4 * math.log(2)) == pytest.approx(16 / 17, rel=1e-15)
    assert ref.sigmoid(0.0) == 0.5
    x = np.linspace(-50, 50, 1001)
    assert np.allclose(ref.sigmoid(x), scipy.special.expit(x), rtol=1e-14, atol=0)


def test_situ_closed_form_and_silu_limit():
    # SiTU(4 ln 2; 4) = 4 * 3/5 * 16/17 = 192/85
    assert ref.situ(4 * math.log(2), 4.0) == pytest.approx(192 / 85, rel=1e-14)
    assert ref.situ(0.0, 4.0) == 0.0
    x = np.linspace(-30, 30, 6001)
    silu = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(ref.situ(x, 1e30), silu, rtol=1e-13, atol=1e-300)
    assert np.allclose(ref.situ(x, np.inf), silu, rtol=1e-14, atol=1e-300)


def test_situ_range():
    # bounded by beta; the true range for beta = 4 is about (-0.2698, 4)
    x = np.linspace(-200, 200, 400001)
    v = ref.situ(x, 4.0)
    # open bound in exact arithmetic; tanh and sigmoid saturate to 1 in fp64, so it closes
    assert v.max() <= 4.0 and v.min() > -4.0
    assert ref.situ(10.0, 4.0) < 4.0
    assert -0.2700 < v.min() < -0.2695
    xmin = x[np.argmin(v)]
    assert -1.25 < xmin < -1.19


def test_situ_glu_product_bound_and_swiglu_limit():
    rng = np.random.default_rng(2)
    p1 = rng.standard_normal(100000) * 1e4
    p2 = rng.standard_normal(100000) * 1e4
    a = ref.situ_glu_hidden(p1, p2, 4.0, 25.0)
    assert np.all(np.abs(a) <= 100.0)      # beta1 * beta2 (reached only after saturation)
    assert np.all(np.abs(ref.situ_glu_hidden(p1 / 1e3, p2 / 1e3, 4.0, 25.0)) < 100.0)
    # beta -> infinity gives SwiGLU's hidden SiLU(p1) * p2
    q1 = rng.standard_normal(1000) * 5
    q2 = rng.standard_normal(1000) * 5
    sw = (torch.nn.functional.silu(torch.from_numpy(q1)) * torch.from_numpy(q2)).numpy()
    assert np.allclose(ref.situ_glu_hidden(q1, q2, 1e30, 1e30), sw, rtol=1e-13)
    assert np.allclose(ref.situ_glu_hidden(q1, q2, np.inf, np.inf), sw, rtol=1e-14)
    # without the caps the outlier-scale products above are no longer bounded
    assert np.abs(ref.situ_glu_hidden(p1, p2, np.inf, np.inf)).max() > 1e6


def test_situ_glu_branch_assignment():
    # gate (SiTU, beta1) on W1, linear branch (softcap, beta2) on W2: 192/85 * 20 = 768/17
    a = ref.situ_glu_hidden(4 * math.log(2), 25 * math.log(3), 4.0, 25.0)
    assert a == pytest.approx(768 / 17, rel=1e-14)
    swapped = ref.situ_glu_hidden(25 * math.log(3), 4 * math.log(2), 4.0, 25.0)
    assert abs(swapped - 768 / 17) > 1.0


def test_hard_clip_is_hardtanh_and_its_gate():
    # the hard clip the softcap replaces ([DD] §1) is torch's hardtanh at the same ceiling
    x = np.concatenate([np.linspace(-200, 200, 40001), [4.0, -4.0, 25.0, -25.0, np.inf, -np.inf]])
    for beta in (4.0, 25.0):
        ht = torch.nn.functional.hardtanh(torch.from_numpy(x), -beta, beta).numpy()
        assert np.array_equal(ref.hard_clip(x, beta), ht)
        assert np.array_equal(ref.cap(x, beta, "clip"), ht)
    # clipped SiTU: SiLU inside the ceiling, beta * sigmoid beyond it
    silu = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    inside = np.abs(x) <= 4.0
    assert np.allclose(ref.situ(x[inside], 4.0, "clip"), silu[inside], rtol=1e-14, atol=1e-300)
    out = x[x > 4.0]
    assert np.allclose(ref.situ(out, 4.0, "clip"), 4.0 * scipy.special.expit(out), rtol=1e-14)
    # the gated product keeps the ceiling beta1 * beta2 and reaches it once both saturate
    rng = np.random.default_rng(3)
    p1 = rng.standard_normal(100000) * 1e4
    p2 = rng.standard_normal(100000) * 1e4
    a = ref.situ_glu_hidden(p1, p2, 4.0, 25.0, "clip")
    assert np.all(np.abs(a) <= 100.0) and np.abs(a).max() == 100.0
    # unlike the softcap, the clip maps every value past the ceiling to the same number
    assert ref.hard_clip(30.0, 25.0) == ref.hard_clip(60.0, 25.0) == 25.0
    assert ref.softcap(30.0, 25.0) < ref.softcap(60.0, 25.0) < 25.0
    with pytest.raises(ValueError):
        ref.cap(x, 4.0, "relu")
