"""The seeded input generator: published SplitMix64 outputs, host C filler vs a
NumPy restatement of the same definition, distribution moments, bf16 rounding."""
import numpy as np
import pytest
import torch

import synth


def test_splitmix64_published_outputs():
    # SplitMix64 started from state 0 (Steele, Lea & Flood 2014; Vigna's reference code)
    assert synth.splitmix_output(0, 0) == 0xE220A8397B1DCDAF
    assert synth.splitmix_output(0, 1) == 0x6E789E6AA1B965F4
    assert synth.splitmix_output(0, 2) == 0x06C45D188009454F


@pytest.mark.parametrize("seed,tid,start", [(0, 0, 0), (2, 3, 123456789), (7, 100, 5)])
def test_host_filler_matches_numpy_definition(seed, tid, start):
    a = synth.host_fill(4096, seed, tid, start, 0.37)
    b = synth.numpy_fill_f32(4096, seed, tid, start, 0.37)
    assert a.dtype == np.float32
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_random_access_is_consistent():
    whole = synth.host_fill(10000, 3, 4, 0, 1.0)
    part = synth.host_fill(1000, 3, 4, 5000, 1.0)
    assert np.array_equal(whole[5000:6000], part)


def test_moments_are_normal_like():
    v = synth.host_fill(4_000_000, 11, 2, 0, 0.5).astype(np.float64)
    assert abs(v.mean()) < 2e-3
    assert abs(v.std() - 0.5) < 2e-3
    kurt = np.mean((v / v.std()) ** 4)
    assert 2.7 < kurt < 3.0          # Irwin-Hall(12): 3 - 0.1 = 2.9


def test_bf16_filler_is_rne_of_f32_filler():
    f = synth.host_fill(100000, 1, 9, 0, 0.05)
    b = synth.host_fill(100000, 1, 9, 0, 0.05, bf16=True)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_row_multiplier_applies_after_scale():
    rm = np.array([1.0, 50.0, 1.0], dtype=np.float32)
    f = synth.host_fill(3 * 16, 2, 0, 0, 1.0, row_mult=rm, row_len=16)
    base = synth.host_fill(3 * 16, 2, 0, 0, 1.0)
    assert np.array_equal(f[:16], base[:16]) and np.array_equal(f[32:], base[32:])
    assert np.array_equal(f[16:32], base[16:32] * np.float32(50.0))
    # a single row generated alone gets the same values
    one = synth.host_fill(16, 2, 0, 16, 1.0, row_mult=rm[1:2], row_len=16)
    assert np.array_equal(one, f[16:32])


def test_configs_shapes():
    c2 = synth.get_config("C2")
    assert (c2.d, c2.L, c2.n, c2.k, c2.n_shared) == (7168, 3584, 896, 16, 2)
    assert c2.L * 2 == c2.d
    assert abs(c2.flops_per_token() - 307.36e6) < 0.01e6
    assert synth.outlier_rows(c2).size == 8
    o = synth.zipf_logit_offset(synth.get_config("C4"))
    assert o.shape == (896,) and abs(o.max() - 2.0) < 1e-6
