"""The oracle and the K3-shaped workloads against the values the pages print
(tests/golden/k3_printed_values.json, each value with its page and section)."""
import json
import math
import os

import numpy as np

import synth
from oracle import ref

GOLDEN = {v["name"]: v["value"] for v in
          json.load(open(os.path.join(os.path.dirname(__file__), "golden", "k3_printed_values.json")))["values"]}


def test_gated_product_bound_is_beta1_times_beta2():
    """The gated product SiTU(p1; beta1) * softcap(p2; beta2) stays below the
    printed bound and approaches it when both inputs are large and positive."""
    b1, b2 = GOLDEN["beta1"], GOLDEN["beta2"]
    assert b1 * b2 == GOLDEN["gated_product_bound"]
    x = np.concatenate([np.linspace(-1e4, 1e4, 2001), [-1e30, 1e30]])
    p1, p2 = np.meshgrid(x, x)
    a = ref.situ_glu_hidden(p1, p2, b1, b2)
    assert np.all(np.abs(a) <= GOLDEN["gated_product_bound"])
    top = ref.situ_glu_hidden(np.array([1e6]), np.array([1e6]), b1, b2)[0]
    assert math.isclose(top, GOLDEN["gated_product_bound"], rel_tol=1e-12)


def test_situ_gate_within_its_printed_range():
    """SiTU(x; 4) lies in (-4, 4): the cap's range times a sigmoid in (0, 1)."""
    b = GOLDEN["situ_gate_bound"]
    assert b == GOLDEN["beta1"]
    x = np.linspace(-60.0, 60.0, 24001)  # tanh(x / 4) still below 1 in fp64
    g = ref.situ(x, b)
    assert np.all(g > -b) and np.all(g < b)
    assert g.max() > b - 1e-9  # reaches towards the upper cap for large positive inputs
    assert np.all(np.abs(ref.situ(np.array([-1e30, 1e30]), b)) <= b)  # and never beyond it


def test_k3_workload_shapes_follow_the_printed_layer():
    """The K3-shaped workloads use the printed widths, expert pool, top-k, shared
    experts and bin count; the latent is half the hidden width, and the larger
    pool keeps the sparsity of the one it replaced."""
    for name in ("C2", "C3", "C4"):
        cfg = synth.get_config(name)
        assert cfg.d == GOLDEN["hidden_d"] and cfg.L == GOLDEN["latent_dim"] == cfg.d // 2
        assert cfg.n == GOLDEN["routed_experts"] and cfg.k == GOLDEN["top_k"]
        assert cfg.n_shared == GOLDEN["shared_experts"]
        assert (cfg.beta1, cfg.beta2) == (GOLDEN["beta1"], GOLDEN["beta2"])
    assert synth.get_config("C4").nbins == GOLDEN["qb_bins"]
    assert GOLDEN["top_k"] * GOLDEN["routed_experts_before_latent"] == \
        GOLDEN["top_k_before_latent"] * GOLDEN["routed_experts"]


def test_qb_reads_agree_between_the_two_printed_bin_counts():
    """With 1000 and with 10000 bins the QB read of a smooth score distribution
    agrees to within one 1000-bin width (the pages find 1000 bins enough)."""
    rng = np.random.default_rng(0)
    s = (1.0 / (1.0 + np.exp(-rng.standard_normal((20000, 8)) * 1.5))).astype(np.float32)
    k, n = 2, 8
    for e in range(n):
        h1 = ref.qb_histogram(s[:, e:e + 1], GOLDEN["qb_bins"])[0]
        h2 = ref.qb_histogram(s[:, e:e + 1], GOLDEN["qb_bins_compared"])[0]
        q1 = ref.qb_read(h1, h1.sum() * k / n)
        q2 = ref.qb_read(h2, h2.sum() * k / n)
        assert abs(q1 - q2) <= 1.0 / GOLDEN["qb_bins"]
