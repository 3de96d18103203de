"""Pins of the oracle's full layer: a hand-worked example with closed-form
values, library special cases (RMSNorm, SwiGLU limit) and invariances.

Sources: "Kimi K3 Architecture Deep Dive" §2 (LatentMoE d -> d/2 -> D -> d/2
-> d, one RMS norm before the up-projection, no hand-tuned routed scale);
LeiPhone report "LatentMoE: paying for a bigger pool" (two always-on shared
experts) and "Keeping the numbers in range" (norm after aggregation).
"""
import math

import numpy as np
import pytest
import torch

from oracle import ref
import synth

LN2, LN3 = math.log(2), math.log(3)
A = 768 / 17          # SiTU(4 ln2; 4) * softcap(25 ln3; 25) = (192/85) * 20


def hand_params(bias=None):
    """T=1, d=4, L=2, n=2, D=1, one shared expert; x = e0 gives z = (ln2, ln3),
    router logits (ln3, 0) -> scores (3/4, 1/2); every expert's gate sees 4 ln2 and
    its linear branch 25 ln3, so each gated hidden equals A = 768/17."""
    w_down = np.array([[LN2, 0, 0, 0], [LN3, 0, 0, 0]])
    w_router = np.array([[0.0, 1.0], [0.0, 0.0]])
    w1 = np.array([[[4.0, 0.0]], [[4.0, 0.0]]])
    w2 = np.array([[[0.0, 25.0]], [[0.0, 25.0]]])
    w3 = np.array([[[1.0], [0.0]], [[0.0], [1.0]]])
    ws1 = np.array([[[4.0, 0.0]]])
    ws2 = np.array([[[0.0, 25.0]]])
    ws3 = np.array([[[0.0], [0.75]]])
    w_up = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [1.0, -1.0]])
    return ref.ArrayParams(w_down, w_router, w1, w2, w3, w_up, ws1, ws2, ws3, bias=bias)


X1 = np.array([[1.0, 0.0, 0.0, 0.0]])


def test_hand_example_top1():
    # expert 0 chosen (3/4 > 1/2), g = 1: u = (A, 0) + shared (0, 3A/4);
    # RMS(u) = 5A / (4 sqrt 2)  ->  v = (4 sqrt2 / 5, 3 sqrt2 / 5)
    out = ref.forward(X1, hand_params(), k=1, n_shared=1, dtype="f64", eps=0.0)
    assert out["z"] == pytest.approx(np.array([[LN2, LN3]]), rel=1e-15)
    assert out["s"] == pytest.approx(np.array([[0.75, 0.5]]), rel=1e-15)
    assert out["idx"].tolist() == [[0]] and out["g"].tolist() == [[1.0]]
    assert out["u"] == pytest.approx(np.array([[A, 0.75 * A]]), rel=1e-13)
    r2 = math.sqrt(2)
    assert out["v"] == pytest.approx(np.array([[4 * r2 / 5, 3 * r2 / 5]]), rel=1e-13)
    assert out["y"] == pytest.approx(np.array([[4 * r2 / 5, 3 * r2 / 5, 7 * r2 / 5, r2 / 5]]), rel=1e-13)


def test_hand_example_bias_selects_other_expert():
    # bias (0, 0.3): biased scores (0.75, 0.8) -> expert 1; u = (0, A) + (0, 3A/4) = (0, 7A/4)
    out = ref.forward(X1, hand_params(bias=np.array([0.0, 0.3])), k=1, n_shared=1, dtype="f64", eps=0.0)
    assert out["idx"].tolist() == [[1]]
    assert out["u"] == pytest.approx(np.array([[0.0, 1.75 * A]]), rel=1e-13)
    r2 = math.sqrt(2)
    assert out["y"] == pytest.approx(np.array([[0.0, r2, r2, -r2]]), rel=1e-13, abs=1e-15)


def test_hand_example_top2_weights():
    # both experts, g = (3/5, 2/5) from unbiased scores even with a bias present
    out = ref.forward(X1, hand_params(bias=np.array([0.1, 0.0])), k=2, n_shared=1, dtype="f64", eps=0.0)
    assert out["g"] == pytest.approx(np.array([[0.6, 0.4]]), rel=1e-15)
    u = np.array([0.6 * A, 0.4 * A + 0.75 * A])
    assert out["u"] == pytest.approx(u[None], rel=1e-13)
    rms = A * math.sqrt((0.36 + 1.15 ** 2) / 2)
    v = u / rms
    assert out["v"] == pytest.approx(v[None], rel=1e-13)
    assert out["y"] == pytest.approx(np.array([[v[0], v[1], v[0] + v[1], v[0] - v[1]]]), rel=1e-13)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(5)
    u = rng.standard_normal((7, 96)) * 3
    gamma = rng.random(96) + 0.5
    mine = ref.rms_norm(u, gamma, 1e-6)
    lib = torch.nn.functional.rms_norm(torch.from_numpy(u), (96,), torch.from_numpy(gamma), 1e-6).numpy()
    assert np.allclose(mine, lib, rtol=1e-14, atol=0)
    # with gamma = 1, RMS(v) = sqrt(ms / (ms + eps))
    v = ref.rms_norm(u, np.ones(96), 0.5)
    ms = np.mean(u * u, axis=1)
    assert np.allclose(np.sqrt(np.mean(v * v, axis=1)), np.sqrt(ms / (ms + 0.5)), rtol=1e-14)


# --------------------------------------------------------------- randomised properties

def rand_params(rng, d=64, n=8, D=16, n_s=2, same_experts=False):
    L = d // 2
    w_down = rng.standard_normal((L, d)) / math.sqrt(d)
    w_router = rng.standard_normal((n, L)) / math.sqrt(L)
    if same_experts:
        w1 = np.repeat(rng.standard_normal((1, D, L)), n, 0) / math.sqrt(L)
        w2 = np.repeat(rng.standard_normal((1, D, L)), n, 0) / math.sqrt(L)
        w3 = np.repeat(rng.standard_normal((1, L, D)), n, 0) / math.sqrt(D)
    else:
        w1 = rng.standard_normal((n, D, L)) / math.sqrt(L)
        w2 = rng.standard_normal((n, D, L)) / math.sqrt(L)
        w3 = rng.standard_normal((n, L, D)) / math.sqrt(D)
    ws1 = rng.standard_normal((n_s, D, L)) / math.sqrt(L)
    ws2 = rng.standard_normal((n_s, D, L)) / math.sqrt(L)
    ws3 = rng.standard_normal((n_s, L, D)) / math.sqrt(D)
    w_up = rng.standard_normal((d, L)) / math.sqrt(L)
    bias = rng.standard_normal(n) * 0.05
    return dict(w_down=w_down, w_router=w_router, w1=w1, w2=w2, w3=w3, w_up=w_up, ws1=ws1, ws2=ws2,
                ws3=ws3, bias=bias)


def P(dct, **kw):
    d = dict(dct)
    d.update(kw)
    return ref.ArrayParams(**d)


def test_identical_experts_all_selected_reduce_to_one_expert():
    # k = n with identical experts: the routed mixture is that one expert (weights sum to 1)
    rng = np.random.default_rng(6)
    p = rand_params(rng, same_experts=True, n_s=1)
    x = rng.standard_normal((5, 64))
    out = ref.forward(x, P(p), k=8, n_shared=1, dtype="f64")
    z = out["z"]
    one = ref.expert_hidden(z, p["w1"][0], p["w2"][0], 4.0, 25.0, "f64") @ p["w3"][0].T
    sh = ref.expert_hidden(z, p["ws1"][0], p["ws2"][0], 4.0, 25.0, "f64") @ p["ws3"][0].T
    assert np.allclose(out["u"], one + sh, rtol=1e-12, atol=1e-14)


def test_zero_routed_output_leaves_shared_path():
    rng = np.random.default_rng(7)
    p = rand_params(rng)
    x = rng.standard_normal((6, 64))
    out = ref.forward(x, P(p, w3=np.zeros_like(p["w3"])), k=3, n_shared=2, dtype="f64")
    z = x @ p["w_down"].T
    sh = sum(ref.expert_hidden(z, p["ws1"][j], p["ws2"][j], 4.0, 25.0, "f64") @ p["ws3"][j].T for j in range(2))
    y = ref.rms_norm(sh, np.ones(32), 1e-6) @ p["w_up"].T
    assert np.allclose(out["y"], y, rtol=1e-12, atol=1e-14)


def test_norm_makes_output_invariant_to_expert_output_scale():
    rng = np.random.default_rng(8)
    p = rand_params(rng)
    x = rng.standard_normal((6, 64))
    y0 = ref.forward(x, P(p), k=3, n_shared=2, dtype="f64", eps=0.0)["y"]
    y1 = ref.forward(x, P(p, w3=3.0 * p["w3"], ws3=3.0 * p["ws3"]), k=3, n_shared=2, dtype="f64", eps=0.0)["y"]
    assert np.allclose(y0, y1, rtol=1e-12, atol=1e-14)
    # scaling only the routed part changes the output (shared/routed balance matters)
    y2 = ref.forward(x, P(p, w3=3.0 * p["w3"]), k=3, n_shared=2, dtype="f64", eps=0.0)["y"]
    assert not np.allclose(y0, y2, rtol=1e-6)


def test_bias_shift_and_expert_permutation_invariance():
    rng = np.random.default_rng(9)
    p = rand_params(rng)
    x = rng.standard_normal((10, 64))
    base = ref.forward(x, P(p), k=3, n_shared=2, dtype="f64")
    shifted = ref.forward(x, P(p, bias=p["bias"] + 0.25), k=3, n_shared=2, dtype="f64")
    assert np.array_equal(base["idx"], shifted["idx"])
    assert np.allclose(base["y"], shifted["y"], rtol=1e-13, atol=1e-15)
    perm = rng.permutation(8)
    inv = np.argsort(perm)
    pp = P(p, w_router=p["w_router"][perm], w1=p["w1"][perm], w2=p["w2"][perm], w3=p["w3"][perm],
           bias=p["bias"][perm])
    out = ref.forward(x, pp, k=3, n_shared=2, dtype="f64")
    assert np.array_equal(np.sort(perm[out["idx"]], 1), np.sort(base["idx"], 1))
    assert np.allclose(out["y"], base["y"], rtol=1e-12, atol=1e-14)
    _ = inv


def test_token_independence():
    rng = np.random.default_rng(10)
    p = rand_params(rng)
    x = rng.standard_normal((12, 64))
    full = ref.forward(x, P(p), k=3, n_shared=2, dtype="bf16")
    for t in (0, 5, 11):
        one = ref.forward(x[t:t + 1], P(p), k=3, n_shared=2, dtype="bf16")
        assert np.array_equal(one["y"][0], full["y"][t])


@pytest.mark.parametrize("beta,gate", [(1e30, "tanh"), (np.inf, "tanh"), (1e30, "clip"), (np.inf, "clip")])
def test_swiglu_limit_of_layer_against_torch_experts(beta, gate):
    # beta -> infinity turns every expert into SwiGLU, whichever cap (softcap or
    # hard clip) is lifted; build that expert from torch's silu
    rng = np.random.default_rng(11)
    p = rand_params(rng, n_s=1)
    x = rng.standard_normal((4, 64))
    out = ref.forward(x, P(p), k=2, n_shared=1, dtype="f64", beta1=beta, beta2=beta, eps=0.0, gate=gate)
    z = torch.from_numpy(out["z"])
    u = torch.zeros_like(z)
    for t in range(4):
        for j in range(2):
            e = int(out["idx"][t, j])
            h = torch.nn.functional.silu(torch.from_numpy(p["w1"][e]) @ z[t]) * (torch.from_numpy(p["w2"][e]) @ z[t])
            u[t] += float(out["g"][t, j]) * (torch.from_numpy(p["w3"][e]) @ h)
        hs = torch.nn.functional.silu(torch.from_numpy(p["ws1"][0]) @ z[t]) * (torch.from_numpy(p["ws2"][0]) @ z[t])
        u[t] += torch.from_numpy(p["ws3"][0]) @ hs
    assert np.allclose(out["u"], u.numpy(), rtol=1e-12, atol=1e-14)


def test_hard_clip_layer_matches_hardtanh_experts():
    # the hard-clip ablation: every expert's caps are torch's hardtanh at beta1, beta2
    rng = np.random.default_rng(13)
    p = rand_params(rng, n_s=1)
    x = rng.standard_normal((4, 64)) * 30
    out = ref.forward(x, P(p), k=2, n_shared=1, dtype="f64", eps=0.0, gate="clip")
    tanh = ref.forward(x, P(p), k=2, n_shared=1, dtype="f64", eps=0.0)
    assert np.array_equal(out["idx"], tanh["idx"])   # the gate does not touch routing
    z = torch.from_numpy(out["z"])
    ht = torch.nn.functional.hardtanh

    def hidden(w1, w2, zt):
        q1, q2 = w1 @ zt, w2 @ zt
        return ht(q1, -4.0, 4.0) * torch.sigmoid(q1) * ht(q2, -25.0, 25.0)

    u = torch.zeros_like(z)
    for t in range(4):
        for j in range(2):
            e = int(out["idx"][t, j])
            h = hidden(torch.from_numpy(p["w1"][e]), torch.from_numpy(p["w2"][e]), z[t])
            u[t] += float(out["g"][t, j]) * (torch.from_numpy(p["w3"][e]) @ h)
        u[t] += torch.from_numpy(p["ws3"][0]) @ hidden(torch.from_numpy(p["ws1"][0]), torch.from_numpy(p["ws2"][0]), z[t])
    assert np.allclose(out["u"], u.numpy(), rtol=1e-12, atol=1e-12)
    assert not np.allclose(out["u"], tanh["u"])


def test_no_norm_ablation_against_the_normed_layer():
    # without the norm, v = u: y is the normed layer's y times each token's RMS(u)
    # (gain 1, eps 0), and it scales with the expert outputs, which the norm cancels
    rng = np.random.default_rng(14)
    p = rand_params(rng, n_s=1)
    x = rng.standard_normal((5, 64))
    normed = ref.forward(x, P(p), k=2, n_shared=1, dtype="f64", eps=0.0)
    plain = ref.forward(x, P(p), k=2, n_shared=1, dtype="f64", eps=0.0, norm="none")
    assert np.array_equal(plain["u"], normed["u"]) and np.array_equal(plain["v"], plain["u"])
    rms = np.sqrt(np.mean(normed["u"] ** 2, axis=1, keepdims=True))
    assert np.allclose(plain["y"], normed["y"] * rms, rtol=1e-12, atol=1e-14)
    q = dict(p)
    q["w3"] = p["w3"] * 3.0
    q["ws3"] = p["ws3"] * 3.0
    assert np.allclose(ref.forward(x, P(q), k=2, n_shared=1, dtype="f64", eps=0.0, norm="none")["y"],
                       3.0 * plain["y"], rtol=1e-12, atol=1e-14)
    assert np.allclose(ref.forward(x, P(q), k=2, n_shared=1, dtype="f64", eps=0.0)["y"], normed["y"],
                       rtol=1e-12, atol=1e-14)
    with pytest.raises(ValueError):
        ref.forward(x, P(p), k=2, n_shared=1, dtype="f64", norm="layer")


def test_extra_down_norm_ablation_is_a_per_token_input_rescale():
    # z is linear in x, so norming z after the down-projection (eps 0) is the
    # normed layer run on x_t / RMS(z_t); and the layer forgets each token's scale
    rng = np.random.default_rng(15)
    p = rand_params(rng, n_s=1)
    x = rng.standard_normal((5, 64))
    both = ref.forward(x, P(p), k=2, n_shared=1, dtype="f64", eps=0.0, norm="both")
    z = x @ p["w_down"].T
    xs = x / np.sqrt(np.mean(z ** 2, axis=1, keepdims=True))
    rms = ref.forward(xs, P(p), k=2, n_shared=1, dtype="f64", eps=0.0)
    assert np.array_equal(both["idx"], rms["idx"])
    assert np.allclose(both["z"], rms["z"], rtol=1e-12, atol=1e-14)
    assert np.allclose(both["y"], rms["y"], rtol=1e-10, atol=1e-12)
    assert np.allclose(np.mean(both["z"] ** 2, axis=1), 1.0, rtol=1e-12)
    c = np.array([0.01, 0.5, 3.0, 40.0, 1e3])[:, None]
    scaled = ref.forward(x * c, P(p), k=2, n_shared=1, dtype="f64", eps=0.0, norm="both")
    assert np.array_equal(scaled["idx"], both["idx"])
    assert np.allclose(scaled["y"], both["y"], rtol=1e-10, atol=1e-12)
    # without it a token's scale reaches the router (the sigmoid is not scale free)
    plain = ref.forward(x * c, P(p), k=2, n_shared=1, dtype="f64", eps=0.0)
    assert not np.allclose(plain["s"], ref.forward(x, P(p), k=2, n_shared=1, dtype="f64", eps=0.0)["s"])


def test_gated_hidden_bounded_on_outlier_tokens():
    # the configured C2 outliers (x50) saturate the caps but never exceed beta1*beta2
    rng = np.random.default_rng(12)
    p = rand_params(rng)
    x = rng.standard_normal((4, 64)) * 50
    z = x @ p["w_down"].T
    a = ref.expert_hidden(z, p["w1"][0] * 20, p["w2"][0] * 20, 4.0, 25.0, "bf16")
    assert np.all(np.abs(a) <= 100.0)


def test_synth_params_feed_the_oracle():
    cfg = synth.get_config("C0")
    hp = synth.HostParams(cfg)
    x = hp.x()
    assert x.shape == (64, 256) and x.dtype == np.float64
    out = ref.forward(x[:8], hp, cfg.k, cfg.n_shared, "f32")
    assert out["y"].shape == (8, 256) and np.all(np.isfinite(out["y"]))
    assert np.array_equal(out["y"], out["y"].astype(np.float32).astype(np.float64))
