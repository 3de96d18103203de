"""Pins of the oracle's backward pass.

Sources: "Kimi K3 Architecture Deep Dive" §1 (softcap and SiTU, whose
gradients do not vanish abruptly as a clip's do) and §2 (effect 6: the
up-projection's gradient in the normalised form g (h / |h|_RMS)^T).

The backward is checked against what fixes it independently of its own
formulas: central finite differences of the forward (with the routing held
fixed, so the layer is smooth), torch autograd through a torch statement of
the same forward, closed forms of the cap derivatives, and the norm's scale
invariance.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ref

B1, B2 = 1.5, 2.0  # small caps so that the tiny layer's gate inputs reach the curved part


def test_cap_derivatives_closed_forms():
    # tanh(ln 3) = 4/5: softcap'(beta ln 3) = 1 - 16/25 = 9/25; sigmoid(ln 3) = 3/4
    b = 2.5
    x = b * math.log(3)
    assert ref.softcap_grad(x, b) == pytest.approx(9 / 25, rel=1e-14)
    sg = 0.75 if x == math.log(3) else 1 / (1 + math.exp(-x))
    want = 9 / 25 * sg + b * 0.8 * sg * (1 - sg)
    assert ref.situ_grad(x, b) == pytest.approx(want, rel=1e-13)
    assert ref.softcap_grad(np.array([0.3, -7.0]), np.inf).tolist() == [1.0, 1.0]
    assert ref.softcap_grad(np.array([-2.0, 0.5, 1.9, 2.0, 3.0]), 2.0, "clip").tolist() == [0, 1, 1, 0, 0]


def test_cap_derivatives_match_finite_differences():
    x = np.linspace(-9, 9, 37) + 0.013
    h = 1e-6
    for gate in ("tanh", "clip"):
        for b in (1.0, 4.0, 25.0):
            fd = (ref.cap(x + h, b, gate) - ref.cap(x - h, b, gate)) / (2 * h)
            assert np.allclose(ref.softcap_grad(x, b, gate), fd, atol=1e-7)
            fd = (ref.situ(x + h, b, gate) - ref.situ(x - h, b, gate)) / (2 * h)
            assert np.allclose(ref.situ_grad(x, b, gate), fd, atol=1e-7)


def tiny(seed=0, T=5, d=8, L=4, n=6, k=2, ns=1, D=3, scale=1.2):
    rng = np.random.default_rng(seed)

    def w(*shape):
        return rng.standard_normal(shape) * scale / math.sqrt(shape[-1])

    arrs = dict(w_down=w(L, d), w_router=w(n, L) * 2, w1=w(n, D, L) * 3, w2=w(n, D, L) * 3, w3=w(n, L, D),
                w_up=w(d, L), ws1=w(ns, D, L) * 3, ws2=w(ns, D, L) * 3, ws3=w(ns, L, D),
                gamma=1 + 0.3 * rng.standard_normal(L), bias=0.1 * rng.standard_normal(n),
                logit_offset=0.2 * rng.standard_normal(n))
    x = rng.standard_normal((T, d)) * 2
    dy = rng.standard_normal((T, d))
    return arrs, x, dy, k, ns


def params(a):
    return ref.ArrayParams(a["w_down"], a["w_router"], a["w1"], a["w2"], a["w3"], a["w_up"], a["ws1"], a["ws2"],
                           a["ws3"], bias=a["bias"], logit_offset=a["logit_offset"], gamma=a["gamma"])


GRADS = {"w_down": "dw_down", "w_router": "dw_router", "w1": "dw1", "w2": "dw2", "w3": "dw3", "w_up": "dw_up",
         "ws1": "dws1", "ws2": "dws2", "ws3": "dws3", "gamma": "dgamma"}


@pytest.mark.parametrize("gate,norm,betas", [("tanh", "rms", (B1, B2)), ("tanh", "rms", (4.0, 25.0)),
                                             ("clip", "rms", (B1, B2)), ("tanh", "none", (B1, B2))])
def test_gradients_match_finite_differences(gate, norm, betas):
    """Directional derivatives of L = sum(dy * y) along random directions, for
    every parameter and the input, against the backward's gradients; the
    routing is held fixed (forced) so L is smooth, and eps keeps the norm
    smooth.  Everything in fp64 (no store rounding)."""
    a, x, dy, k, ns = tiny()
    b1, b2 = betas
    eps = 1e-3
    out = ref.forward(x, params(a), k, ns, "f64", b1, b2, eps, gate=gate, norm=norm)
    idx = out["idx"]
    g = ref.backward(x, params(a), k, ns, "f64", dy, b1, b2, eps, forced_idx=idx, gate=gate, norm=norm)

    def loss(aa, xx):
        y = ref.forward(xx, params(aa), k, ns, "f64", b1, b2, eps, forced_idx=idx, gate=gate, norm=norm)["y"]
        return float(np.sum(dy * y))

    rng = np.random.default_rng(1)
    h = 1e-6
    names = [nm for nm in GRADS if not (norm == "none" and nm == "gamma")]
    for nm in names + ["x"]:
        base = x if nm == "x" else a[nm]
        dirn = rng.standard_normal(base.shape)
        if nm == "x":
            fd = (loss(a, x + h * dirn) - loss(a, x - h * dirn)) / (2 * h)
            an = float(np.sum(g["dx"] * dirn))
        else:
            ap, am = dict(a), dict(a)
            ap[nm], am[nm] = base + h * dirn, base - h * dirn
            fd = (loss(ap, x) - loss(am, x)) / (2 * h)
            an = float(np.sum(g[GRADS[nm]] * dirn))
        assert an == pytest.approx(fd, rel=1e-6, abs=1e-8), nm
    if norm == "none":
        assert not g["dgamma"].any()


def torch_forward(a, x, k, ns, idx, b1, b2, eps):
    """The layer in torch (fp64), routing forced to idx, for autograd."""
    t = {kk: torch.tensor(v, dtype=torch.float64, requires_grad=kk not in ("bias", "logit_offset"))
         for kk, v in a.items()}
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    z = xt @ t["w_down"].T
    s = torch.sigmoid(z @ t["w_router"].T + t["logit_offset"])
    it = torch.tensor(idx)
    sk = torch.gather(s, 1, it)
    g = sk / sk.sum(1, keepdim=True)

    def capf(v, b):
        return b * torch.tanh(v / b)

    def hidden(zr, w1, w2):
        p1, p2 = zr @ w1.T, zr @ w2.T
        return capf(p1, b1) * torch.sigmoid(p1) * capf(p2, b2)

    u = torch.zeros_like(z)
    for j in range(k):
        rows = []
        for i in range(z.shape[0]):
            e = int(idx[i, j])
            rows.append(hidden(z[i:i + 1], t["w1"][e], t["w2"][e]) @ t["w3"][e].T)
        u = u + g[:, j:j + 1] * torch.cat(rows)
    for j in range(ns):
        u = u + hidden(z, t["ws1"][j], t["ws2"][j]) @ t["ws3"][j].T
    v = t["gamma"] * u / torch.sqrt(torch.mean(u * u, 1, keepdim=True) + eps)
    return t, xt, v @ t["w_up"].T


def test_gradients_match_torch_autograd():
    a, x, dy, k, ns = tiny(seed=3, T=7)
    eps = 1e-6
    idx = ref.forward(x, params(a), k, ns, "f64", B1, B2, eps)["idx"]
    g = ref.backward(x, params(a), k, ns, "f64", dy, B1, B2, eps, forced_idx=idx)
    t, xt, y = torch_forward(a, x, k, ns, idx, B1, B2, eps)
    (y * torch.tensor(dy)).sum().backward()
    assert np.allclose(g["dx"], xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    for nm, gk in GRADS.items():
        assert np.allclose(g[gk], t[nm].grad.numpy(), rtol=1e-10, atol=1e-12), nm


def test_norm_backward_is_orthogonal_to_u():
    """With eps = 0 and unit gain the normed latent is invariant to each token's
    scale, so the latent's gradient is orthogonal to u: sum_l du_l u_l = 0."""
    a, x, dy, k, ns = tiny(seed=5)
    a["gamma"] = np.ones_like(a["gamma"])
    g = ref.backward(x, params(a), k, ns, "f64", dy, B1, B2, 0.0)
    u = g["fw"]["u"]
    assert np.allclose(np.sum(g["du"] * u, axis=1), 0.0, atol=1e-12)


def test_router_gradient_only_on_chosen_experts_and_bias_shift_invariant():
    a, x, dy, k, ns = tiny(seed=7, T=9)
    g = ref.backward(x, params(a), k, ns, "f64", dy, B1, B2, 1e-6)
    chosen = np.zeros_like(g["dl"], dtype=bool)
    np.put_along_axis(chosen, g["fw"]["idx"], True, axis=1)
    assert not g["dl"][~chosen].any()
    # the routing weights sum to one, so their gradient has no component along g: sum_j ds_j s_j = 0
    sk = np.take_along_axis(g["fw"]["s"], g["fw"]["idx"], 1)
    dlk = np.take_along_axis(g["dl"], g["fw"]["idx"], 1)
    assert np.allclose(np.sum(dlk / (1 - sk), axis=1), 0.0, atol=1e-12)
    a2 = dict(a)
    a2["bias"] = a["bias"] + 0.375
    g2 = ref.backward(x, params(a2), k, ns, "f64", dy, B1, B2, 1e-6)
    for key in ("dx", "dw_router", "dw1", "dw_up"):
        assert np.array_equal(g[key], g2[key])


def _nudged_pair(cfg, rel, seed=0):
    """The oracle's backward, plain and with every value nudged by a relative
    N(0, rel) just before each of its work-dtype stores (a second correct
    implementation whose pre-store values differ by rel)."""
    import synth
    P = synth.HostParams(cfg, cache=True)
    x = P.x()
    dy = synth.host_fill_values((cfg.T, cfg.d), cfg.x_seed, synth.TID["dy"], 0, 1.0, cfg.dtype)
    args = (cfg.k, cfg.n_shared, cfg.dtype, dy, cfg.beta1, cfg.beta2, cfg.eps)
    idx = ref.forward(x, P, cfg.k, cfg.n_shared, cfg.dtype, cfg.beta1, cfg.beta2, cfg.eps)["idx"]
    a = ref.backward(x, P, *args, forced_idx=idx)
    rng = np.random.default_rng(seed)
    plain = ref.round_to
    ref.round_to = lambda v, dt: plain(np.asarray(v, np.float64) * (1 + rel * rng.standard_normal(np.shape(v))), dt)
    try:
        b = ref.backward(x, P, *args, forced_idx=idx)
    finally:
        ref.round_to = plain
    return a, b, np.bincount(idx.ravel(), minlength=cfg.n)


BF16_SHAPES = {
    "mid": dict(T=1024, d=512, L=256, n=64, k=8, n_shared=2, D=128, dtype="bf16"),
    "sparse": dict(T=130, d=384, L=192, n=1024, k=3, n_shared=2, D=192, dtype="bf16"),  # most experts 0-1 tokens
}


@pytest.mark.parametrize("shape", list(BF16_SHAPES))
def test_bf16_gradient_rule_sits_above_the_rounding_floor(shape):
    """The bf16 matching rule for the gradients is not tighter than the
    arithmetic allows: the oracle against itself, with pre-store values nudged
    by 5e-4 (fp16 staging of the expert rows is 2^-11), meets it with 0.6 of
    every bound."""
    import bwd_rule
    import synth
    cfg = synth.get_config("C0").with_(x_seed=21, w_seed=21, bias_std=0.05, **BF16_SHAPES[shape])
    a, b, counts = _nudged_pair(cfg, 5e-4)
    for nm in ("dx", "dw_down", "dw_router", "dw1", "dw2", "dw3", "dws1", "dws2", "dws3", "dgamma", "dw_up"):
        m, bad = bwd_rule.failures("bf16", cfg.d, nm, b[nm], a[nm], counts, scale=0.6)
        assert not bad, (nm, bad)


def test_routed_bank_maximum_is_ill_conditioned():
    """Why the rule bounds a routed bank's bulk and each expert's RMS rather than
    the bank's maximum: with about one token per expert, nudging the pre-store
    values by only 1e-6 already moves some element of dW1 by more than the
    forward's 2e-2 of the bank's RMS."""
    import synth
    cfg = synth.get_config("C0").with_(x_seed=21, w_seed=21, bias_std=0.05, **BF16_SHAPES["sparse"])
    a, b, _ = _nudged_pair(cfg, 1e-6)
    d = np.abs(a["dw1"] - b["dw1"]).max() / np.sqrt(np.mean(a["dw1"] ** 2))
    assert d > 2e-2
