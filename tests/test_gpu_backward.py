"""GPU parity of lmoe_backward (the layer's backward pass, through the C ABI)
against the oracle's backward on the GPU's routing, by the matching rule of
bwd_rule (fp32 as the forward; bf16 bounds on the bulk everywhere, on the
maximum of the dense gradients and on each routed expert's own RMS, derived
there from the chained bf16 stores and pinned against the oracle's rounding
floor by a CPU test).

Sources: "Kimi K3 Architecture Deep Dive" §1 (the capped gate) and §2 (the
norm before the up-projection and its normalised gradient form).

The oracle stores the backward's intermediates (du, g du, da, dp1, dp2, dl,
dz) in the work dtype where the library does, and compares before each
gradient's own store rounding.  The upstream gradient dy is a seeded
synthetic N(0, 1) tensor.
"""
import numpy as np
import pytest
import torch

import sparse_moe_layer_down_amd as lmoe
import synth
from oracle import ref

import bwd_rule
from test_gpu_forward import check_topk_valid

pytestmark = pytest.mark.gpu

GRADS = ("dx", "dw_down", "dw_router", "dw1", "dw2", "dw3", "dws1", "dws2", "dws3", "dgamma", "dw_up")


def dy_host(cfg, T):
    return synth.host_fill_values((T, cfg.d), cfg.x_seed, synth.TID["dy"], 0, 1.0, cfg.dtype)


def run_gpu_bwd(cfg, weights=None):
    dev = torch.device("cuda:0")
    w = weights if weights is not None else synth.device_params(cfg, device=dev, with_x=False)
    x = synth.params.device_x(cfg, dev)
    T = x.shape[0]
    dy = torch.empty_like(x)
    synth.device_fill(dy, cfg.x_seed, synth.TID["dy"], 0, 1.0)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    s = torch.empty((T, cfg.n), dtype=torch.float32, device=dev)
    dims = lmoe.dims_of(x, w, cfg.k)
    ws = lmoe.make_workspace(dims, x.dtype, dev)
    kw = dict(beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, gate=cfg.gate, norm=cfg.norm)
    lmoe.forward(x, w, cfg.k, topk_idx=idx, topk_w=tw, scores=s, workspace=ws, **kw)
    g = lmoe.backward(x, dy, w, cfg.k, idx, tw, s, ws, **kw)
    torch.cuda.synchronize()
    out = {kk: (None if v is None else v.double().cpu().numpy()) for kk, v in g.items()}
    out["idx"] = idx.cpu().numpy().astype(np.int64)
    out["s"] = s.double().cpu().numpy()
    out["_v"] = lmoe.workspace_view(ws, dims, x.dtype, "v")
    out["_dy"] = dy
    return out


def check_grad(dtype, K, name, got, want, label, counts=None):
    """Apply the matching rule to one gradient; returns the failure text or None."""
    import conftest
    m, bad = bwd_rule.failures(dtype, K, name, got, want, counts)
    for key, bound in (("max", bwd_rule.fp32_tol(K)),) if dtype == "f32" else \
            (("rms", bwd_rule.BF16_RMS), ("max", bwd_rule.BF16_MAX), ("expert_rms", bwd_rule.BF16_EXPERT_RMS)):
        if key in m and (key != "max" or dtype == "f32" or bwd_rule.kind_of(name) == "dense"):
            conftest.MARGINS.append((f"{label} {key}", m[key], bound))
    print(f"  {label:34s} {bwd_rule.describe(m)}", flush=True)
    return f"{label}: " + ", ".join(bad) if bad else None


def compare(cfg, gpu, want, label, keys=GRADS):
    counts = np.bincount(gpu["idx"].ravel(), minlength=cfg.n)
    bad = [f for kk in keys if gpu.get(kk) is not None
           for f in [check_grad(cfg.dtype, max(cfg.d, cfg.T), kk, gpu[kk], want[kk], f"{label} {kk}", counts)] if f]
    assert not bad, "; ".join(bad)


def full_check(cfg):
    print(f"\n[{cfg.name} T={cfg.T} n={cfg.n} k={cfg.k} {cfg.dtype}] GPU backward", flush=True)
    gpu = run_gpu_bwd(cfg)
    print("  GPU done; oracle backward", flush=True)
    P = synth.HostParams(cfg, cache=True)
    check_topk_valid(gpu["s"], P.bias(), gpu["idx"])
    want = ref.backward(P.x(), P, cfg.k, cfg.n_shared, cfg.dtype, dy_host(cfg, cfg.T), cfg.beta1, cfg.beta2, cfg.eps,
                        forced_idx=gpu["idx"], gate=cfg.gate, norm=cfg.norm)
    compare(cfg, gpu, want, f"{cfg.name} T={cfg.T} bwd")
    for kk in GRADS:
        if gpu.get(kk) is not None:
            assert np.isfinite(gpu[kk]).all(), kk
    return gpu, want


def test_backward_c0_tiny_fp32():
    full_check(synth.get_config("C0"))


def test_backward_c1_small_bf16():
    full_check(synth.get_config("C1"))


@pytest.mark.parametrize("shape", [
    dict(T=1000, d=256, L=128, n=40, k=5, n_shared=0, D=128, dtype="bf16"),     # no shared experts
    dict(T=333, d=512, L=256, n=200, k=7, n_shared=3, D=64, dtype="bf16"),      # three shared experts
    dict(T=257, d=256, L=128, n=64, k=64, n_shared=1, D=64, dtype="f32"),       # k = n: every expert
    dict(T=1, d=128, L=64, n=1, k=1, n_shared=1, D=64, dtype="f32"),            # one token
    dict(T=130, d=384, L=192, n=1024, k=3, n_shared=2, D=192, dtype="bf16"),    # most experts get no token
    dict(T=777, d=256, L=128, n=700, k=16, n_shared=2, D=64, dtype="bf16"),     # the K3 top-k kernel
    dict(T=70, d=4096, L=2048, n=16, k=2, n_shared=1, D=64, dtype="bf16"),      # wider latent
])
def test_backward_ragged_and_edge_shapes(shape):
    full_check(synth.get_config("C0").with_(x_seed=21, w_seed=21, bias_std=0.05, **shape))


@pytest.mark.parametrize("over", [dict(gate="clip"), dict(norm="none"), dict(beta1=np.inf, beta2=np.inf)])
def test_backward_ablations(over):
    # the hard clip's gradient (zero past the ceiling), no norm (du = dv) and
    # the uncapped SwiGLU experts (fp32 staged rows) through the same kernels
    full_check(synth.get_config("C1").with_(T=512, x_seed=41, **over))


def test_backward_k3_prefill_sampled():
    """The K3 prefill shape in the benchmark's launch configuration: dx of
    sampled tokens and the weight gradients of two routed experts are exact
    functions of the tokens involved, so the oracle's backward on exactly those
    tokens gives them; dW_up = dy^T v is checked on 16 of its rows from the
    GPU's stored v."""
    cfg = synth.get_config("C2")
    print("\n[C2] GPU backward", flush=True)
    gpu = run_gpu_bwd(cfg)
    print("  GPU done; oracle backward on sampled tokens", flush=True)
    for kk in GRADS:
        assert np.isfinite(gpu[kk]).all(), kk
    P = synth.HostParams(cfg, cache=True)
    rng = np.random.default_rng(5)
    counts = np.bincount(gpu["idx"].ravel(), minlength=cfg.n)
    experts = rng.choice(np.nonzero(counts)[0], 2, replace=False)
    toks = np.unique(np.concatenate([np.nonzero((gpu["idx"] == e).any(1))[0] for e in experts] +
                                    [rng.choice(cfg.T, 8, replace=False), synth.outlier_rows(cfg)[:2]]))
    x = P.x_rows(toks)
    dy = dy_host(cfg, cfg.T)[toks]
    want = ref.backward(x, P, cfg.k, cfg.n_shared, cfg.dtype, dy, cfg.beta1, cfg.beta2, cfg.eps,
                        forced_idx=gpu["idx"][toks])
    out = np.isin(toks, synth.outlier_rows(cfg))
    bad = []
    for sel, lab in ((~out, ""), (out, "outlier ")):
        if sel.any():
            bad.append(check_grad(cfg.dtype, cfg.d, "dx", gpu["dx"][toks[sel]], want["dx"][sel],
                                  f"C2 bwd {lab}sampled dx"))
    for kk in ("dw1", "dw2", "dw3"):  # the two experts as a bank of two, both with rows
        bad.append(check_grad(cfg.dtype, cfg.d, kk, gpu[kk][experts], want[kk][experts], f"C2 bwd experts {kk}",
                              np.ones(len(experts))))
    rows = rng.choice(cfg.d, 16, replace=False)
    v = gpu["_v"].double().cpu().numpy()
    dyg = gpu["_dy"].double().cpu().numpy()
    wup = dyg[:, rows].T @ v
    bad.append(check_grad(cfg.dtype, cfg.d, "dw_up", gpu["dw_up"][rows], wup, "C2 bwd dw_up rows"))
    bad = [b for b in bad if b]
    assert not bad, "; ".join(bad)


def test_backward_replays_from_a_hip_graph():
    """The backward enqueues kernels only (its tile counters are zeroed by a
    kernel, not a memset; no host synchronisation), and every output element is
    computed by one work-group, so a captured backward replays bit for bit: each
    of several replays, with a new upstream gradient copied in before two of them
    and unrelated eager forwards between them, equals the eager backward."""
    cfg = synth.get_config("C1").with_(T=512)
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev, with_x=False)
    x = synth.params.device_x(cfg, dev)
    T = x.shape[0]
    dy1 = torch.empty_like(x)
    synth.device_fill(dy1, cfg.x_seed, synth.TID["dy"], 0, 1.0)
    dy2 = torch.empty_like(x)
    synth.device_fill(dy2, cfg.x_seed + 1, synth.TID["dy"], 0, 1.0)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    s = torch.empty((T, cfg.n), dtype=torch.float32, device=dev)
    dims = lmoe.dims_of(x, w, cfg.k)
    ws = lmoe.make_workspace(dims, x.dtype, dev)
    kw = dict(beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps)
    lmoe.forward(x, w, cfg.k, topk_idx=idx, topk_w=tw, scores=s, workspace=ws, **kw)
    bws = torch.empty(lmoe.backward_workspace_size(dims, x.dtype), dtype=torch.uint8, device=dev)
    refs = []
    for dy in (dy1, dy2):
        g = lmoe.backward(x, dy, w, cfg.k, idx, tw, s, ws, workspace=bws, **kw)
        refs.append({kk: v.clone() for kk, v in g.items() if v is not None})
    dyin = dy1.clone()
    grads = lmoe.backward(x, dyin, w, cfg.k, idx, tw, s, ws, workspace=bws, **kw)  # the buffers the graph writes
    x_other = synth.params.device_x(cfg.with_(x_seed=9), dev)
    ws_other = lmoe.make_workspace(dims, x.dtype, dev)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lmoe.backward(x, dyin, w, cfg.k, idx, tw, s, ws, grads=grads, workspace=bws, **kw)
    for i, (src, want) in enumerate([(dy1, refs[0]), (dy2, refs[1]), (dy2, refs[1]), (dy1, refs[0])]):
        dyin.copy_(src)
        lmoe.forward(x_other, w, cfg.k, workspace=ws_other, **kw)  # unrelated eager work on the stream
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for kk, v in want.items():
            assert torch.equal(grads[kk], v), f"replay {i}: {kk}"
