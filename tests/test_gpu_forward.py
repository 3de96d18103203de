"""GPU parity of lmoe_forward against the CPU oracle (through the C ABI).

Matching rules: expert sets and the dispatch permutation bit-exact (sets are
compared only where the oracle's k-th/(k+1)-th biased-score gap is >= 1e-4;
the permutation is checked against the oracle's dispatch of the GPU's own
routing); floating-point outputs within max|err| <= 2e-2 * RMS(ref) for bf16
and 1e-5 * RMS(ref) for fp32.  The reference of a stored tensor is the
oracle's value before that tensor's own store rounding: a one-ulp difference
in the final bf16 rounding of an element above 2.56 * RMS already exceeds
2e-2 * RMS, whichever side of the rounding boundary is right.  Expert math is
compared with the oracle run on the GPU's routing, so near-tie tokens are
still checked.
"""
import numpy as np
import pytest
import torch

import sparse_moe_layer_down_amd as lmoe
import synth
from oracle import ref

pytestmark = pytest.mark.gpu

GAP = 1e-4


def tol(dtype, K=1024):
    """1e-5 for fp32 (the tiny fp32 configuration), 2e-2 for bf16.  For fp32 the
    rounding error of a K-term fp32 dot product grows like sqrt(K) * 2^-24 of the
    terms' RMS, so shapes whose longest contraction K (= d, the W_down length)
    exceeds 1024 get 1e-5 * sqrt(K / 1024); bf16 is dominated by the operand
    rounding and keeps 2e-2."""
    if dtype != "f32":
        return 2e-2
    return 1e-5 * max(1.0, (K / 1024.0) ** 0.5)


def rel_err(got, want, label=None, t=None):
    """max|got - want| / RMS(want); recorded for the run's margin summary when labelled."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rms = np.sqrt(np.mean(want ** 2))
    e = np.abs(got - want).max() / rms if want.size else 0.0
    if label is not None:
        import conftest
        conftest.MARGINS.append((label, float(e), t))
    return e


def rel_err_rows(got, want, label=None, t=None):
    """max over token rows of max|got - want| / RMS(want row).

    Without the norm the layer's v and y scale with each token's RMS(u)
    (y = RMS(u) * the normed y, with unit gain and zero epsilon), so the
    normed layer's bound relative to the batch RMS becomes a bound relative to
    each token's own RMS: the same rounding argument, token by token."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rms = np.sqrt(np.mean(want ** 2, axis=1))
    e = float((np.abs(got - want).max(axis=1) / rms).max()) if want.size else 0.0
    if label is not None:
        import conftest
        conftest.MARGINS.append((label, e, t))
    return e


def run_gpu(cfg, x=None, weights=None, step=None):
    dev = torch.device("cuda:0")
    w = weights if weights is not None else synth.device_params(cfg, device=dev, with_x=False)
    if x is None:
        x = synth.params.device_x(cfg, dev, step)
    T = x.shape[0]
    idx = torch.full((T, cfg.k), -1, dtype=torch.int32, device=dev)
    tw = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    s = torch.empty((T, cfg.n), dtype=torch.float32, device=dev)
    dims = lmoe.dims_of(x, w, cfg.k)
    ws = lmoe.make_workspace(dims, x.dtype, dev)
    y = lmoe.forward(x, w, cfg.k, topk_idx=idx, topk_w=tw, scores=s, workspace=ws,
                     beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, gate=cfg.gate, norm=cfg.norm)
    torch.cuda.synchronize()
    out = dict(y=y.double().cpu().numpy(), idx=idx.cpu().numpy().astype(np.int64), g=tw.double().cpu().numpy(),
               s=s.double().cpu().numpy())
    for r in ("z", "counts", "offs", "row_token", "row_slot", "hidden", "v"):
        out[r] = lmoe.workspace_view(ws, dims, x.dtype, r).cpu()
    # the staged rows stay on the device (up to ~1 GB); tests gather what they check
    out["rows_dev"] = lmoe.workspace_view(ws, dims, x.dtype, "rows",
                                          capped=bool(np.isfinite(cfg.beta1) and np.isfinite(cfg.beta2)))
    for r in ("z", "hidden", "v"):
        out[r] = out[r].double().numpy()
    for r in ("counts", "offs", "row_token", "row_slot"):
        out[r] = out[r].numpy().astype(np.int64)
    return out


def check_topk_valid(s, bias, idx):
    """Every token's list is a valid biased top-k of the GPU's own fp32 scores.

    The selection key is fp32(s) + fp32(b), one IEEE fp32 add as in the kernel.
    For every token: k distinct experts; min(chosen keys) >= max(unchosen keys);
    where the two meet, every chosen expert at that key has a lower index than
    every unchosen one (ties go to the lower index); the list is ordered by
    decreasing key, equal keys by increasing index.  Returns the number of
    tokens that had an exact tie at the threshold."""
    s32 = np.asarray(s, dtype=np.float32)
    b32 = np.asarray(bias, dtype=np.float32)
    sel = s32 + b32[None, :]
    idx = np.asarray(idx, dtype=np.int64)
    T, n = sel.shape
    k = idx.shape[1]
    assert idx.min() >= 0 and idx.max() < n, "expert index out of range"
    assert np.all(np.diff(np.sort(idx, axis=1), axis=1) > 0), "repeated expert in a token's list"
    chosen = np.zeros((T, n), dtype=bool)
    np.put_along_axis(chosen, idx, True, axis=1)
    cs = np.take_along_axis(sel, idx, axis=1)
    lo = cs.min(axis=1)
    if k == n:
        hi = np.full(T, -np.inf, dtype=np.float32)
    else:
        hi = np.where(chosen, np.float32(-np.inf), sel).max(axis=1)
    bad = np.nonzero(lo < hi)[0]
    assert bad.size == 0, f"{bad.size} tokens chose a lower key than one left out (first: token {bad[:1]})"
    ties = np.nonzero(lo == hi)[0]
    for t in ties:
        c_at = idx[t][cs[t] == lo[t]].max()
        u_at = np.nonzero(~chosen[t] & (sel[t] == lo[t]))[0].min()
        assert c_at < u_at, f"token {t}: tie at the threshold not broken by the lower index"
    d, di = np.diff(cs, axis=1), np.diff(idx, axis=1)
    assert np.all((d < 0) | ((d == 0) & (di > 0))), "list not ordered by (-key, index)"
    return int(ties.size)


def check_against_oracle(cfg, gpu, x_host, P, rows=None):
    """Compare a GPU forward with the oracle on the token rows `rows` (all if None)."""
    dt = cfg.dtype
    sel = np.arange(x_host.shape[0]) if rows is None else np.asarray(rows)
    g_idx = gpu["idx"][sel]
    # the oracle's own routing decision
    own = ref.forward(x_host, P, cfg.k, cfg.n_shared, dt, cfg.beta1, cfg.beta2, cfg.eps, gate=cfg.gate,
                      norm=cfg.norm)
    clear = own["gap"] >= GAP
    assert clear.mean() > 0.5
    assert np.array_equal(np.sort(own["idx"][clear], 1), np.sort(g_idx[clear], 1)), "top-k sets differ"
    # expert math on the GPU's routing
    forced = ref.forward(x_host, P, cfg.k, cfg.n_shared, dt, cfg.beta1, cfg.beta2, cfg.eps, forced_idx=g_idx,
                         gate=cfg.gate, norm=cfg.norm)
    tl = tol(dt, cfg.d)
    assert rel_err(gpu["z"][sel], forced["z_pre"], f"{cfg.name} z", tl) <= tl, "z"
    assert rel_err(gpu["s"][sel], forced["s"], f"{cfg.name} s", tl) <= tl, "scores"
    # routing weights from the GPU's own fp32 scores, order matching the GPU's list
    g_ref = ref.routing_weights(gpu["s"][sel], g_idx)
    assert np.abs(gpu["g"][sel] - g_ref).max() <= 1e-6
    # every token (near-ties included) chose a valid biased top-k of its own fp32 scores
    check_topk_valid(gpu["s"][sel], P.bias(), g_idx)
    err = rel_err_rows if cfg.norm == "none" else rel_err
    assert err(gpu["v"][sel], forced["v_pre"], f"{cfg.name} v", tl) <= tl, "v"
    assert err(gpu["y"][sel], forced["y_pre"], f"{cfg.name} y", tl) <= tl, "y"
    return own, forced


def check_dispatch(cfg, gpu):
    counts, offs, row_token, row_slot = ref.dispatch(gpu["idx"], cfg.n)
    T = gpu["idx"].shape[0]
    assert np.array_equal(gpu["counts"], counts)
    assert np.array_equal(gpu["offs"], offs)
    assert np.array_equal(gpu["row_token"][:T * cfg.k], row_token)
    # the shared experts' rows follow: row T*k + s*T + t is token t
    assert np.array_equal(gpu["row_token"][T * cfg.k:], np.tile(np.arange(T), cfg.n_shared))
    # row_slot region holds the dispatched row of each (token, slot)
    inv = np.empty_like(row_token)
    inv[row_token * cfg.k + row_slot] = np.arange(row_token.size)
    assert np.array_equal(gpu["row_slot"], inv)


def check_hidden(cfg, gpu, P, x_host):
    """Gated hidden of every dispatched row vs the oracle's unrounded SiTU-GLU on the GPU's z rows.

    Elementwise bound from the arithmetic: the store rounding (half an ulp:
    2^-9 |a| in bf16, 2^-24 |a| in fp32) plus fp32 dot-product and tanh/exp
    error, far below 1e-3 of the expert's RMS in bf16 and 1e-5 in fp32.  (A
    max-norm bound relative to the RMS does not fit this heavy-tailed tensor:
    half an ulp of an element above 10 RMS is already more than 2e-2 RMS.)
    """
    z = gpu["z"]
    # fp32: the W1/W2 contraction has L terms, whose rounding error grows like sqrt(L)
    rel, floor = (2.0 ** -8, 1e-3) if cfg.dtype == "bf16" else (1e-6, 1e-5 * max(1.0, (cfg.L / 1024.0) ** 0.5))

    def worst(got, a):
        rms = np.sqrt(np.mean(a ** 2))
        return float(np.max(np.abs(got - a) / (rel * np.abs(a) + floor * rms)))

    for e in range(cfg.n):
        lo, hi = gpu["offs"][e], gpu["offs"][e + 1]
        if lo == hi:
            continue
        toks = gpu["row_token"][lo:hi]
        a = ref.expert_hidden(z[toks], P.w1(e), P.w2(e), cfg.beta1, cfg.beta2, "f64", cfg.gate)
        r = worst(gpu["hidden"][lo:hi], a)
        assert r <= 1.0, f"expert {e}: error {r:.3g} x the bound"
    T = z.shape[0]
    for j in range(cfg.n_shared):  # shared expert j: rows T*k + j*T .. + T, one per token
        a = ref.expert_hidden(z, P.ws1(j), P.ws2(j), cfg.beta1, cfg.beta2, "f64", cfg.gate)
        r = worst(gpu["hidden"][T * cfg.k + j * T:T * cfg.k + (j + 1) * T], a)
        assert r <= 1.0, f"shared expert {j}: error {r:.3g} x the bound"
    assert np.all(np.abs(gpu["hidden"]) <= cfg.beta1 * cfg.beta2)


def test_c0_tiny_fp32_full_parity():
    cfg = synth.get_config("C0")
    gpu = run_gpu(cfg)
    P = synth.HostParams(cfg)
    x = P.x()
    check_against_oracle(cfg, gpu, x, P)
    check_dispatch(cfg, gpu)
    check_hidden(cfg, gpu, P, x)


def test_c0_qb_from_forward_scores():
    cfg = synth.get_config("C0")
    gpu = run_gpu(cfg)
    s = torch.from_numpy(gpu["s"].astype(np.float32)).cuda()
    hist = torch.empty((cfg.n, cfg.nbins), dtype=torch.int32, device="cuda")
    bias = torch.zeros(cfg.n, dtype=torch.float32, device="cuda")
    lmoe.qb_update(s, cfg.k, hist, bias)
    torch.cuda.synchronize()
    H, b = ref.qb_update(gpu["s"].astype(np.float32), cfg.nbins, cfg.k)
    assert np.array_equal(hist.cpu().numpy(), H)
    assert np.array_equal(bias.cpu().numpy().view(np.uint32), b.view(np.uint32))


def test_c1_small_bf16_full_parity():
    cfg = synth.get_config("C1")
    gpu = run_gpu(cfg)
    P = synth.HostParams(cfg, cache=True)
    x = P.x()
    check_against_oracle(cfg, gpu, x, P)
    check_dispatch(cfg, gpu)


@pytest.mark.parametrize("shape", [
    dict(T=1000, d=256, L=128, n=40, k=5, n_shared=0, D=128, dtype="bf16"),     # ragged T, ragged router N, no shared
    dict(T=333, d=512, L=256, n=200, k=7, n_shared=3, D=64, dtype="bf16"),      # ragged, three shared experts
    dict(T=257, d=256, L=128, n=64, k=64, n_shared=1, D=64, dtype="f32"),       # k = n = 64: every expert
    dict(T=1, d=128, L=64, n=1, k=1, n_shared=1, D=64, dtype="f32"),            # one token, one expert
    dict(T=130, d=384, L=192, n=1024, k=3, n_shared=2, D=192, dtype="bf16"),    # largest expert count
    dict(T=777, d=256, L=128, n=700, k=16, n_shared=2, D=64, dtype="bf16"),     # 512 < n <= 896: the K3 top-k kernel
    # latent widths that take each combine + RMSNorm layout: 4 and 8 chunks of
    # 8 elements per lane (one wavefront per token), then one work-group per token
    dict(T=70, d=4096, L=2048, n=16, k=2, n_shared=1, D=64, dtype="bf16"),
    dict(T=40, d=8192, L=4096, n=8, k=2, n_shared=1, D=64, dtype="f32"),
    dict(T=20, d=16384, L=8192, n=8, k=2, n_shared=1, D=64, dtype="bf16"),      # widest latent accepted
])
def test_ragged_and_edge_shapes(shape):
    cfg = synth.get_config("C0").with_(x_seed=21, w_seed=21, bias_std=0.05, **shape)
    gpu = run_gpu(cfg)
    P = synth.HostParams(cfg)
    x = P.x()
    check_against_oracle(cfg, gpu, x, P)
    check_dispatch(cfg, gpu)
    check_hidden(cfg, gpu, P, x)


@pytest.mark.parametrize("n,k", [(896, 16), (1024, 64), (200, 7), (40, 5)])
def test_topk_exact_ties_go_to_the_lower_index(n, k):
    """Exact ties in the top-k kernel that serves each expert count (896 is the
    K3 pool of "Kimi K3 Architecture Deep Dive" §3).  With W_r = 0 every logit
    is exactly 0 and every score exactly sigmoid(0) = 1/2, so (1) with zero bias
    every key ties and each token's list must be experts 0 .. k-1 in that order,
    with weights 1/k; (2) with the bias on a few exactly representable levels
    the list must be the stable order of (-b, e): the oracle's top-k of the
    same keys, order included; (3) with the router rows repeated (expert e uses
    row e mod 37) and a bias equal within each class, tokens differ but every
    list must still be a valid top-k that breaks ties by the lower index."""
    cfg = synth.get_config("C0").with_(T=300, d=256, L=128, n=n, k=k, n_shared=1, D=64, dtype="bf16",
                                       x_seed=61, w_seed=61)
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    wr = w["w_router"].clone()

    def route(bias):
        w["router_bias"] = torch.as_tensor(np.asarray(bias, dtype=np.float32)).to(dev)
        idx = torch.full((cfg.T, k), -1, dtype=torch.int32, device=dev)
        g = torch.empty((cfg.T, k), dtype=torch.float32, device=dev)
        s = torch.empty((cfg.T, n), dtype=torch.float32, device=dev)
        lmoe.forward(x, w, k, topk_idx=idx, topk_w=g, scores=s)
        torch.cuda.synchronize()
        return idx.cpu().numpy().astype(np.int64), g.cpu().numpy(), s.cpu().numpy()

    w["w_router"].zero_()
    idx, g, s = route(np.zeros(n))
    assert np.all(s == 0.5)
    assert np.array_equal(idx, np.broadcast_to(np.arange(k), (cfg.T, k)))
    assert np.allclose(g, 1.0 / k, rtol=1e-7, atol=0)
    assert check_topk_valid(s, np.zeros(n), idx) == (cfg.T if k < n else 0)

    b = np.random.default_rng(n).integers(0, 4, n) * 0.125
    idx, g, s = route(b)
    want, _ = ref.biased_topk(np.full((1, n), 0.5), b, k)
    assert np.array_equal(idx, np.broadcast_to(want[0], (cfg.T, k)))
    check_topk_valid(s, b, idx)

    w["w_router"].copy_(wr[torch.arange(n, device=dev) % 37])
    b = (np.arange(n) % 37 % 3) * 0.0625
    idx, g, s = route(b)
    check_topk_valid(s, b, idx)


def test_bias_shift_invariance_on_gpu():
    cfg = synth.get_config("C0").with_(T=300, bias_std=0.1)
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    y0 = lmoe.forward(x, w, cfg.k).clone()
    i0 = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    i1 = torch.empty_like(i0)
    lmoe.forward(x, w, cfg.k, topk_idx=i0)
    w2 = dict(w)
    w2["router_bias"] = w["router_bias"] + 0.25
    y1 = lmoe.forward(x, w2, cfg.k, topk_idx=i1)
    torch.cuda.synchronize()
    same = (i0 == i1).all(1)
    assert same.float().mean() > 0.95
    assert torch.allclose(y0[same], y1[same], rtol=0, atol=1e-6)


def test_nan_token_propagates_and_others_unaffected():
    cfg = synth.get_config("C0").with_(T=64)
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    y0 = lmoe.forward(x, w, cfg.k).clone()
    x[3, 5] = float("nan")
    y1 = lmoe.forward(x, w, cfg.k)
    torch.cuda.synchronize()
    assert torch.isnan(y1[3]).all()
    others = torch.ones(cfg.T, dtype=torch.bool)
    others[3] = False
    assert torch.equal(y0[others.cuda()], y1[others.cuda()])


def test_repeat_calls_are_deterministic():
    cfg = synth.get_config("C1").with_(T=512)
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    a = lmoe.forward(x, w, cfg.k).clone()
    b = lmoe.forward(x, w, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_empty_batch():
    cfg = synth.get_config("C0")
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev, with_x=False)
    x = torch.empty((0, cfg.d), dtype=torch.float32, device=dev)
    y = lmoe.forward(x, w, cfg.k)
    assert y.shape == (0, cfg.d)


def test_stale_workspace_counters_are_reset():
    """The grouped GEMMs hand out tiles beyond the first round from counters that
    live in the caller's workspace; every forward resets them, so a workspace
    holding stale bytes gives the same result as a zeroed one.  0x40 bytes make a
    counter that was not reset hand out no tile at all (so a regression shows as
    missing output, never as an out-of-range tile).  Eight routed experts, 20
    tokens and an 8192-wide latent put 288 expert W3 tiles on 256 work-groups, so
    the counters are used, and n < 16 covers counters past the expert count."""
    cfg = synth.get_config("C0").with_(x_seed=21, w_seed=21, bias_std=0.05, T=20, d=16384, L=8192, n=8, k=2,
                                       n_shared=1, D=64, dtype="bf16")
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    dims = lmoe.dims_of(x, w, cfg.k)
    ws0 = lmoe.make_workspace(dims, x.dtype, dev).zero_()
    y0 = lmoe.forward(x, w, cfg.k, workspace=ws0).clone()
    ws1 = lmoe.make_workspace(dims, x.dtype, dev).fill_(0x40)
    y1 = lmoe.forward(x, w, cfg.k, workspace=ws1).clone()
    y2 = lmoe.forward(x, w, cfg.k, workspace=ws1)  # the same workspace again
    torch.cuda.synchronize()
    assert torch.isfinite(y0.float()).all()
    assert torch.equal(y0, y1)
    assert torch.equal(y0, y2)


def test_concurrent_calls_from_two_host_threads():
    """Two host threads, each with its own stream and workspace, call the forward
    at the same time (the binding releases the interpreter lock during the call,
    and the library's once-per-device launch setup is thread-safe); every result
    equals a sequential forward bit for bit."""
    import threading
    cfg = synth.get_config("C1").with_(T=512)
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    ref_y = lmoe.forward(x, w, cfg.k).clone()
    torch.cuda.synchronize()
    dims = lmoe.dims_of(x, w, cfg.k)
    outs, errors = [], []

    def worker():
        try:
            s = torch.cuda.Stream(device=dev)
            ws = lmoe.make_workspace(dims, x.dtype, dev)
            ys = [torch.empty_like(x) for _ in range(3)]
            with torch.cuda.stream(s):
                for y in ys:
                    lmoe.forward(x, w, cfg.k, y=y, workspace=ws, stream=s.cuda_stream)
            s.synchronize()
            outs.extend(ys)
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker) for _ in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    assert len(outs) == 6
    for y in outs:
        assert torch.equal(y, ref_y)


def test_forward_replays_from_a_hip_graph():
    """The forward enqueues kernels only (no memsets, no host synchronisation), so
    it can be captured in a HIP graph: each of several replays, with eager work
    and synchronisations between them and a new input copied in before two of
    them, equals the eager forward of the same input bit for bit."""
    cfg = synth.get_config("C1").with_(T=512)
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    x2 = synth.params.device_x(cfg.with_(x_seed=7), dev)
    dims = lmoe.dims_of(x, w, cfg.k)
    ws = lmoe.make_workspace(dims, x.dtype, dev)
    xin, y = x.clone(), torch.empty_like(x)
    ref1 = lmoe.forward(x, w, cfg.k).clone()
    ref2 = lmoe.forward(x2, w, cfg.k).clone()
    lmoe.forward(xin, w, cfg.k, y=y, workspace=ws)  # first call on this device before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lmoe.forward(xin, w, cfg.k, y=y, workspace=ws)
    for i, (src, want) in enumerate([(x, ref1), (x2, ref2), (x2, ref2), (x, ref1)]):
        xin.copy_(src)
        lmoe.forward(x2, w, cfg.k)  # unrelated eager work on the same stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {i}"


def test_timed_forward_with_null_events_equals_forward():
    """lmoe_forward_timed with only some stage boundaries given (the rest NULL)
    computes what lmoe_forward computes, and the given events time their stage."""
    cfg = synth.get_config("C1").with_(T=512)
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    ref_y = lmoe.forward(x, w, cfg.k).clone()
    ev = [None] * (lmoe.N_STAGES + 1)
    i = lmoe.STAGES.index("experts_w12")
    ev[i], ev[i + 1] = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    y = lmoe.forward(x, w, cfg.k, stage_events=ev)
    torch.cuda.synchronize()
    assert torch.equal(y, ref_y)
    assert ev[i].elapsed_time(ev[i + 1]) > 0.0


def test_swiglu_ablation_full_parity():
    # both caps at +inf: the uncapped limit, every expert a SwiGLU ([DD] §1 compares
    # SiTU-GLU against it); same kernels, same parity bar
    cfg = synth.get_config("C1").with_(beta1=np.inf, beta2=np.inf)
    gpu = run_gpu(cfg)
    P = synth.HostParams(cfg, cache=True)
    x = P.x()
    check_against_oracle(cfg, gpu, x, P)
    check_dispatch(cfg, gpu)
    check_hidden(cfg, gpu, P, x)


def test_caps_bound_the_hidden_of_outlier_tokens():
    """Forward activation maxima on outlier tokens, capped against uncapped.

    One token in a hundred is scaled by 50 ([DD] §1: the caps exist for such
    tokens, whose SwiGLU gate grows like the square of the input).  With
    beta1 = 4, beta2 = 25 the gated hidden of those tokens saturates just below
    beta1 * beta2 = 100; without the caps the oracle puts the shared experts'
    maximum near 2.6e4 on this input, while the other tokens stay near 10
    either way.  Both runs are held to the parity bar first, the outlier rows
    apart from the rest (their elements are some 40 RMS of the whole batch, so
    half an ulp of bf16 there would exceed a bound relative to the batch RMS)."""
    base = synth.get_config("C1").with_(T=512, outlier_frac=0.01)
    rows = synth.outlier_rows(base)
    assert rows.size == 5
    rest = np.setdiff1d(np.arange(base.T), rows)
    peak = {}
    for b in (4.0, np.inf):
        cfg = base.with_(beta1=b, beta2=25.0 if b == 4.0 else np.inf)
        gpu = run_gpu(cfg)
        P = synth.HostParams(cfg)
        x = P.x()
        check_against_oracle(cfg, gpu, x[rows], P, rows=rows)
        check_against_oracle(cfg, gpu, x[rest], P, rows=rest)
        check_hidden(cfg, gpu, P, x)
        T = cfg.T
        shared = np.abs(gpu["hidden"][T * cfg.k:T * cfg.k + T * cfg.n_shared]).reshape(cfg.n_shared, T, -1)
        per_tok = shared.max(axis=(0, 2))
        others = np.delete(per_tok, rows)
        peak[b] = (per_tok[rows].max(), others.max())
    capped, free = peak[4.0], peak[np.inf]
    assert 90.0 < capped[0] <= 100.0
    assert free[0] > 1e4
    assert capped[1] < 20.0 and free[1] < 20.0


@pytest.mark.parametrize("shape", [
    dict(name="C1"),
    dict(name="C0", T=333, d=512, L=256, n=200, k=7, n_shared=3, D=64, dtype="bf16"),   # ragged, small experts
])
def test_hard_clip_ablation_full_parity(shape):
    # both caps a hard clip at beta1 = 4, beta2 = 25: the ablation the tanh softcap
    # is compared against ([DD] §1), in the same kernels, at the same parity bar
    shape = dict(shape)
    cfg = synth.get_config(shape.pop("name")).with_(gate="clip", x_seed=31, **shape)
    gpu = run_gpu(cfg)
    P = synth.HostParams(cfg)
    x = P.x()
    check_against_oracle(cfg, gpu, x, P)
    check_dispatch(cfg, gpu)
    check_hidden(cfg, gpu, P, x)


def test_hard_clip_collapses_outlier_hidden_to_the_ceiling():
    """On 1% x50 outlier tokens both caps hold the gated hidden to the same
    ceiling beta1 * beta2 = 100, but the hard clip maps every unit past both
    thresholds onto 100 * sigmoid(x1), i.e. onto the ceiling itself once
    stored in bf16, while the softcap keeps most of them below it (the pages:
    a clamp collapses every value past the threshold onto one number).  On
    this input the oracle puts 1459 of the outlier tokens' 5120 shared-expert
    units at exactly 100 with the clip and 208 with the softcap."""
    base = synth.get_config("C1").with_(T=512, outlier_frac=0.01)
    rows = synth.outlier_rows(base)
    T = base.T
    sat = {}
    for gate in ("tanh", "clip"):
        cfg = base.with_(gate=gate)
        gpu = run_gpu(cfg)
        P = synth.HostParams(cfg)
        x = P.x()
        check_against_oracle(cfg, gpu, x[rows], P, rows=rows)
        check_hidden(cfg, gpu, P, x)
        h = np.abs(gpu["hidden"][T * cfg.k:T * cfg.k + T * cfg.n_shared]).reshape(cfg.n_shared, T, -1)[:, rows]
        assert h.max() == 100.0
        sat[gate] = int((h == 100.0).sum())
    assert sat["clip"] > 3 * sat["tanh"]


@pytest.mark.parametrize("shape", [
    dict(name="C1"),
    dict(name="C0", T=20, d=16384, L=8192, n=8, k=2, n_shared=1, D=64, dtype="bf16"),  # one work-group per token
])
def test_no_norm_ablation_full_parity(shape):
    # the one retained RMSNorm dropped, v = u ([DD] §2 keeps only this norm): same
    # kernels, same parity bar, for both combine layouts
    shape = dict(shape)
    cfg = synth.get_config(shape.pop("name")).with_(norm="none", x_seed=41, **shape)
    gpu = run_gpu(cfg)
    P = synth.HostParams(cfg)
    x = P.x()
    check_against_oracle(cfg, gpu, x, P)
    check_dispatch(cfg, gpu)


@pytest.mark.parametrize("shape", [
    dict(name="C1"),
    dict(name="C0", T=1000, d=256, L=128, n=40, k=5, n_shared=0, D=128, dtype="bf16"),   # ragged, no shared
])
def test_extra_down_norm_ablation_full_parity(shape):
    # an RMSNorm on z after the down-projection, the one the layer leaves out
    # ([DD] §2), normed in place before routing: same parity bar; every stored
    # z row then has unit RMS up to its bf16 rounding
    shape = dict(shape)
    cfg = synth.get_config(shape.pop("name")).with_(norm="both", x_seed=51, **shape)
    gpu = run_gpu(cfg)
    P = synth.HostParams(cfg)
    x = P.x()
    check_against_oracle(cfg, gpu, x, P)
    check_dispatch(cfg, gpu)
    check_hidden(cfg, gpu, P, x)
    assert np.allclose(np.sqrt(np.mean(gpu["z"] ** 2, axis=1)), 1.0, rtol=1e-2)
