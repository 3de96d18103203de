"""Throughput of the Stable LatentMoE forward on one MI355X.

One step = one lmoe_forward over one batch of the K3-shaped prefill workload
(T=8192 tokens, d=7168, latent 3584, 896 routed experts choose 16, 2 shared,
expert hidden 512, bf16, every weight resident in HBM), seeded synthetic
inputs already in device memory.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config C2] [--no-cpu-baseline] [--only all|prefill|backward|decode|qb|calib]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=512)
    ap.add_argument("--only", choices=("all", "prefill", "backward", "decode", "qb", "calib"), default="all",
                    help="run one part alone (for profiler runs of one workload): the timed prefill forwards, "
                         "the decode forwards, the Quantile Balancing protocol, or 'calib': a single 1 GiB "
                         "device-to-device copy (a plain copy of known size, whose memory counters calibrate "
                         "the byte counters of the other profiler runs), nothing else")
    return ap.parse_args()


def experts_w12_bytes(cfg, counts):
    """Algorithmic HBM bytes of the W1/W2 + SiTU-GLU grouped GEMM (routed and shared experts)
    for one launch: each touched routed expert's and each shared expert's W1 and W2 once, the
    latent z of every token once, the gated hidden of every expert row written once.  (Re-reads
    of a token's latent by its other experts are not algorithmic: they are what the kernel
    should serve from the caches.)"""
    es = 2 if cfg.dtype == "bf16" else 4
    touched = int((counts > 0).sum())
    rows = int(counts.sum()) + cfg.n_shared * cfg.T
    return (touched + cfg.n_shared) * 2 * cfg.D * cfg.L * es + cfg.T * cfg.L * es + rows * cfg.D * es, touched


def qb_protocol(w, dev, lmoe, synth):
    """Skewed-routing workload (K3 shapes, T=32768, Zipf(1.1) logit skew, same weights as the
    prefill workload): forward -> expert loads -> bias update -> next step's bias, for 20 steps;
    loads at step 0 (bias 0) and step 20 (bias from step 19, fresh batch), and the max/mean load
    of every step.  Bias updates compared on the same batches: Quantile Balancing
    (lmoe_qb_update: 1000-bin histograms, bias solve for share k/n; and with 10000 bins, which
    the pages find no better than 1000), its margin form (lmoe_qb_margin_update: the scores read
    against each token's top-k threshold) and the K2-style fixed step it replaces
    (lmoe_bias_signsgd, steps 1e-3, 1e-2 and 1e-1: the pages give no step size).  Each update
    launch is timed with events."""
    import torch
    cfg = synth.get_config("C4")
    w = dict(w)
    w["router_logit_offset"] = torch.as_tensor(synth.zipf_logit_offset(cfg)).to(dev)
    x = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=dev)
    dims = lmoe.dims_of(x, w, cfg.k)
    ws = lmoe.make_workspace(dims, x.dtype, dev)
    y = torch.empty_like(x)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    s = torch.empty((cfg.T, cfg.n), dtype=torch.float32, device=dev)

    fwd_ms = []  # every forward of the protocol, timed alone with events

    def run(method, nbins=cfg.nbins, step=0.0):
        bias = torch.zeros(cfg.n, dtype=torch.float32, device=dev)
        w["router_bias"] = bias
        hist = torch.empty((cfg.n, nbins), dtype=torch.int32, device=dev)
        qws = torch.empty(lmoe.qb_workspace_size(cfg.n, nbins), dtype=torch.uint8, device=dev)
        mws = torch.empty(lmoe.qb_margin_workspace_size(cfg.T, cfg.n, nbins), dtype=torch.uint8, device=dev)
        traj, mins, upd_ms = [], [], []
        for t in range(cfg.qb_steps + 1):
            x.copy_(synth.params.device_x(cfg, dev, step=t))
            f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            f0.record()
            lmoe.forward(x, w, cfg.k, y=y, topk_idx=idx, scores=s, workspace=ws, beta1=cfg.beta1,
                         beta2=cfg.beta2, eps=cfg.eps)
            f1.record()
            torch.cuda.synchronize()
            fwd_ms.append((method, nbins, t, f0.elapsed_time(f1)))
            load = torch.bincount(idx.flatten().long(), minlength=cfg.n).double()
            m = load.mean()
            traj.append(float(load.max() / m))
            mins.append(float(load.min() / m))
            if t < cfg.qb_steps:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                if method == "qb":
                    lmoe.qb_update(s, cfg.k, hist, bias, accumulate=False, solve=True, workspace=qws)
                elif method == "margin":
                    lmoe.qb_margin_update(s, cfg.k, hist, bias, workspace=mws)
                else:
                    lmoe.bias_signsgd(idx, cfg.n, step, bias)
                e1.record()
                torch.cuda.synchronize()
                upd_ms.append(e0.elapsed_time(e1))
        last = cfg.qb_steps
        return {"load_max_over_mean": {"step0_bias0": traj[0], f"step{last}": traj[last]},
                "load_min_over_mean": {"step0_bias0": mins[0], f"step{last}": mins[last]},
                "max_over_mean_by_step": [round(v, 4) for v in traj],
                "update_ms_median": float(sorted(upd_ms)[len(upd_ms) // 2])}

    out = {"workload": f"C4: T={cfg.T}, K3 shapes, Zipf({cfg.zipf_s}) logit skew alpha={cfg.zipf_alpha}",
           "steps": cfg.qb_steps, "nbins": cfg.nbins}
    out.update(run("qb"))
    out["qb_update_ms_median"] = out["update_ms_median"]
    out["qb_scores_read_GBps"] = cfg.T * cfg.n * 4 / (out["qb_update_ms_median"] * 1e-3) / 1e9
    out["bins_10000"] = run("qb", nbins=10000)
    out["margin"] = run("margin")
    out["signsgd"] = {f"step_{st:g}": run("signsgd", step=st) for st in (1e-3, 1e-2, 1e-1)}
    # the C4 forward itself (T = 32768 tokens): at step 0 (bias 0, the skewed routing) and once
    # Quantile Balancing (1000 bins) has set the bias (steps 1-20)
    def med(v):
        v = sorted(v)
        return float(v[len(v) // 2])

    flops = cfg.flops_per_token() * cfg.T
    out["forward"] = {}
    for key, sel in (("skewed_step0", [m for (_, _, t, m) in fwd_ms if t == 0]),
                     ("qb_balanced", [m for (me, nb, t, m) in fwd_ms if me == "qb" and nb == cfg.nbins and t > 0])):
        fm = med(sel)
        out["forward"][key] = {"ms_median": fm, "forwards": len(sel), "tokens_per_s": cfg.T / (fm * 1e-3),
                               "tflops": flops / (fm * 1e-3) / 1e12,
                               "mfma_peak_frac": flops / (fm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    return out


def decode_protocol(w, dev, lmoe, synth, steps):
    """Decode-shaped forward (K3 shapes, T=64 tokens, the prefill workload's weights, which are
    already resident): weight-read bound.  A 512 MB buffer is written between forwards so that
    the 256 MB MALL cannot keep the dense weights (131 MB) from one forward to the next; each
    forward is timed alone with events on the library's stream.  Algorithmic bytes: each touched
    routed expert's W1, W2, W3 once, the shared experts, W_down, W_up and W_router once, x and y."""
    import numpy as np
    import torch
    cfg = synth.get_config("C3")
    x = synth.params.device_x(cfg, dev)
    dims = lmoe.dims_of(x, w, cfg.k)
    ws = lmoe.make_workspace(dims, x.dtype, dev)
    y = torch.empty_like(x)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def fwd():
        lmoe.forward(x, w, cfg.k, y=y, workspace=ws, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps)

    for _ in range(3):
        flush.fill_(1)
        fwd()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fwd()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    counts = lmoe.workspace_view(ws, dims, x.dtype, "counts").cpu().numpy()
    touched = int((counts > 0).sum())
    es = 2
    expert_bytes = 3 * cfg.D * cfg.L * es
    dense_bytes = (2 * cfg.d * cfg.L + cfg.n * cfg.L) * es
    nbytes = (touched + cfg.n_shared) * expert_bytes + dense_bytes + 2 * cfg.T * cfg.d * es
    gbs = nbytes / (ms * 1e-3) / 1e9
    del flush, ws
    torch.cuda.empty_cache()
    return {"workload": f"C3: K3-shaped decode forward, T={cfg.T}, prefill weights",
            "ms_per_forward_median": ms, "tokens_per_s": cfg.T / (ms * 1e-3), "steps": steps,
            "experts_touched": touched, "algorithmic_bytes": nbytes, "achieved_GBps": gbs,
            "hbm_peak_frac": gbs / PEAK_HBM_GBS,
            "cache_state": "512 MB written between forwards (MALL and L2 hold no weights at the start)"}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, n_tok):
    """Time the oracle (as it stands) on bounded samples of each workload, on the host cores.

    Headline: the first n_tok tokens of the prefill workload.  Beside it: the tiny fp32
    workload in full, the first 512 tokens of the small bf16 one, the decode workload in full,
    and for the skewed workload the router + Quantile Balancing path (down-projection, scores,
    histogram, bias solve) on the first 256 tokens of each of its 21 batches plus one forward
    of 64 tokens.  Weight synthesis is done before each timed call (the oracle regenerates
    expert weights on demand; the cache holds them)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import synth
    from oracle import ref
    cache = {}
    per = {}

    def fwd(c, rows, step=None, P=None, synthesise=True):
        P = P or synth.HostParams(c, cache=cache)
        x = P.x_rows(rows, step=step)
        if synthesise:  # untimed: generate the weights the sample touches into the cache
            ref.forward(x, P, c.k, c.n_shared, c.dtype, c.beta1, c.beta2, c.eps)
        t0 = time.perf_counter()
        ref.forward(x, P, c.k, c.n_shared, c.dtype, c.beta1, c.beta2, c.eps)
        dt = time.perf_counter() - t0
        return {"tokens_per_s": len(rows) / dt, "gflops": len(rows) * c.flops_per_token() / dt / 1e9,
                "seconds": dt}

    main_cfg = cfg
    head = fwd(main_cfg, np.arange(n_tok))
    for name, ntok in (("C0", None), ("C1", 512), ("C3", None)):
        c = synth.get_config(name)
        # the decode workload shares the prefill weights, already synthesised above
        r = fwd(c, np.arange(c.T if ntok is None else ntok), synthesise=name != "C3")
        r["sample"] = f"{'all' if ntok is None else 'first ' + str(ntok)} of {c.T} tokens, full forward"
        per[name] = r
    c4 = synth.get_config("C4")
    P4 = synth.HostParams(c4, cache=cache)
    w_down, w_r, off = P4.w_down(), P4.w_router(), P4.logit_offset()
    rows = np.arange(256)
    xs = [P4.x_rows(rows, step=t) for t in range(c4.qb_steps + 1)]
    t0 = time.perf_counter()
    bias = np.zeros(c4.n, np.float32)
    for x in xs:
        z = ref.round_to(x @ w_down.T, c4.dtype)
        s = ref.router_scores(z, w_r, off)
        _, bias = ref.qb_update(s.astype(np.float32), c4.nbins, c4.k, bias=bias)
    dt = time.perf_counter() - t0
    r4 = fwd(c4, np.arange(64), step=0, P=P4, synthesise=False)
    per["C4"] = {"router_qb_tokens_per_s": len(xs) * rows.size / dt, "router_qb_seconds": dt,
                 "forward": r4,
                 "sample": f"router + QB on the first {rows.size} tokens of each of the {len(xs)} batches; "
                           "full forward of the first 64 tokens of batch 0"}
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": head["tokens_per_s"], "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_tok} tokens of the {main_cfg.name} workload (T={main_cfg.T}), NumPy fp64 oracle, "
                      f"weight synthesis excluded; {head['seconds']:.2f} s",
            "cpu_model": _cpu_model(), "gflops": head["gflops"], "per_config": per}


def other_configs(lmoe, synth, dev, steps=50):
    """GPU time of the tiny fp32 and the small bf16 workloads (whole forward, events on the
    library's stream, median of `steps` forwards after warm-up)."""
    import numpy as np
    import torch
    out = {}
    for name in ("C0", "C1"):
        c = synth.get_config(name)
        w = synth.device_params(c, device=dev)
        x = w.pop("x")
        ws = lmoe.make_workspace(lmoe.dims_of(x, w, c.k), x.dtype, dev)
        y = torch.empty_like(x)
        for _ in range(5):
            lmoe.forward(x, w, c.k, y=y, workspace=ws)
        times = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lmoe.forward(x, w, c.k, y=y, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        out[name] = {"T": c.T, "dtype": c.dtype, "ms_per_forward_median": ms, "tokens_per_s": c.T / (ms * 1e-3),
                     "tflops": c.flops_per_token() * c.T / (ms * 1e-3) / 1e12}
        del w, x, ws, y
    torch.cuda.empty_cache()
    return out


def measured_ceilings(dev):
    """Ceilings measured on this GPU beside the datasheet peaks: a 1 GiB device-to-device copy
    (torch's copy kernel; read + write bytes over its time) and the vendor library's bf16 GEMM
    (torch.matmul, 8192 x 7168 x 3584, B stored [N, K] as the layer's weights)."""
    import numpy as np
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ts = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    copy_gbs = 2 * (1 << 30) / (float(np.median(ts)) * 1e-3) / 1e9
    del src, dst
    a = torch.randn(8192, 3584, device=dev).to(torch.bfloat16)
    b = torch.randn(7168, 3584, device=dev).to(torch.bfloat16)
    for _ in range(3):
        a @ b.t()
    ts = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        a @ b.t()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    gemm_tf = 2 * 8192 * 7168 * 3584 / (float(np.median(ts)) * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"copy_1GiB_GBps": copy_gbs, "vendor_bf16_gemm_8192x7168x3584_TFLOPs": gemm_tf}


def profile_avg_ms(cfg_name):
    """Average duration (ms) of the expert W1/W2 kernel in the committed kernel-trace summary
    of this workload, if that summary was taken on the sources being run; else None."""
    from sparse_moe_layer_down_amd import profsum
    path = os.path.join(ROOT, "profiles", f"{cfg_name.lower()}_prefill_kernel_trace.md")
    if not os.path.exists(path):
        return None
    sha, avg = None, None
    for line in open(path):
        if line.startswith("Kernel-source SHA-256:"):
            sha = line.split("`")[1]
        elif "expert W1/W2 + SiTU-GLU" in line and avg is None:
            avg = float(line.split("|")[4]) / 1e3
    return avg if sha == profsum.source_sha256() else None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's expert bank is "
              "resident on a single MI355X and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import sparse_moe_layer_down_amd as lmoe
    import synth

    dev = torch.device("cuda:0")
    if args.only == "calib":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": 1 << 30}))
        return

    cfg = synth.get_config(args.config)
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    dims = lmoe.dims_of(x, w, cfg.k)
    ws = lmoe.make_workspace(dims, x.dtype, dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    out = {}
    if args.only in ("all", "prefill"):
        out = prefill(args, cfg, w, x, y, ws, dims, stream, lmoe, np, torch)
    if args.only in ("all", "backward"):
        out["backward"] = backward_protocol(cfg, w, x, ws, dims, lmoe, synth, torch, stream, steps=5)
    if args.only in ("all", "decode") and cfg.name == "C2":
        out["decode"] = decode_protocol(w, dev, lmoe, synth, steps=20)
    if args.only in ("all", "qb") and cfg.name == "C2":
        del ws
        torch.cuda.empty_cache()
        out["qb_protocol"] = qb_protocol(w, dev, lmoe, synth)
    if args.only == "all":
        del w, x, y
        torch.cuda.empty_cache()
        out["other_configs"] = other_configs(lmoe, synth, dev)
        out["measured_ceilings"] = measured_ceilings(dev)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample_tokens)
    print(json.dumps(out))


def backward_protocol(cfg, w, x, ws, dims, lmoe, synth, torch, stream, steps):
    """Timed backward passes (lmoe_backward) of the headline workload for a seeded
    synthetic upstream gradient, after one forward that leaves the routing and
    the forward workspace in place.  FLOPs: twice the forward's (each product
    has a data and a weight gradient) plus the W1/W2 gate products recomputed
    from the stored latent rather than kept from the forward."""
    T = x.shape[0]
    dev = x.device
    dy = torch.empty_like(x)
    synth.device_fill(dy, cfg.x_seed, synth.TID["dy"], 0, 1.0)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    s = torch.empty((T, cfg.n), dtype=torch.float32, device=dev)
    kw = dict(beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps)
    lmoe.forward(x, w, cfg.k, topk_idx=idx, topk_w=tw, scores=s, workspace=ws, **kw)
    bws = torch.empty(lmoe.backward_workspace_size(dims, x.dtype), dtype=torch.uint8, device=dev)
    grads = lmoe.backward(x, dy, w, cfg.k, idx, tw, s, ws, workspace=bws, **kw)
    for _ in range(2):
        lmoe.backward(x, dy, w, cfg.k, idx, tw, s, ws, grads=grads, workspace=bws, **kw)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        lmoe.backward(x, dy, w, cfg.k, idx, tw, s, ws, grads=grads, workspace=bws, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2 * cfg.flops_per_token() * T
    recompute = (cfg.k + cfg.n_shared) * 2 * 2 * cfg.L * cfg.D * T
    out = {"ms": ms, "tokens_per_s": T / (ms * 1e-3), "steps": steps, "tflops": flops / (ms * 1e-3) / 1e12,
           "mfma_peak_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "tflops_with_recompute": (flops + recompute) / (ms * 1e-3) / 1e12,
           "workspace_bytes": bws.numel()}
    del grads, bws
    torch.cuda.empty_cache()
    return out


def prefill(args, cfg, w, x, y, ws, dims, stream, lmoe, np, torch):
    """The timed forwards of the headline workload and the roofline of its dominant kernel."""
    def step(ev=None):
        lmoe.forward(x, w, cfg.k, y=y, workspace=ws, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps,
                     stage_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K forwards, each recording HIP events on the library's stream around the
    # dominant kernel (expert W1/W2 + SiTU-GLU) only, so its roofline duration is measured in
    # these same forwards at the cost of two event records per forward
    w12 = lmoe.STAGES.index("experts_w12")

    def w12_events():
        ev = [None] * (lmoe.N_STAGES + 1)
        ev[w12], ev[w12 + 1] = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        return ev

    evs = [w12_events() for _ in range(args.steps)]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    w12_ms = float(np.mean([ev[w12].elapsed_time(ev[w12 + 1]) for ev in evs]))

    # per-stage breakdown (reported, not used for the roofline): K more forwards with events at
    # every stage boundary
    stage_ms = np.zeros(lmoe.N_STAGES)
    for _ in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(lmoe.N_STAGES + 1)]
        step(ev)
        torch.cuda.synchronize()
        stage_ms += np.array([ev[j].elapsed_time(ev[j + 1]) for j in range(lmoe.N_STAGES)])
    stage_ms /= args.steps

    counts = lmoe.workspace_view(ws, dims, x.dtype, "counts").cpu().numpy()
    # HBM traffic of the W1/W2 launch from the committed rocprofv3 counter summary, if it was
    # taken on these exact kernel sources and this workload
    from sparse_moe_layer_down_amd import profsum
    tb, sha = profsum.read_counters(os.path.join(ROOT, "profiles", f"experts_w12_{cfg.name.lower()}_hbm_counters.md"))
    traffic = tb if (tb is not None and sha == profsum.source_sha256()) else None
    flops = cfg.flops_per_token() * cfg.T
    tflops = flops / (ms * 1e-3) / 1e12
    w12_bytes, touched = experts_w12_bytes(cfg, counts)
    achieved = w12_bytes / (w12_ms * 1e-3) / 1e9
    return {
        "metric": "LatentMoE fwd tokens/s + % bf16 MFMA peak (d=7168, 896c16) on 1 MI355X",
        "value": cfg.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded SplitMix64/Irwin-Hall normal inputs and weights, generated in HBM)",
        "config": {"workload": f"{cfg.name}: K3-shaped LatentMoE prefill forward" if cfg.name == "C2" else cfg.name,
                   "T": cfg.T, "d": cfg.d, "latent": cfg.L, "experts": cfg.n, "top_k": cfg.k,
                   "shared": cfg.n_shared, "expert_hidden": cfg.D},
        "tflops": tflops,
        "mfma_peak_frac": tflops / PEAK_BF16_TFLOPS,
        "stage_ms": {name: float(v) for name, v in zip(lmoe.STAGES, stage_ms)},
        "roofline": {"kernel": "expert W1/W2 + SiTU-GLU grouped GEMM (routed + shared)", "bound": "hbm",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic,
                     "traffic_over_algorithmic": None if traffic is None else traffic / w12_bytes,
                     "algorithmic_bytes": w12_bytes, "experts_touched": touched, "avg_ms": w12_ms,
                     "profile_avg_ms": profile_avg_ms(cfg.name)},
    }


if __name__ == "__main__":
    main()
