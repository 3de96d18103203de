"""Turn rocprofv3 CSV output of `bench.py` into the short text summaries kept
under profiles/.

  python -m sparse_moe_layer_down_amd.profsum trace  <kernel_stats.csv> <out.md> "<command>" ["<title>"]
  python -m sparse_moe_layer_down_amd.profsum counters <fetch_dir> <write_dir> <calib_fetch_dir> <calib_write_dir> <out.md> "<commands>" ["<title>"] [<kernel_stats.csv>]
  python -m sparse_moe_layer_down_amd.profsum mfma <pmc_dir> <out.md> "<command>" ["<title>"]
  python -m sparse_moe_layer_down_amd.profsum lds <pmc_dir> <out.md> "<command>" ["<title>"]

The counters summary records, for every kernel of the forward, the mean
FETCH_SIZE and WRITE_SIZE per dispatch (KiB, as the counters read), with a
kernel trace of the same workload also the achieved GB/s (scaled bytes over the
kernel's average duration in that trace), the same
counters for the 1 GiB device copy that `bench.py --only calib` runs in a
process of its own, the calibration factors they give, and a SHA-256 of the library's kernel sources.
`bench.py` reports the expert W1/W2 kernel's traffic from this file only while
that hash matches the sources it runs.
"""
import csv
import glob
import hashlib
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
COPY_BYTES = 1 << 30
EPI = {0: "store", 1: "sigmoid", 2: "SiTU-GLU", 3: "rowscale", 4: "split-K partial", 5: "clip-GLU",
       6: "gate backward", 7: "clip gate backward"}


def source_sha256():
    """SHA-256 over the kernel sources and the C header, in a fixed order."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*"))) + [os.path.join(ROOT, "include", "lmoe.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def label(name):
    """Readable name for a kernel symbol (mangled or demangled)."""
    m = re.search(r"gemm_kernelI(DF16b|f)(DF16b|DF16_|f)Li(\d+)ELi(\d+)ELi(\d)ELi(\d)ELi(\d)ELi(\d)ELb(\d)ELb(\d)E"
                  r"(?:Lb(\d)E)?(?:Lb(\d)E)?", name)
    if m:
        out = {"f": "fp32", "DF16b": "bf16", "DF16_": "fp16"}[m.group(2)]
        return (f"gemm {m.group(3)}x{m.group(4)} waves {m.group(5)}x{m.group(6)} pf{m.group(7)} "
                f"epi={EPI[int(m.group(8))]} out={out} gather={m.group(9)} grouped={m.group(10)}"
                + (" B[K,N]" if m.group(12) == "1" else ""))
    m = re.search(r"gemm_kernel<[^,]*, (\d+), (\d+), (\d), (\d), (\d), (\d), (\w+), (\w+)(?:, (\w+))?(?:, (\w+))?>",
                  name)
    if m:  # rocprofv3 demangles only the instances with a float output type
        return (f"gemm {m.group(1)}x{m.group(2)} waves {m.group(3)}x{m.group(4)} pf{m.group(5)} "
                f"epi={EPI[int(m.group(6))]} out=fp32 gather={int(m.group(7) == 'true')} "
                f"grouped={int(m.group(8) == 'true')}" + (" B[K,N]" if m.group(10) == "true" else ""))
    m = re.search(r"(\w+_kernel)", name)
    if not m:
        return name[:60]
    lab = re.sub(r"^_ZN4lmoe\d+", "", m.group(1))  # drop the mangled namespace prefix
    # the histogram's first template argument selects the margin form
    if lab == "qb_hist_kernel" and ("qb_hist_kernelILb1E" in name or "qb_hist_kernel<true" in name):
        return "qb_hist_kernel (margin)"
    return lab


def stage(lab, name):
    rules = [("SiTU-GLU out=bf16 gather=1 grouped=1", "expert W1/W2 + SiTU-GLU"),
             ("gate backward", "backward: gate (W1/W2 products recomputed)"),
             ("rowscale out=bf16 gather=1 grouped=1 B[K,N]", "backward: da (W3 read in place)"),
             ("grouped=1 B[K,N]", "backward: dz rows (W1, W2 read in place)"),
             ("rowscale", "expert W3 x row weight"),
             ("store out=bf16 gather=0 grouped=1", "backward: expert weight gradients (K-range)"),
             ("norm_bwd", "backward: RMSNorm backward, routing-weight gradients"),
             ("colsum", "backward: gain gradient"),
             ("router_bwd", "backward: router-logit gradients"),
             ("bwd_scan", "backward: expert segments"),
             ("transpose", "backward: transposes"),
             ("epi=sigmoid", "router scores"),
             ("store out=bf16 gather=0 grouped=0", "W_down / W_up"),
             ("split-K", "split-K partial sums"),
             ("splitk_finalize", "split-K finalize"),
             # the backward sums the dz rows with the combine kernel over bf16 rows (the
             # forward's staged rows are fp16)
             ("combine_rmsnorm_wave_kernelIDF16bDF16b", "backward: dz sum (the token's dz rows)"),
             ("combine", "combine + RMSNorm"),
             ("topk", "top-k + routing weights"),
             ("perm_", "permutation"),
             ("(margin)", "QB margin form: histogram"),
             ("qb_thresholds", "QB margin form: token thresholds"),
             ("qb_margin_solve", "QB margin form: bias solve"),
             ("signsgd", "fixed-step (SignSGD) bias update"),
             ("qb_hist", "QB histogram"),
             ("qb_merge_pool", "QB histogram: the runs' counts merged, pooled sum"),
             ("qb_merge", "QB histogram: the runs' counts merged"),
             ("qb_pool", "QB pooled histogram"),
             ("qb_solve", "QB bias solve"),
             ("synth", "input synthesis (outside the timed region)")]
    for key, st in rules:
        if key in lab or key in name:
            return st
    return ""


PREFILL = "K3-shaped prefill forward (T=8192, d=7168, 896 experts choose 16), bf16"


def trace(stats_csv, out, cmd, title=PREFILL):
    rows = list(csv.DictReader(open(stats_csv)))
    with open(out, "w") as f:
        f.write(f"# Kernel trace: {title}\n\n")
        f.write(f"Kernel-source SHA-256: `{source_sha256()}`\n\n")
        f.write(f"Command (from the repository root, one MI355X):\n\n```\n{cmd}\n```\n\n")
        f.write("| kernel | stage | calls | avg (us) | min (us) | max (us) | share |\n|---|---|---|---|---|---|---|\n")
        for r in rows:
            lab = label(r["Name"])
            f.write(f"| `{lab}` | {stage(lab, r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                    f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |\n")


def _means(d, counter, by_grid=False):
    """Mean value of `counter` per kernel (per (kernel, grid size) with by_grid) and dispatch counts."""
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                key = (r["Kernel_Name"], int(r.get("Grid_Size") or 0)) if by_grid else r["Kernel_Name"]
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def _durations(stats_csv):
    """Average duration (s) per kernel label from a rocprofv3 kernel_stats.csv."""
    if not stats_csv:
        return {}
    return {label(r["Name"]): float(r["AverageNs"]) * 1e-9 for r in csv.DictReader(open(stats_csv))}


def _grid_durations(stats_csv):
    """Average duration (s) per (kernel name, grid size) from the kernel_trace.csv
    written beside a kernel_stats.csv (empty if there is none)."""
    if not stats_csv or not stats_csv.endswith("_kernel_stats.csv"):
        return {}
    trace = stats_csv[: -len("_kernel_stats.csv")] + "_kernel_trace.csv"
    if not os.path.exists(trace):
        return {}
    acc = {}
    for r in csv.DictReader(open(trace)):
        key = (r["Kernel_Name"], int(r.get("Grid_Size_X") or 0) * int(r.get("Grid_Size_Y") or 1) *
               int(r.get("Grid_Size_Z") or 1))
        acc.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    return {k: sum(v) / len(v) for k, v in acc.items()}


def calibration(calib_fetch, calib_write):
    """KiB the counters read for the 1 GiB device copy of `bench.py --only calib`
    (run alone in its own profiled process, so every copy dispatch there is that
    copy): (fetch KiB, write KiB), summed over its dispatches."""
    fetch, nf = _means(calib_fetch, "FETCH_SIZE")
    write, nw = _means(calib_write, "WRITE_SIZE")
    cf = sum(v * nf[k] for k, v in fetch.items() if "copyBuffer" in k)
    cw = sum(v * nw[k] for k, v in write.items() if "copyBuffer" in k)
    if cf <= 0 or cw <= 0:
        raise SystemExit("no device copy in the calibration runs")
    return cf, cw


def counters(fetch_dir, write_dir, out, cmd, title=PREFILL, stats_csv=None, calib_fetch=None, calib_write=None):
    """Counter summary of one workload.  The calibration copy comes from its own
    profiled runs (calib_fetch / calib_write directories).  Rows are per
    (kernel, grid size), so launches of one kernel with different grids (e.g.
    the QB histogram at 1000 and at 10000 bins) stay apart."""
    dur = _durations(stats_csv)
    gdur = _grid_durations(stats_csv)
    fetch, nf = _means(fetch_dir, "FETCH_SIZE", by_grid=True)
    write, _ = _means(write_dir, "WRITE_SIZE", by_grid=True)
    cf, cw = calibration(calib_fetch, calib_write)
    ff = COPY_BYTES / (cf * 1024.0)
    wf = COPY_BYTES / (cw * 1024.0)
    with open(out, "w") as f:
        f.write(f"# HBM counters per dispatch: {title}\n\n")
        f.write(f"source_sha256: {source_sha256()}\n")
        f.write(f"fetch_factor: {ff:.4f}\nwrite_factor: {wf:.4f}\n\n")
        f.write("FETCH_SIZE and WRITE_SIZE are in KiB per dispatch as rocprofv3 reports them. The factors scale them to "
                f"bytes moved: a 1 GiB device-to-device copy, profiled alone in its own process, read {cf:.0f} KiB "
                f"(FETCH_SIZE) and wrote {cw:.0f} KiB (WRITE_SIZE), summed over its dispatches.\n\n")
        f.write(f"Commands (from the repository root, one MI355X):\n\n```\n{cmd}\n```\n\n")
        if dur:
            f.write("GB/s = scaled traffic over the kernel's average duration in the kernel trace of the same "
                    "workload (a separate run of the same command without counters), per launch grid where the "
                    "trace's dispatch list gives one.\n\n")
        f.write("| kernel | stage | grid | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled traffic (GB) | GB/s |\n"
                "|---|---|---|---|---|---|---|---|\n")
        for key in sorted(fetch, key=lambda k: -fetch[k]):
            k, grid = key
            lab = label(k)
            st = "device copy" if "copyBuffer" in k else stage(lab, k)
            if st.startswith("input synthesis"):
                continue
            w = write.get(key, 0.0)
            gb = (fetch[key] * ff + w * wf) * 1024 / 1e9
            tag = "experts_w12: " if st == "expert W1/W2 + SiTU-GLU" else ""
            t = gdur.get((k, grid)) or dur.get(lab)
            rate = f"{gb / t:.0f}" if t and "copyBuffer" not in k else ""
            f.write(f"| `{lab}` | {tag}{st} | {grid} | {nf[key]} | {fetch[key]:.0f} | {w:.0f} | {gb:.3f} | {rate} |\n")
        rw = [key for key in fetch if stage(label(key[0]), key[0]) == "expert W1/W2 + SiTU-GLU"]
        if len(rw) == 1:
            key = rw[0]
            tb = (fetch[key] * ff + write.get(key, 0.0) * wf) * 1024
            f.write(f"\nexperts_w12_traffic_bytes: {tb:.0f}\n")


def mfma(pmc_dir, out, cmd, title=PREFILL, cus=256, simds=4, xcds=8):
    """MFMA utilisation per kernel from SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs),
    SQ_INSTS_VALU_MFMA_MOPS_BF16 (units of 512 flops) and GRBM_GUI_ACTIVE (GPU clocks,
    summed over the XCDs)."""
    busy, _ = _means(pmc_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    mops, n = _means(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    gui, _ = _means(pmc_dir, "GRBM_GUI_ACTIVE")
    with open(out, "w") as f:
        f.write(f"# MFMA utilisation per dispatch: {title}\n\n")
        f.write("busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d XCDs x %d CUs x %d SIMDs): the share of "
                "SIMD cycles with the matrix core busy while the kernel ran. bf16 MFMA flops = "
                "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, including MFMAs on padding rows.\n\n" % (xcds, cus, simds))
        f.write(f"Command (from the repository root, one MI355X):\n\n```\n{cmd}\n```\n\n")
        f.write("| kernel | stage | dispatches | GPU clocks | MFMA busy | bf16 MFMA GFLOP |\n|---|---|---|---|---|---|\n")
        for k in sorted(busy, key=lambda k: -busy[k]):
            if busy[k] <= 0:
                continue
            lab = label(k)
            clocks = gui.get(k, 0.0) / xcds
            frac = busy[k] / (clocks * cus * simds) if clocks else 0.0
            f.write(f"| `{lab}` | {stage(lab, k)} | {n.get(k, 0)} | {clocks:.0f} | {100 * frac:.1f}% | "
                    f"{mops.get(k, 0.0) * 512 / 1e9:.1f} |\n")


def lds(pmc_dir, out, cmd, title=PREFILL, cus=256, xcds=8):
    """LDS traffic per kernel: SQ_INSTS_LDS_LOAD_BANDWIDTH and _STORE_BANDWIDTH count
    64-byte units (checked against the expert W1/W2 kernel's fragment reads, 160 KB per
    K step and CU); bytes per clock and CU over GRBM_GUI_ACTIVE / XCDs; bank-conflict
    cycles as a share of SQ_LDS_IDX_ACTIVE; SQ_WAIT_INST_LDS as a share of
    SQ_WAVE_CYCLES."""
    c = {k: _means(pmc_dir, k)[0] for k in ("SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_INSTS_LDS_STORE_BANDWIDTH",
                                            "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS",
                                            "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")}
    n = _means(pmc_dir, "GRBM_GUI_ACTIVE")[1]
    ld, st = c["SQ_INSTS_LDS_LOAD_BANDWIDTH"], c["SQ_INSTS_LDS_STORE_BANDWIDTH"]
    with open(out, "w") as f:
        f.write(f"# LDS traffic per dispatch: {title}\n\n")
        f.write("LDS read / written GB = SQ_INSTS_LDS_LOAD_BANDWIDTH / _STORE_BANDWIDTH x 64 B; B/clk/CU = both over "
                "GRBM_GUI_ACTIVE / %d XCDs x %d CUs; bank conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; "
                "LDS issue wait = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES. Operands written by the global-load-to-LDS "
                "instruction are not LDS instructions: they appear in neither bandwidth counter (the written column "
                "then holds only LDS stores such as epilogue staging).\n\n" % (xcds, cus))
        f.write(f"Command (from the repository root, one MI355X):\n\n```\n{cmd}\n```\n\n")
        f.write("| kernel | stage | dispatches | LDS read (GB) | LDS written (GB) | B/clk/CU | bank conflicts | "
                "LDS issue wait |\n|---|---|---|---|---|---|---|---|\n")
        for k in sorted(ld, key=lambda k: -(ld[k] + st.get(k, 0.0))):
            tot = ld[k] + st.get(k, 0.0)
            if tot <= 0:
                continue
            lab = label(k)
            clocks = c["GRBM_GUI_ACTIVE"].get(k, 0.0) / xcds
            bpc = tot * 64 / (clocks * cus) if clocks else 0.0
            act = c["SQ_LDS_IDX_ACTIVE"].get(k, 0.0)
            bank = c["SQ_LDS_BANK_CONFLICT"].get(k, 0.0) / act if act else 0.0
            wc = c["SQ_WAVE_CYCLES"].get(k, 0.0)
            wait = c["SQ_WAIT_INST_LDS"].get(k, 0.0) / wc if wc else 0.0
            f.write(f"| `{lab}` | {stage(lab, k)} | {n.get(k, 0)} | {ld[k] * 64 / 1e9:.2f} | "
                    f"{st.get(k, 0.0) * 64 / 1e9:.2f} | {bpc:.1f} | {100 * bank:.1f}% | {100 * wait:.1f}% |\n")


def read_counters(path):
    """(traffic bytes of the expert W1/W2 launch, recorded source hash) or (None, None)."""
    if not os.path.exists(path):
        return None, None
    sha, tb = None, None
    for line in open(path):
        if line.startswith("source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif line.startswith("experts_w12_traffic_bytes:"):
            tb = float(line.split(":", 1)[1])
    return tb, sha


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "trace":
        trace(*sys.argv[2:6])
    elif len(sys.argv) >= 6 and sys.argv[1] == "counters":
        # counters <fetch_dir> <write_dir> <calib_fetch_dir> <calib_write_dir> <out.md> "<cmd>" ["<title>"] [<stats.csv>]
        a = sys.argv[2:]
        counters(a[0], a[1], a[4], a[5], *(a[6:8]), calib_fetch=a[2], calib_write=a[3])
    elif len(sys.argv) >= 5 and sys.argv[1] == "mfma":
        mfma(*sys.argv[2:6])
    elif len(sys.argv) >= 5 and sys.argv[1] == "lds":
        lds(*sys.argv[2:6])
    else:
        print(__doc__)
        sys.exit(2)
