"""Host logic behind the bench's roofline traffic: the profile-summary tool's
kernel labels, the copy-calibrated scaling of the HBM byte counters, and the
source hash that decides whether a committed counter summary still applies."""
import csv

from sparse_moe_layer_down_amd import profsum

W12 = "_ZN4lmoe11gemm_kernelIDF16bDF16bLi192ELi256ELi2ELi4ELi2ELi2ELb1ELb1EEEvNS_8GemmArgsE"
W3 = "_ZN4lmoe11gemm_kernelIDF16bDF16_Li192ELi256ELi2ELi4ELi2ELi3ELb0ELb1EEEvNS_8GemmArgsE"
COPY = "__amd_rocclr_copyBuffer"


def test_labels_and_stages():
    lab = profsum.label(W12)
    assert lab == "gemm 192x256 waves 2x4 pf2 epi=SiTU-GLU out=bf16 gather=1 grouped=1"
    assert profsum.stage(lab, W12) == "expert W1/W2 + SiTU-GLU"
    lab3 = profsum.label(W3)
    assert lab3 == "gemm 192x256 waves 2x4 pf2 epi=rowscale out=fp16 gather=0 grouped=1"
    assert profsum.stage(lab3, W3) == "expert W3 x row weight"
    assert profsum.stage(profsum.label("void lmoe::topk_kernel<14>(...)"), "topk_kernel") == "top-k + routing weights"


def test_backward_labels():
    da = "_ZN4lmoe11gemm_kernelIDF16bDF16bLi192ELi256ELi2ELi4ELi1ELi3ELb1ELb1ELb0ELb1EEEvNS_8GemmArgsE"
    lab = profsum.label(da)
    assert lab.endswith("B[K,N]") and profsum.stage(lab, da) == "backward: da (W3 read in place)"
    dz = "void gemm_kernel<bool _Accum, 192, 256, 2, 4, 1, 0, false, true, false, true>"
    assert profsum.stage(profsum.label(dz), dz) == "backward: dz rows (W1, W2 read in place)"
    kr = "_ZN4lmoe11gemm_kernelIDF16bDF16bLi192ELi256ELi2ELi4ELi2ELi0ELb0ELb1ELb1ELb0EEEvNS_8GemmArgsE"
    assert profsum.stage(profsum.label(kr), kr) == "backward: expert weight gradients (K-range)"
    gate = "_ZN4lmoe11gemm_kernelIDF16bDF16bLi192ELi256ELi2ELi4ELi2ELi6ELb1ELb1ELb1ELb0EEEvNS_8GemmArgsE"
    assert profsum.stage(profsum.label(gate), gate).startswith("backward: gate")
    w12 = "_ZN4lmoe11gemm_kernelIDF16bDF16bLi192ELi256ELi2ELi4ELi2ELi2ELb1ELb1ELb1ELb0EEEvNS_8GemmArgsE"
    assert profsum.stage(profsum.label(w12), w12) == "expert W1/W2 + SiTU-GLU"


def _write_pass(d, counter, values):
    """values: {kernel: [value, ...]} or {kernel: [(value, grid), ...]}."""
    d.mkdir()
    with open(d / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, vals in values.items():
            for v in vals:
                val, grid = v if isinstance(v, tuple) else (v, 256)
                w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": val})


def _calib(tmp_path):
    # a 1 GiB copy split over two dispatches reads half its bytes in FETCH_SIZE and writes all of them
    _write_pass(tmp_path / "cf", "FETCH_SIZE", {COPY: [262144, 262144]})
    _write_pass(tmp_path / "cw", "WRITE_SIZE", {COPY: [524288, 524288]})
    return dict(calib_fetch=str(tmp_path / "cf"), calib_write=str(tmp_path / "cw"))


def test_counter_scaling_and_round_trip(tmp_path):
    # the workload's own device copies (of other sizes) do not enter the calibration
    _write_pass(tmp_path / "f", "FETCH_SIZE", {COPY: [1000, 5000], W12: [1000, 3000]})
    _write_pass(tmp_path / "w", "WRITE_SIZE", {COPY: [2000, 9000], W12: [100, 300]})
    out = tmp_path / "summary.md"
    profsum.counters(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "cmd", **_calib(tmp_path))
    text = out.read_text()
    assert "fetch_factor: 2.0000" in text and "write_factor: 1.0000" in text
    tb, sha = profsum.read_counters(str(out))
    assert tb == (2000 * 2.0 + 200 * 1.0) * 1024  # per-dispatch means, scaled, in bytes
    assert sha == profsum.source_sha256()


def test_rows_are_split_by_grid(tmp_path):
    # one kernel launched with two grids (e.g. the QB histogram at 1000 and 10000 bins): two rows
    hist = "_ZN4lmoe14qb_hist_kernelEPKflii"
    _write_pass(tmp_path / "f", "FETCH_SIZE", {hist: [(100, 1024), (100, 1024), (900, 8192)]})
    _write_pass(tmp_path / "w", "WRITE_SIZE", {hist: [(10, 1024), (10, 1024), (90, 8192)]})
    out = tmp_path / "summary.md"
    profsum.counters(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "cmd", **_calib(tmp_path))
    rows = [ln.split("|") for ln in out.read_text().splitlines() if "QB histogram" in ln]
    got = sorted((int(r[3]), int(r[4]), r[5].strip()) for r in rows)
    assert got == [(1024, 2, "100"), (8192, 1, "900")]


def test_qb_kernel_labels():
    # histogram instances <MARGIN, QUAD>, mangled and demangled
    assert profsum.label("_ZN4lmoe14qb_hist_kernelILb1ELb1EEEvPKfl") == "qb_hist_kernel (margin)"
    assert profsum.label("void lmoe::qb_hist_kernel<true, false>(float const*)") == "qb_hist_kernel (margin)"
    for plain in ("_ZN4lmoe14qb_hist_kernelILb0ELb1EEEvPKfl", "void lmoe::qb_hist_kernel<false, true>(float const*)"):
        assert profsum.label(plain) == "qb_hist_kernel"
        assert profsum.stage(profsum.label(plain), plain) == "QB histogram"
    mp = "lmoe::qb_merge_pool_kernel(int const*, int, int, int, int*, int, unsigned long long*)"
    assert profsum.stage(profsum.label(mp), mp) == "QB histogram: the runs' counts merged, pooled sum"
    dzsum = "_ZN4lmoe27combine_rmsnorm_wave_kernelIDF16bDF16bLi7EEEvPKT0_PKiPKT_PS6_iiiifi"
    assert profsum.stage(profsum.label(dzsum), dzsum) == "backward: dz sum (the token's dz rows)"
    fwd = "_ZN4lmoe27combine_rmsnorm_wave_kernelIDF16bDF16_Li7EEEvPKT0_PKiPKT_PS6_iiiifi"
    assert profsum.stage(profsum.label(fwd), fwd) == "combine + RMSNorm"


def test_missing_summary_and_stable_hash(tmp_path):
    assert profsum.read_counters(str(tmp_path / "none.md")) == (None, None)
    h = profsum.source_sha256()
    assert h == profsum.source_sha256() and len(h) == 64


def test_achieved_rate_from_kernel_trace(tmp_path):
    _write_pass(tmp_path / "f", "FETCH_SIZE", {W12: [1000]})
    _write_pass(tmp_path / "w", "WRITE_SIZE", {W12: [0]})
    stats = tmp_path / "k_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": W12, "Calls": 1, "AverageNs": 1000.0, "MinNs": 1000.0, "MaxNs": 1000.0, "Percentage": 100})
    out = tmp_path / "summary.md"
    profsum.counters(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "cmd", "title", str(stats),
                     **_calib(tmp_path))
    row = [ln for ln in out.read_text().splitlines() if "SiTU-GLU" in ln][0]
    gb = 1000 * 2.0 * 1024 / 1e9  # scaled bytes in GB
    assert row.rstrip(" |").split("|")[-1].strip() == f"{gb / 1e-6:.0f}"  # over 1 us


def test_lds_summary(tmp_path):
    d = tmp_path / "l"
    d.mkdir()
    rows = {"SQ_INSTS_LDS_LOAD_BANDWIDTH": 1000, "SQ_INSTS_LDS_STORE_BANDWIDTH": 600, "SQ_LDS_IDX_ACTIVE": 400,
            "SQ_LDS_BANK_CONFLICT": 4, "SQ_WAIT_INST_LDS": 10, "SQ_WAVE_CYCLES": 100, "GRBM_GUI_ACTIVE": 8 * 50}
    with open(d / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for c, v in rows.items():
            w.writerow({"Kernel_Name": W12, "Counter_Name": c, "Counter_Value": v})
    out = tmp_path / "lds.md"
    profsum.lds(str(d), str(out), "cmd", cus=4)
    row = [ln for ln in out.read_text().splitlines() if "SiTU-GLU" in ln][0].split("|")
    assert row[4].strip() == f"{1000 * 64 / 1e9:.2f}" and row[5].strip() == f"{600 * 64 / 1e9:.2f}"
    assert row[6].strip() == f"{1600 * 64 / (50 * 4):.1f}"   # bytes per clock and CU
    assert row[7].strip() == "1.0%" and row[8].strip() == "10.0%"
