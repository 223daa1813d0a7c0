"""Host logic of bench.py, no GPU: the per-step HBM byte bookkeeping from profiler
counters, its source-hash gate, the one-GPU guard and the algorithmic byte counts."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_run(directory, counter, rows):
    """A rocprofv3-style counter CSV: rows of (kernel name, dispatch id, value)."""
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "pmc_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for kernel, dispatch, value in rows:
            w.writerow([dispatch, kernel, counter, value])


def _ingest(tmp_path):
    # the same setup dispatch in every run (cancels in the difference), then one dispatch
    # per step with a fixed counter value: fused fetch 100 KiB / write 50 KiB per step,
    # unfused (two kernels) 300 + 40 KiB / 200 KiB per step
    setup = [("void fill_kernel(int)", 1, 7000.0)]
    per_step = {"fused": {"FETCH_SIZE": [("void coda::k_a(int)", 100.0)],
                          "WRITE_SIZE": [("void coda::k_a(int)", 50.0)]},
                "unfused": {"FETCH_SIZE": [("Cijk_x(int)", 300.0), ("at::native::ew(int)", 40.0)],
                            "WRITE_SIZE": [("Cijk_x(int)", 200.0)]}}
    dirs = []
    for path in ("fused", "unfused"):
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            for n in (2, 6):
                rows = list(setup)
                for step in range(n):
                    for j, (kernel, value) in enumerate(per_step[path][counter]):
                        rows.append((kernel, 10 + 4 * step + j, value))
                d = str(tmp_path / f"{path}_{counter}_{n}")
                _write_run(d, counter, rows)
                dirs.append(d)
    # plain copy of 1 MiB: FETCH_SIZE reads 512 KiB (factor 0.5), WRITE_SIZE 1024 KiB (1.0)
    _write_run(str(tmp_path / "copy_f"), "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1, 512.0)])
    _write_run(str(tmp_path / "copy_w"), "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1, 1024.0)])
    bench.ingest_step_traffic(["2", "6", *dirs, str(tmp_path / "copy_f"), str(tmp_path / "copy_w")],
                              "wl_test", 1 << 20, "test command")


def test_step_traffic_by_difference(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _ingest(tmp_path)
    rec = json.load(open(tmp_path / "profiles" / "step_traffic_wl_test.json"))
    assert rec["steps_differenced"] == 4
    assert rec["copy_factor_fetch"] == 0.5 and rec["copy_factor_write"] == 1.0
    # fetch counters are divided by 0.5, write counters by 1.0; the setup kernel cancels
    assert rec["fused"]["hbm_bytes_per_step"] == (200 + 50) * 1024
    assert rec["unfused"]["hbm_bytes_per_step"] == (600 + 80 + 200) * 1024
    assert rec["unfused"]["kernels"]["Cijk_x"] == [600 * 1024, 200 * 1024]
    assert "fill_kernel" not in rec["fused"]["kernels"]
    assert os.path.exists(tmp_path / "profiles" / "step_traffic_wl_test.txt")


def test_step_traffic_source_gate(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _ingest(tmp_path)
    got = bench.load_step_traffic("wl_test")
    assert got["fused"] == 250 * 1024 and got["unfused"] == 880 * 1024
    assert got["unfused_over_fused"] == round(880 / 250, 3)
    # a summary taken on other kernel sources is not reported
    p = tmp_path / "profiles" / "step_traffic_wl_test.json"
    rec = json.load(open(p))
    rec["fused_source_hash"] = "0" * 16
    json.dump(rec, open(p, "w"))
    assert bench.load_step_traffic("wl_test") is None
    assert bench.load_step_traffic("no_such_workload") is None


def test_one_gpu_guard():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "ONE GPU" in r.stderr and not r.stdout.strip()


def test_algorithmic_bytes_workload2():
    import synth_inputs as si

    w = si.WORKLOADS[2]
    fused = bench.algorithmic_bytes(w)
    M, K1, d, N2w, F = 16384, 2048, 2048, 16384, 8192
    # GEMM 1 reads A, Wo and x_res and writes h and 8 partials per row; the reduction
    # reads the partials and writes r; GEMM 2 reads h, W' and r and writes y
    assert fused["gemm1"] == 2 * (M * K1 + d * K1 + 2 * M * d) + 4 * M * 8
    assert fused["reduce"] == 4 * M * 8 + 4 * M
    assert fused["gemm2"] == 2 * (M * d + N2w * d + M * F) + 4 * M
    assert fused["total"] == 613548032
    # unfused: h = x_res + A.Wo written as two kernels, the RMSNorm kernel, the gate/up
    # product written and read back by the SwiGLU kernel
    assert bench.algorithmic_bytes(w, False)["total"] == 1954553856


def test_launch_groups():
    # one kernel launched on two problem sizes per step, interleaved: grouped by
    # duration, longest group first (within a group the indices come in duration order)
    durs = [880.0, 128.0, 905.0, 121.0, 870.0, 131.0]
    assert bench._launch_groups(durs) == [[4, 0, 2], [3, 1, 5]]
    assert bench._launch_groups([50.0]) == [[0]]
    assert bench._launch_groups([10.0, 11.0, 12.0]) == [[0, 1, 2]]


def test_roofline_kernels_resolve_to_their_sources():
    """Every kernel a bench line names for its roofline is defined in a translation unit the
    source hash covers, so its stored traffic is checked against the right files; the
    default workload's stored traffic belongs to the current sources of its kernel."""
    for k in ("k_gemm_rowscale_ovl", "k_gemm_swiglu_persistent", "k_gemm_ce_ovl", "k_gemm_rowscale_swiglu",
              "k_gemm_resid_partialrms",
              "k_gemm_rmsnorm_bwd", "k_gemm_wgrad", "k_rope_bwd", "k_swiglu_bwd_saved"):
        files = bench._kernel_files(k)
        assert any(f.endswith(".hip") for f in files), (k, files)
        if k.startswith("k_gemm"):
            assert "gemm_pipeline.hpp" in files, (k, files)     # the mainloops count too
        assert bench.kernel_source_hash(k) != ""
    rec = json.load(open(os.path.join(bench.ROOT, "profiles", "traffic_llama1b_attnout_mlpin_m16384.json")))
    assert "k_gemm_rowscale_ovl" in rec["kernels"]


def test_kernel_trace_summary_groups_launches(tmp_path):
    """--summarize-trace: per kernel instantiation, launches of one kernel on two problem
    sizes fall into two duration groups; other kernels are left out; the bench line of the
    same run is quoted."""
    d = tmp_path / "kt"
    d.mkdir()
    with open(d / "kt_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        i = 0
        for dur in (100_000, 101_000, 900_000, 905_000, 99_000):      # ns: two sizes
            i += 1
            w.writerow([i, "void coda::k_gemm_x<256, 256, 2>(int)", 1000 * i, 1000 * i + dur])
        w.writerow([99, "Cijk_vendor(int)", 0, 5000])
    log = tmp_path / "bench.log"
    log.write_text('noise\n{"metric": "m", "value": 1.5, "unit": "TFLOP/s", "ms_per_step": 1.0, '
                   '"kernels_ms": {"a": 1}}\n')
    path = bench.summarize_trace(str(d), "wl", str(log), "the command", out_dir=str(tmp_path))
    text = open(path).read()
    assert "# command: the command" in text and "1.0 ms per step, 1.5 TFLOP/s" in text
    rows = [r for r in text.splitlines() if r.startswith("k_gemm_x")]
    assert rows == ['k_gemm_x, "256, 256, 2", 0, 2, 902.5, 900.0, 905.0',     # longest group first
                    'k_gemm_x, "256, 256, 2", 1, 3, 100.0, 99.0, 101.0']
    assert "Cijk" not in text


def test_counter_ingest_pairs_library_and_vendor_kernels(tmp_path):
    """--ingest-counters: the vendor dispatches of a --vendor-probe run are split into the
    two GEMM shapes by duration; medians and the derived clock / MFMA busy / hit rate /
    fabric latency come out of the counters as defined."""
    import synth_inputs as si

    w = si.WORKLOADS[2]
    kern = {"g1": "void coda::k_gemm_resid_partialrms<256>(int)", "g2": "void coda::k_gemm_swiglu_persistent<256>(int)",
            "v": "Cijk_Alik_Bljk_x"}
    # (kernel, dispatch, duration ns); per pass the counters below, the same on every dispatch
    disp = [("g1", 1, 100_000), ("v", 2, 90_000), ("g2", 3, 800_000), ("v", 4, 700_000),
            ("g1", 5, 100_000), ("v", 6, 90_000), ("g2", 7, 800_000), ("v", 8, 700_000)]
    passes = {"p1": {"GRBM_GUI_ACTIVE": 8 * 150_000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 75_000.0},
              "p2": {"TCC_HIT": 80.0, "TCC_MISS": 20.0, "TCC_EA0_RDREQ": 10.0, "TCC_EA0_RDREQ_LEVEL": 5000.0}}
    dirs = []
    for pname, cs in passes.items():
        d = tmp_path / pname
        d.mkdir()
        with open(d / "pmc_counter_collection.csv", "w", newline="") as fh:
            wr = csv.writer(fh)
            wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                         "End_Timestamp"])
            for k, i, dur in disp:
                for c, v in cs.items():
                    wr.writerow([i, kern[k], c, v, 0, dur])
        dirs.append(str(d))
    path = bench.ingest_counters(dirs, w, "cmd", out_dir=str(tmp_path))
    rows = {tuple(r.split(", ")[:2]): r.split(", ") for r in open(path).read().splitlines()
            if not r.startswith("#") and not r.startswith("shape")}
    assert set(rows) == {("gemm1", "library"), ("gemm1", "vendor"), ("gemm2", "library"), ("gemm2", "vendor")}
    lib2 = rows[("gemm2", "library")]
    assert lib2[2] == "800.0" and float(lib2[3]) == round(2.0 * w.M * w.d * w.N2w / 800_000 / 1e3, 1)
    # clock 150000 cycles / 800 us = 0.1875 GHz; busy 75000 / 150000 = 0.5; hit 0.8; latency 500
    assert lib2[-4:] == ["0.188", "0.500", "0.800", "500.000"]
    assert rows[("gemm1", "vendor")][2] == "90.0" and rows[("gemm2", "vendor")][2] == "700.0"
