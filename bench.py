"""Throughput of the fused GEMM -> residual -> RMSNorm -> GEMM(+SwiGLU) chain on one GPU.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload 2]

One step = the whole chain (first GEMM + residual + partial sums of squares, the
row-scale reduction, second GEMM + row scale + SwiGLU) over one batch of synthetic
inputs already resident in HBM; the weight preparation (gamma fold / quantisation) runs
once before timing and is reported separately.  Prints ONE JSON line.

value      = GEMM FLOPs of the chain (2*M*K1*d + 2*M*d*N2w) / seconds per step, TFLOP/s
roofline   = the second GEMM kernel (the dominant one): its algorithmic FLOPs / its
             average duration from HIP events recorded around it on its own stream,
             against the dense MFMA peak of its dtype; `traffic` = its HBM bytes per
             launch from the committed rocprofv3 counter summary when that summary was
             taken on the current kernel sources, else null
cpu_baseline = the fp64 oracle on a bounded row sample of the same workload, on the
             host cores, scaled to TFLOP/s
hbm_bytes_measured = L2-miss bytes of one whole step of the fused chain and of the
             unfused torch chain, from the committed counter summary (two
             --traffic-probe runs differenced) when taken on the current kernel sources
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused chain TFLOP/s and % of MFMA peak at 16K tokens; HBM bytes vs unfused"
PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0}     # MI355X dense MFMA peaks
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "gemm_epilogue_transformer_amd", "csrc")


def _kernel_files(kernel: str) -> list:
    """The source files a kernel's device code is built from: the translation unit that
    defines it and the headers it includes, transitively (launch.hpp, host declarations
    only, excluded)."""
    import re

    tus = [f for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".cpp"))]
    defining = [f for f in tus if re.search(r"__global__[^;{]*?\b" + re.escape(kernel) + r"\s*\(",
                                              open(os.path.join(CSRC, f)).read(), re.S)]
    todo, seen = list(defining), set()
    while todo:
        f = todo.pop()
        if f in seen or f == "launch.hpp" or not os.path.exists(os.path.join(CSRC, f)):
            continue
        seen.add(f)
        todo += re.findall(r'#include\s+"([^"]+)"', open(os.path.join(CSRC, f)).read())
    return sorted(seen)


def kernel_source_hash(kernel: str | None = None) -> str:
    """Hash of the kernel's source files (all sources when kernel is None): a stored
    counter reading belongs to the kernel while this hash is unchanged."""
    files = _kernel_files(kernel) if kernel else [f for f in sorted(os.listdir(CSRC))
                                                   if f.endswith((".hip", ".hpp", ".cpp"))]
    if kernel and not files:
        return ""
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, fused=True) -> dict:
    """Each tensor moved once (bytes).  fused: the three-kernel chain; unfused: GEMM,
    add, RMSNorm, GEMM, SwiGLU as separate kernels with bf16 intermediates."""
    import synth_inputs as si

    eb = 1 if w.dtype == "e4m3" else 2
    M, K1, d, N2w, n_out = w.M, w.K1, w.d, w.N2w, w.n_out
    T = -(-d // 256)                      # one partial per 256-column tile of GEMM 1
    rope = w.act == si.ACT_ROPE
    ce = w.act == si.ACT_CE
    k1 = M * K1 * eb + d * K1 * eb + M * d * 2 + M * d * 2 + M * T * 4
    k2 = M * T * 4 + M * 4
    k3 = M * d * 2 + N2w * d * eb + M * 4 + M * n_out * 2
    if rope:                              # positions, cos / sin table
        k3 += M * 4 + 2 * w.seq_len * 32 * 4
    if ce:
        # no logits: targets in, one (max, sum-exp) pair per row and 256-column tile and
        # the target's logit out; the loss reduction reads those and writes lse and loss
        Tv = -(-N2w // 256)
        k3 = M * d * 2 + N2w * d * eb + M * 4 + M * 4 + M * Tv * 8 + M * 4
        k4 = M * Tv * 8 + M * 4 + M * 4 + 2 * M * 4
        if fused:
            return {"gemm1": k1, "reduce": k2, "gemm2": k3, "ce_reduce": k4, "total": k1 + k2 + k3 + k4}
        # unfused: GEMM 2 writes the bf16 logits, the loss kernel reads them
        tot = (M * K1 * eb + d * K1 * eb + M * d * 2) + 3 * M * d * 2 + 2 * M * d * 2 + d * 4 \
            + (M * d * 2 + N2w * d * eb + M * N2w * 2) + M * N2w * 2 + M * 4 + M * 4
        return {"total": tot}
    if fused:
        return {"gemm1": k1, "reduce": k2, "gemm2": k3, "total": k1 + k2 + k3}
    # unfused: the activation / rotation is a kernel of its own (reads z, writes y)
    act = M * N2w * 2 + M * n_out * 2 if (n_out != N2w or rope) else 0
    if rope:
        act += M * 4 + 2 * w.seq_len * 32 * 4
    tot = (M * K1 * eb + d * K1 * eb + M * d * 2) + 3 * M * d * 2 + 2 * M * d * 2 + d * 4 \
        + (M * d * 2 + N2w * d * eb + M * N2w * 2) + act
    return {"total": tot}


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch of a kernel from the committed counter summary of the workload,
    if it was taken on the kernel's current sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get(kernel)
    if rec is None or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _counter_means(directory: str, counter: str) -> dict:
    """Mean value per dispatch of a derived counter, per kernel name (rocprofv3 CSV)."""
    acc = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"]
        acc.setdefault(name, {}).setdefault(r["Dispatch_Id"], 0.0)
        acc[name][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in acc.items()}


def _counter_sums(directory: str, counter: str) -> dict:
    """Sum of a derived counter over all dispatches, per kernel name (rocprofv3 CSV)."""
    acc = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") == counter:
            acc[r["Kernel_Name"]] = acc.get(r["Kernel_Name"], 0.0) + float(r["Counter_Value"])
    return acc


def _short_kernel_name(name: str) -> str:
    name = name.replace("void ", "")
    return (name.split("(")[0].split("<")[0])[:72]


def ingest_step_traffic(args_list, workload: str, copy_bytes: int, command: str) -> None:
    """HBM bytes of one whole step of the fused chain and of the unfused torch chain.

    args_list: n_small n_big, then for the fused and the unfused path the FETCH_SIZE run
    at n_small and n_big steps and the WRITE_SIZE run at n_small and n_big steps
    (``--traffic-probe``), then the FETCH_SIZE and WRITE_SIZE runs of the plain copy.  The
    setup launches the same kernels at both step counts, so the difference of the summed
    counters over n_big - n_small steps is what the steps themselves moved; each counter
    is divided by what it reads per byte of the plain copy."""
    import torch

    n_small, n_big = int(args_list[0]), int(args_list[1])
    dirs = args_list[2:]
    pick = lambda d: next(v for k, v in d.items() if "copy" in k.lower())  # noqa: E731
    kib = copy_bytes / 1024.0
    ff = pick(_counter_means(dirs[8], "FETCH_SIZE")) / kib
    fw = pick(_counter_means(dirs[9], "WRITE_SIZE")) / kib
    steps = n_big - n_small
    rec = {"workload": workload, "steps_differenced": steps, "copy_factor_fetch": ff, "copy_factor_write": fw,
           "fused_source_hash": kernel_source_hash(), "torch": torch.__version__, "command": command}
    lines = [f"# HBM bytes per step (FETCH_SIZE / copy factor + WRITE_SIZE / copy factor), workload {workload}",
             f"# commands: {command}",
             f"# per step = (counters summed over a run of {n_big} steps - the same over {n_small} steps) / {steps};"
             f" copy factors FETCH_SIZE {ff:.4f}, WRITE_SIZE {fw:.4f} KiB per KiB copied",
             "path, kernel, fetch bytes per step, write bytes per step"]
    for i, path in enumerate(("fused", "unfused")):
        fs, fb, ws, wb = (_counter_sums(d, c) for d, c in
                          zip(dirs[4 * i: 4 * i + 4], ("FETCH_SIZE", "FETCH_SIZE", "WRITE_SIZE", "WRITE_SIZE")))
        per = {}
        for small, big, slot in ((fs, fb, 0), (ws, wb, 1)):
            for k in set(small) | set(big):
                v = (big.get(k, 0.0) - small.get(k, 0.0)) * 1024 / (ff if slot == 0 else fw) / steps
                per.setdefault(_short_kernel_name(k), [0.0, 0.0])[slot] += v
        # kernels of the setup alone difference to zero
        per = {k: v for k, v in per.items() if abs(v[0]) + abs(v[1]) >= 1.0}
        total = sum(v[0] + v[1] for v in per.values())
        rec[path] = {"hbm_bytes_per_step": round(total),
                     "kernels": {k: [round(v[0]), round(v[1])] for k, v in sorted(per.items())}}
        for k, v in sorted(per.items(), key=lambda kv: -(kv[1][0] + kv[1][1])):
            lines.append(f"{path}, {k}, {v[0]:.0f}, {v[1]:.0f}")
        lines.append(f"{path}, TOTAL, {total:.0f}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"step_traffic_{workload}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(os.path.join(ROOT, "profiles", f"step_traffic_{workload}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_step_traffic(workload: str):
    """Measured HBM bytes per step of the fused and the unfused chain, if the fused ones
    were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"step_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("fused_source_hash") != kernel_source_hash():
        return None
    f, u = rec["fused"]["hbm_bytes_per_step"], rec["unfused"]["hbm_bytes_per_step"]
    return {"fused": f, "unfused": u, "unfused_over_fused": round(u / f, 3), "torch": rec.get("torch")}


def _dispatches(directory: str, counter: str) -> dict:
    """Per kernel name: its dispatches in launch order, each [counter value summed over
    its rows, duration in ns] (rocprofv3 CSV)."""
    acc = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        d = acc.setdefault(r["Kernel_Name"], {})
        rec = d.setdefault(int(r["Dispatch_Id"]), [0.0, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])])
        rec[0] += float(r["Counter_Value"])
    return {k: [v[i] for i in sorted(v)] for k, v in acc.items()}


def _launch_groups(durations: list) -> list:
    """Indices of one kernel's dispatches split into groups of similar duration (the
    same kernel launched on different problems within a step), longest first."""
    order = sorted(range(len(durations)), key=lambda i: durations[i])
    groups, cur = [], [order[0]]
    for i in order[1:]:
        if durations[i] > 1.5 * durations[cur[-1]]:
            groups.append(cur)
            cur = []
        cur.append(i)
    groups.append(cur)
    return groups[::-1]


def _template_args(name: str) -> str:
    """The template argument list of a demangled kernel name ('' if none)."""
    i = name.find("<")
    if i < 0 or name.find("(") < i:
        return ""
    depth = 0
    for j in range(i, len(name)):
        if name[j] == "<":
            depth += 1
        elif name[j] == ">":
            depth -= 1
            if depth == 0:
                return name[i + 1:j]
    return ""


def summarize_trace(directory: str, workload: str, bench_log: str, command: str, out_dir: str = "") -> str:
    """Write profiles/kernel_trace_<workload>.txt from a rocprofv3 --kernel-trace csv run:
    the library's kernels per template instantiation and launch group (one kernel on
    problems of different size in one step, told apart by duration), with launches and
    average / min / max duration, plus the bench line of the same run."""
    acc = {}
    for r in _csv_rows(directory, "kernel_trace.csv"):
        n = r["Kernel_Name"]
        if "coda::" not in n:
            continue
        key = (_short_kernel_name(n).split("::")[-1], _template_args(n))
        acc.setdefault(key, []).append((int(r["Dispatch_Id"]),
                                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    line = ""
    for ln in open(bench_log):
        if ln.startswith("{") and '"metric"' in ln:
            line = ln
    b = json.loads(line) if line else {}
    out = [f"# rocprofv3 kernel-trace summary, workload {workload}",
           f"# command: {command}",
           f"# summary: python3 bench.py --summarize-trace DIR {workload} BENCH_LOG --ingest-command '<the command>'",
           f"# kernel source hash (all sources): {kernel_source_hash()}; the same run's bench line: "
           f"{b.get('ms_per_step')} ms per step, {b.get('value')} {b.get('unit', '')}, per-kernel HIP events (ms) "
           f"{json.dumps(b.get('kernels_ms'))}",
           "# per kernel instantiation and launch group (the same kernel on problems of different size in one step, "
           "grouped by duration): launches, average / min / max duration in us",
           "kernel, template arguments, group, launches, avg_us, min_us, max_us"]
    recs = []
    for (base, ta), disp in acc.items():
        disp.sort()
        durs = [x[1] for x in disp]
        for g, idx in enumerate(_launch_groups(durs)):
            v = [durs[i] for i in idx]
            recs.append((len(disp), base, ta, g, len(v), sum(v) / len(v), min(v), max(v)))
    recs.sort(key=lambda x: (-x[0], x[1], x[3]))
    for _, base, ta, g, n, a, mn, mx in recs:
        out.append(f'{base}, "{ta}", {g}, {n}, {a:.1f}, {mn:.1f}, {mx:.1f}')
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"kernel_trace_{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))
    return path


def ingest_counters(dirs, w, command: str, out_dir: str = "") -> str:
    """profiles/counters_<workload>.txt: per kernel of a --vendor-probe run (the library's two
    GEMMs and the vendor GEMM of each shape, told apart by duration), the median over its
    dispatches of every counter collected in the passes `dirs`, and derived figures:
    clock = GRBM_GUI_ACTIVE / 8 XCDs / duration, MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /
    1024 SIMDs / (GRBM_GUI_ACTIVE / 8), L2 hit rate, mean fabric read latency =
    TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ, TFLOP/s of the dispatch."""
    import statistics

    flops = {"gemm1": 2.0 * w.M * w.K1 * w.d, "gemm2": 2.0 * w.M * w.d * w.N2w}
    vals, durs = {}, {}
    for dr in dirs:
        per = {}
        for r in _csv_rows(dr, "counter_collection.csv"):
            name = r["Kernel_Name"]
            if "coda::" in name:
                kind = ("gemm1" if "resid_partialrms" in name else
                        ("gemm2" if "swiglu" in name or "rowscale_ovl" in name else None))
                who = "library"
            elif name.startswith("Cijk") or "Cijk" in name[:40]:
                kind, who = None, "vendor"
            else:
                continue
            key = (name, int(r["Dispatch_Id"]))
            rec = per.setdefault(key, {"who": who, "kind": kind, "dur": int(r["End_Timestamp"]) -
                                       int(r["Start_Timestamp"]), "c": {}})
            rec["c"][r["Counter_Name"]] = rec["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        # the vendor dispatches alternate between the two shapes: the longer ones are GEMM 2
        vend = sorted([k for k, v in per.items() if v["who"] == "vendor"], key=lambda k: per[k]["dur"])
        for k in vend[: len(vend) // 2]:
            per[k]["kind"] = "gemm1"
        for k in vend[len(vend) // 2:]:
            per[k]["kind"] = "gemm2"
        for (name, _), v in per.items():
            if v["kind"] is None:
                continue
            row = (v["kind"], v["who"])
            durs.setdefault(row, []).append(v["dur"])
            for c, x in v["c"].items():
                vals.setdefault(row, {}).setdefault(c, []).append(x)
    rows = sorted(vals, key=lambda r: (r[0], r[1] != "library"))
    counters = sorted({c for r in rows for c in vals[r]})
    med = {r: {c: statistics.median(vals[r][c]) for c in vals[r]} for r in rows}
    mdur = {r: statistics.median(durs[r]) for r in rows}
    lines = [f"# counters per dispatch, workload {w.name}: the library's GEMMs against the vendor GEMM "
             f"(torch.matmul, hipBLASLt) of the same operands",
             f"# command: {command}",
             f"# summary: python3 bench.py --workload <n> --ingest-counters DIR... --ingest-command '<the command>'",
             f"# kernel source hash (all sources): {kernel_source_hash()}",
             "# medians over each kernel's dispatches (durations under the profiler); derived: clock_ghz = "
             "GRBM_GUI_ACTIVE / 8 / duration, mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 / (GRBM_GUI_ACTIVE / 8), "
             "l2_hit = TCC_HIT / (TCC_HIT + TCC_MISS), fabric_read_latency = TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ",
             "shape, kernel, " + ", ".join(["dur_us", "tflops"] + counters +
                                           ["clock_ghz", "mfma_busy", "l2_hit", "fabric_read_latency"])]
    for r in rows:
        m, du = med[r], mdur[r]
        g = m.get("GRBM_GUI_ACTIVE")
        der = [g / 8 / du if g else None,
               m["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (g / 8) if g and "SQ_VALU_MFMA_BUSY_CYCLES" in m else None,
               m["TCC_HIT"] / (m["TCC_HIT"] + m["TCC_MISS"]) if "TCC_HIT" in m and "TCC_MISS" in m else None,
               m["TCC_EA0_RDREQ_LEVEL"] / m["TCC_EA0_RDREQ"] if m.get("TCC_EA0_RDREQ") and
               "TCC_EA0_RDREQ_LEVEL" in m else None]
        cells = [f"{du / 1e3:.1f}", f"{flops[r[0]] / du / 1e3:.1f}"] + \
                [f"{m[c]:.4g}" if c in m else "" for c in counters] + \
                [f"{x:.3f}" if x is not None else "" for x in der]
        lines.append(f"{r[0]}, {r[1]}, " + ", ".join(cells))
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"counters_{w.name}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return path


def ingest_traffic(dirs, workload: str, copy_bytes: int, command: str) -> None:
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the bench, then of the
    plain copy) into profiles/traffic_<workload>.json: HBM-side bytes per launch of each kernel,
    each counter divided by what it reads per byte of the plain copy.  Every library
    kernel of the run is covered.  Where one kernel name ran in several template
    instantiations (a forward run in a backward bench's setup), the instantiation with
    the most dispatches -- the timed one -- is taken; where one instantiation ran on
    problems of different size within a step (the input-gradient kernel for both GEMMs of
    the whole-chain backward), its dispatches are grouped by duration, matched across the
    two runs by launch order, and the longest group -- the dominant launch -- is stored
    (every group is listed in the text summary)."""
    f_run, w_run = _dispatches(dirs[0], "FETCH_SIZE"), _dispatches(dirs[1], "WRITE_SIZE")
    f_cal, w_cal = _counter_means(dirs[2], "FETCH_SIZE"), _counter_means(dirs[3], "WRITE_SIZE")
    pick = lambda d: next(v for k, v in d.items() if "copy" in k.lower())  # noqa: E731
    kib = copy_bytes / 1024.0
    ff, fw = pick(f_cal) / kib, pick(w_cal) / kib
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    lines = [f"# HBM traffic per launch, workload {workload}",
             f"# commands: {command}",
             f"# copy calibration: {copy_bytes} bytes copied; FETCH_SIZE reads {ff:.4f} KiB per KiB, "
             f"WRITE_SIZE {fw:.4f} KiB per KiB",
             "kernel, launch group, dispatches, mean duration us (under the profiler), FETCH_SIZE KiB, "
             "WRITE_SIZE KiB, traffic bytes (scaled)"]
    out = {"workload": workload, "command": command, "copy_factor_fetch": ff, "copy_factor_write": fw,
           "kernels": {}}
    best = {}
    for full, disp in f_run.items():
        if "coda::" not in full or len(w_run.get(full, [])) != len(disp):
            continue
        base = _short_kernel_name(full).split("::")[-1]
        if base not in best or len(disp) > len(f_run[best[base]]):
            best[base] = full
    for base, full in sorted(best.items()):
        fd, wd = f_run[full], w_run[full]
        for g, idx in enumerate(_launch_groups([x[1] for x in fd])):
            fk = sum(fd[i][0] for i in idx) / len(idx)
            wk = sum(wd[i][0] for i in idx) / len(idx)
            us = sum(fd[i][1] for i in idx) / len(idx) / 1e3
            traffic = fk * 1024 / ff + wk * 1024 / fw
            if g == 0:
                out["kernels"][base] = {"instantiation": full.split("(")[0], "source_hash": kernel_source_hash(base),
                                        "dispatches": len(idx), "mean_duration_us_profiled": round(us, 1),
                                        "fetch_kib": fk, "write_kib": wk, "hbm_bytes_per_launch": round(traffic)}
            lines.append(f"{base}, {g}, {len(idx)}, {us:.1f}, {fk:.1f}, {wk:.1f}, {traffic:.0f}")
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def bench_backward(w, args) -> dict:
    """Backward step.  Workload of the MLP-input block: its input gradient (three calls)
    and the weight and gamma gradients (the token-contracting GEMM on dz and h as stored,
    the column sum).  Whole-chain workload: the same plus the first GEMM's input gradient
    dA and weight gradient dWo (the plain GEMM, the token-contracting GEMM on dh and A);
    the residual input's gradient is dh itself.  The saved forward state -- folded
    weight, weight transposes, h and r (from a forward run of the chain) -- is prepared
    outside the timed region."""
    import numpy as np
    import torch

    import gemm_epilogue_transformer_amd as coda
    import synth_inputs as si

    whole = w.act == si.ACT_CHAIN_BWD
    inp = si.generate(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    W, dy = dev(inp["W_t"]), dev(inp["dy"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    M, d, F, K1 = w.M, w.d, w.N2w // 2, w.K1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    Wp = coda.prepare_weight_bf16(W, gamma)
    Wpt = coda.transpose_bf16(Wp)
    saved = args.saved_z
    z = None
    if whole:
        A, Wo, xr, dres = dev(inp["A"]), dev(inp["Wo_t"]), dev(inp["x_res"]), dev(inp["dres"])
        WoT = coda.transpose_bf16(Wo)
        fwd = coda.chain(A, Wo, xr, Wp, w.eps, save_z=saved)
        h, r = fwd[0], fwd[2]
        z = fwd[4] if saved else None
    else:
        h = dev(inp["h"])
        dres = None
        r = coda.rowscale_from_h(h, w.eps)
        if saved:
            _, z = coda.gemm_rowscale_swiglu_save(h, Wp, r)
    torch.cuda.synchronize()
    prep_ms = (time.perf_counter() - t0) * 1e3
    TW = coda.wgrad_partials_rows(2 * F)
    f32 = dict(dtype=torch.float32, device="cuda")
    b16 = dict(dtype=torch.bfloat16, device="cuda")
    out = {"dz": torch.empty((M, 2 * F), **b16), "partials": torch.empty((M, -(-F // 128)), **f32),
           "q": torch.empty(M, **f32), "dh": torch.empty((M, d), **b16),
           "dW": torch.empty((2 * F, d), **f32), "wpartials": torch.empty((TW, d), **f32),
           "dgamma": torch.empty(d, **f32)}
    if whole:
        out.update({"dA": torch.empty((M, K1), **b16), "dWo": torch.empty((d, K1), **f32)})
        nws = coda.wgrad_workspace_bytes(d, K1, M)
        out["ws"] = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws > 0 else None
    stream = torch.cuda.current_stream()
    # (name, kernel, call); the calls write into `out`
    if saved:
        stages = [("swiglu_bwd_saved", "k_swiglu_bwd_saved",
                   lambda: coda.swiglu_bwd_saved(z, dy, r, out["dz"], None, out["partials"], transpose=False))]
    else:
        stages = [("gemm_swiglu_bwd", "k_gemm_rowscale_swiglu",
                   lambda: coda.gemm_swiglu_bwd(h, Wp, r, dy, out["dz"], out["partials"]))]
    stages += [
        ("rmsnorm_bwd_reduce", "k_rmsnorm_bwd_reduce",
         lambda: coda.rmsnorm_bwd_reduce(out["partials"], r, d, F, out["q"])),
        ("gemm_rmsnorm_bwd", "k_gemm_rmsnorm_bwd",
         lambda: coda.gemm_rmsnorm_bwd(out["dz"], Wpt, h, out["q"], dres, out["dh"]))]
    # the weight gradients read dz, h, dh and A as stored (token-major): no transposes
    stages += [
        ("gemm_wgrad", "k_gemm_wgrad",
         lambda: coda.gemm_wgrad_tok(out["dz"], h, gamma, W, out["dW"], out["wpartials"])),
        ("colsum_reduce", "k_colsum_reduce", lambda: coda.colsum_reduce(out["wpartials"], out["dgamma"]))]
    if whole:
        stages += [
            ("gemm_dA", "k_gemm_rmsnorm_bwd", lambda: coda.gemm_bf16(out["dh"], WoT, None, out["dA"])),
            ("gemm_wgrad_dWo", "k_gemm_wgrad",                                # token split + its reduce
             lambda: coda.gemm_wgrad_tok(out["dh"], A, None, None, out["dWo"], None, out["ws"]))]
    names = [x[0] for x in stages]
    kern = [x[1] for x in stages]

    def step(ev=None):
        for i, (_, _, call) in enumerate(stages):
            if ev is not None:
                ev[i].record(stream)
            call()
        if ev is not None:
            ev[len(stages)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    k_ms = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i in range(len(names))]
    g_flops = 2 * M * d * 2 * F
    g1_flops = 2 * M * d * K1
    flops = w.gemm_flops - (g_flops if saved else 0)          # the GEMMs executed
    fl_of = {"gemm_swiglu_bwd": g_flops, "gemm_rmsnorm_bwd": g_flops, "gemm_wgrad": g_flops,
             "gemm_dA": g1_flops, "gemm_wgrad_dWo": g1_flops}
    gemm_fl = {i: fl_of[n] for i, n in enumerate(names) if n in fl_of}
    gemms = list(gemm_fl)
    value = flops / (ms_per_step * 1e-3) / 1e12
    dom = max(gemms, key=lambda i: k_ms[i])
    T = -(-F // 128)
    byt = {"gemm_swiglu_bwd": M * d * 2 + 2 * F * d * 2 + M * 4 + M * F * 2 + M * 2 * F * 2 + M * T * 4,
           "swiglu_bwd_saved": M * 2 * F * 2 + M * F * 2 + M * 4 + M * 2 * F * 2 + M * T * 4,
           "rmsnorm_bwd_reduce": M * T * 4 + 2 * M * 4,
           "gemm_rmsnorm_bwd": M * 2 * F * 2 + d * 2 * F * 2 + M * d * 2 + M * 4 + M * d * 2
                               + (M * d * 2 if whole else 0),
           "transpose_dz": 2 * M * 2 * F * 2,
           "transpose_h": 2 * M * d * 2,
           "gemm_wgrad": 2 * F * M * 2 + d * M * 2 + d * 4 + 2 * F * d * 2 + 2 * F * d * 4 + TW * d * 4,
           "colsum_reduce": TW * d * 4 + d * 4}
    if whole:
        byt.update({"gemm_dA": M * d * 2 + K1 * d * 2 + M * K1 * 2, "transpose_dh": 2 * M * d * 2,
                    "transpose_A": 2 * M * K1 * 2, "gemm_wgrad_dWo": d * M * 2 + K1 * M * 2 + d * K1 * 4})
    achieved = gemm_fl[dom] / (k_ms[dom] * 1e-3) / 1e12
    direction = "backward of the whole chain (dx_res = dh, dA, dWo, dW, dgamma)" if whole else \
        "backward (input, weight and gamma gradients)"
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "M": M, "K1": K1, "d": d, "F": F, "direction": direction,
                   "pre_activation": "saved by the forward" if saved else "recomputed", "eps": w.eps,
                   "seed": w.seed},
        "note": "FLOPs of the executed GEMMs: " + ("" if saved else "the recomputed gate/up product, ")
                + "the input-gradient product and the weight-gradient product"
                + (", and the first GEMM's input- and weight-gradient products" if whole else ""),
        "kernels_ms": {n: round(t, 4) for n, t in zip(names, k_ms)},
        "gemm_tflops": {names[i]: round(gemm_fl[i] / (k_ms[i] * 1e-3) / 1e12, 1) for i in gemms},
        "hbm_bytes_algorithmic": {"fused": sum(byt[n] for n in names)},
        "prep_ms": round(prep_ms, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": load_traffic(w.name + ("_saved_z" if saved else ""), kern[dom]), "kernel": kern[dom],
                     "kernel_ms": round(k_ms[dom], 4), "algorithmic_bytes": byt[names[dom]],
                     "kernel_source_hash": kernel_source_hash(kern[dom])},
        "kernel_source_hash": kernel_source_hash(),
    }
    if args.unfused:
        # torch autograd of the unfused forward (bf16 GEMMs, element-wise RMSNorm / SwiGLU)
        # for the same gradients; the forward runs once outside the timed region and its
        # saved activations are reused: this baseline does NOT recompute the gate/up product
        Wl = W.clone().requires_grad_(True)
        gl = gamma.clone().requires_grad_(True)
        if whole:
            Al, Wol, xl = A.clone().requires_grad_(True), Wo.clone().requires_grad_(True), \
                xr.clone().requires_grad_(True)
            hh = xl + Al @ Wol.t()
            leaves = (Al, Wol, xl, Wl, gl)
        else:
            hh = h.clone().requires_grad_(True)
            leaves = (hh, Wl, gl)
        hf = hh.float()
        n = (hf * torch.rsqrt(hf.pow(2).mean(-1, keepdim=True) + w.eps)).to(torch.bfloat16) * gl.to(torch.bfloat16)
        z = n @ Wl.t()
        y = torch.nn.functional.silu(z[:, :F]) * z[:, F:]
        outs, grads = ((y, hh), (dy, dres)) if whole else ((y,), (dy,))

        def ubwd():
            torch.autograd.grad(outs, leaves, grads, retain_graph=True)

        for _ in range(3):
            ubwd()
        torch.cuda.synchronize()
        s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s2.record(stream)
        for _ in range(args.steps):
            ubwd()
        e2.record(stream)
        torch.cuda.synchronize()
        ums = s2.elapsed_time(e2) / args.steps
        rec["unfused_torch"] = {"ms_per_step": round(ums, 4), "speedup_of_fused": round(ums / ms_per_step, 3),
                                "note": "torch autograd of the same gradients from saved activations "
                                        f"({4 if whole else 2} GEMMs, no recompute)"}
    if not args.no_cpu_baseline:
        import oracle

        rng = np.random.default_rng(0)
        # input gradient: sampled rows (a fraction rows / M of the two GEMMs it runs);
        # weight gradients: sampled rows of dW, every column (a fraction js / 2F of the third)
        if whole:
            prep = oracle.prepare(inp, "bf16")
            Wp_ref = prep["Wp"]
        else:
            Wp_ref = oracle.fold_bf16(inp["W_t"], inp["gamma"])
        n_rows, dt1 = 8, 0.0
        while True:
            rows = np.sort(rng.choice(M, size=min(n_rows, M), replace=False))
            t1 = time.perf_counter()
            if whole:
                oracle.chain_bwd(prep, inp["x_res"], inp["gamma"], inp["W_t"], inp["dy"], w.eps, dres=inp["dres"],
                                 rows=rows)
            else:
                oracle.mlpin_bwd(inp["h"], inp["gamma"], Wp_ref, oracle.BF16, 1.0, inp["dy"], w.eps, rows=rows)
            dt1 = time.perf_counter() - t1
            if dt1 >= args.cpu_seconds / 4 or n_rows >= M:
                break
            n_rows *= 2
        hb_all = oracle.chain(prep, inp["x_res"], inp["gamma"], oracle.ACT_SWIGLU, w.eps)["hb"] if whole \
            else inp["h"]
        n_js, dt2 = 1, 0.0
        while True:
            js = np.sort(rng.choice(2 * F, size=min(n_js, 2 * F), replace=False))
            t1 = time.perf_counter()
            oracle.mlpin_wgrad(hb_all, inp["gamma"], Wp_ref, oracle.BF16, 1.0, inp["W_t"], inp["dy"], w.eps, js=js)
            dt2 = time.perf_counter() - t1
            if dt2 >= args.cpu_seconds / 4 or n_js >= 2 * F:
                break
            n_js *= 2
        per_row = (2 * g_flops + (g1_flops if whole else 0)) / M       # recompute, dh (and dA) per row
        done = rows.size * per_row + js.size / (2 * F) * g_flops
        rec["cpu_baseline"] = {"value": round(done / (dt1 + dt2) / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": f"{rows.size} random rows of dh{' and dA' if whole else ''} ({dt1:.1f} s) "
                                         f"and {js.size} random rows of dW, all columns ({dt2:.1f} s), of the "
                                         f"{M}-token workload (fp64, recomputed forward included)"}
    return rec


def bench_rope_backward(w, args) -> dict:
    """Backward step of the QKV block y = RoPE(RMSNorm(h) . W^T): the RoPE backward from
    the forward's output y (r * RoPE^T(dy) and the row-scale partials in one pass), the
    row coefficient, the input-gradient GEMM, the weight-gradient GEMM on dz and h as
    stored, and the column sum for gamma.  The saved forward state -- folded weight and
    its transpose, r, y and the angle table -- is prepared outside the timed region."""
    import numpy as np
    import torch

    import gemm_epilogue_transformer_amd as coda

    import synth_inputs as si

    inp = si.generate(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    h, W, dy = dev(inp["h"]), dev(inp["W_t"]), dev(inp["dy"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    pos = torch.from_numpy(inp["pos"]).cuda()
    M, d, N, rot = w.M, w.d, w.N2w, w.rot_cols
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    Wp = coda.prepare_weight_bf16(W, gamma)
    Wpt = coda.transpose_bf16(Wp)
    r = coda.rowscale_from_h(h, w.eps)
    cos_t, sin_t = coda.rope_table(w.seq_len, w.rope_base)
    y = coda.gemm_rowscale_rope(h, Wp, r, pos, cos_t, sin_t, rot)
    torch.cuda.synchronize()
    prep_ms = (time.perf_counter() - t0) * 1e3
    T = -(-N // 128)
    TW = coda.wgrad_partials_rows(N)
    f32 = dict(dtype=torch.float32, device="cuda")
    b16 = dict(dtype=torch.bfloat16, device="cuda")
    out = {"dz": torch.empty((M, N), **b16), "partials": torch.empty((M, T), **f32), "q": torch.empty(M, **f32),
           "dh": torch.empty((M, d), **b16), "dW": torch.empty((N, d), **f32),
           "wpartials": torch.empty((TW, d), **f32), "dgamma": torch.empty(d, **f32)}
    # the weight has few 256-row tiles (N / 256 x d / 256): its gradient splits the tokens
    nws = coda.wgrad_workspace_bytes(N, d, M)
    out["wws"] = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws > 0 else None
    stream = torch.cuda.current_stream()
    stages = [
        ("rope_bwd", "k_rope_bwd",
         lambda: coda.rope_bwd(dy, y, r, pos, cos_t, sin_t, rot, out["dz"], out["partials"])),
        ("rmsnorm_bwd_reduce", "k_rmsnorm_bwd_reduce",
         lambda: coda.rmsnorm_bwd_reduce(out["partials"], r, d, N, out["q"])),
        ("gemm_rmsnorm_bwd", "k_gemm_rmsnorm_bwd",
         lambda: coda.gemm_rmsnorm_bwd(out["dz"], Wpt, h, out["q"], None, out["dh"])),
        ("gemm_wgrad", "k_gemm_wgrad",          # with the token split and its fixed-order reduce
         lambda: coda.gemm_wgrad_tok(out["dz"], h, gamma, W, out["dW"], out["wpartials"], out["wws"])),
        ("colsum_reduce", "k_colsum_reduce", lambda: coda.colsum_reduce(out["wpartials"], out["dgamma"]))]
    names = [x[0] for x in stages]
    kern = [x[1] for x in stages]

    def step(ev=None):
        for i, (_, _, call) in enumerate(stages):
            if ev is not None:
                ev[i].record(stream)
            call()
        if ev is not None:
            ev[len(stages)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    k_ms = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i in range(len(names))]
    g_flops = 2 * M * d * N
    gemm_fl = {names.index("gemm_rmsnorm_bwd"): g_flops, names.index("gemm_wgrad"): g_flops}
    value = w.gemm_flops / (ms_per_step * 1e-3) / 1e12
    dom = max(gemm_fl, key=lambda i: k_ms[i])
    byt = {"rope_bwd": 3 * M * N * 2 + 2 * M * 4 + 2 * w.seq_len * 32 * 4 + M * T * 4,
           "rmsnorm_bwd_reduce": M * T * 4 + 2 * M * 4,
           "gemm_rmsnorm_bwd": M * N * 2 + d * N * 2 + M * d * 2 + M * 4 + M * d * 2,
           "gemm_wgrad": M * N * 2 + M * d * 2 + d * 4 + N * d * 2 + N * d * 4 + TW * d * 4,
           "colsum_reduce": TW * d * 4 + d * 4}
    achieved = gemm_fl[dom] / (k_ms[dom] * 1e-3) / 1e12
    i_rb = names.index("rope_bwd")
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "M": M, "d": d, "N": N, "rot_cols": rot, "seq_len": w.seq_len,
                   "rope_base": w.rope_base, "direction": "backward of the QKV block (dh, dW, dgamma)",
                   "eps": w.eps, "seed": w.seed},
        "note": "FLOPs of the executed GEMMs: the input-gradient product and the weight-gradient product",
        "kernels_ms": {n: round(t, 4) for n, t in zip(names, k_ms)},
        "gemm_tflops": {names[i]: round(gemm_fl[i] / (k_ms[i] * 1e-3) / 1e12, 1) for i in gemm_fl},
        "rope_bwd_gbs": round(byt["rope_bwd"] / (k_ms[i_rb] * 1e-3) / 1e9, 1),
        "hbm_bytes_algorithmic": {"fused": sum(byt[n] for n in names)},
        "prep_ms": round(prep_ms, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": load_traffic(w.name, kern[dom]), "kernel": kern[dom],
                     "kernel_ms": round(k_ms[dom], 4), "algorithmic_bytes": byt[names[dom]],
                     "kernel_source_hash": kernel_source_hash(kern[dom])},
        "kernel_source_hash": kernel_source_hash(),
    }
    if args.unfused:
        # torch autograd of the unfused forward (bf16 GEMM, element-wise RMSNorm and
        # rotation with the table gathered by position) for the same gradients
        hh = h.clone().requires_grad_(True)
        Wl = W.clone().requires_grad_(True)
        gl = gamma.clone().requires_grad_(True)
        hf = hh.float()
        n = (hf * torch.rsqrt(hf.pow(2).mean(-1, keepdim=True) + w.eps)).to(torch.bfloat16) * gl.to(torch.bfloat16)
        z = n @ Wl.t()
        q = z[:, :rot].view(M, -1, 64)
        c, s_ = cos_t[pos].unsqueeze(1), sin_t[pos].unsqueeze(1)
        x1, x2 = q[..., :32], q[..., 32:]
        rq = torch.cat([x1 * c - x2 * s_, x2 * c + x1 * s_], -1).to(torch.bfloat16)
        yu = torch.cat([rq.view(M, -1), z[:, rot:]], 1)

        def ubwd():
            torch.autograd.grad((yu,), (hh, Wl, gl), (dy,), retain_graph=True)

        for _ in range(3):
            ubwd()
        torch.cuda.synchronize()
        s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s2.record(stream)
        for _ in range(args.steps):
            ubwd()
        e2.record(stream)
        torch.cuda.synchronize()
        ums = s2.elapsed_time(e2) / args.steps
        rec["unfused_torch"] = {"ms_per_step": round(ums, 4), "speedup_of_fused": round(ums / ms_per_step, 3),
                                "note": "torch autograd of the same gradients from saved activations (2 GEMMs)"}
    if not args.no_cpu_baseline:
        import oracle

        rng = np.random.default_rng(0)
        Wp_ref = oracle.fold_bf16(inp["W_t"], inp["gamma"])
        n_rows, n_js = 8, 1
        while True:
            rows = np.sort(rng.choice(M, size=min(n_rows, M), replace=False))
            js = np.sort(rng.choice(N, size=min(n_js, N), replace=False))
            t1 = time.perf_counter()
            oracle.qkv_rope_bwd(inp["h"], inp["gamma"], Wp_ref, 1.0, inp["W_t"], inp["dy"], inp["pos"],
                                w.rope_base, w.head_dim, rot, w.eps, rows=rows, js=js)
            dt = time.perf_counter() - t1
            if dt >= args.cpu_seconds / 2 or (n_rows >= M and n_js >= N):
                break
            n_rows, n_js = min(2 * n_rows, M), min(2 * n_js, N)
        done = rows.size * (2 * N * d) + js.size / N * g_flops
        rec["cpu_baseline"] = {"value": round(done / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": f"{rows.size} random rows of dh and {js.size} random rows of dW (all "
                                         f"columns) of the {M}-token workload in one oracle call (fp64), {dt:.1f} s"}
    return rec


def bench_ce_backward(w, args) -> dict:
    """Backward step of the LM-head block loss_m = CE(RMSNorm(h) . W^T, t_m) for the mean
    loss: the recomputed logits product with the loss backward in its epilogue, the row
    coefficient, the input-gradient GEMM, the weight-gradient GEMM on dz and h as stored
    (split over the tokens: dz's rows are too wide for one 32-bit addressed range) and
    the column sum for gamma.  The forward state -- folded weight and its transpose, r
    and the log-sum-exp from a forward run of the loss -- is prepared outside the timed
    region."""
    import numpy as np
    import torch

    import gemm_epilogue_transformer_amd as coda
    import synth_inputs as si

    inp = si.generate(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    h, W = dev(inp["h"]), dev(inp["W_t"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    tgt = torch.from_numpy(inp["targets"]).cuda()
    gw = torch.from_numpy(inp["g"]).cuda()
    M, d, V = w.M, w.d, w.N2w
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    Wp = coda.prepare_weight_bf16(W, gamma)
    Wpt = coda.transpose_bf16(Wp)
    r = coda.rowscale_from_h(h, w.eps)
    fp, tl = coda.gemm_rowscale_ce(h, Wp, r, tgt)
    lse, _ = coda.ce_reduce(fp, tgt, tl, V)
    del fp
    torch.cuda.synchronize()
    prep_ms = (time.perf_counter() - t0) * 1e3
    T = -(-V // 128)
    TW = coda.wgrad_partials_rows(V)
    f32 = dict(dtype=torch.float32, device="cuda")
    b16 = dict(dtype=torch.bfloat16, device="cuda")
    out = {"dz": torch.empty((M, V), **b16), "partials": torch.empty((M, T), **f32), "q": torch.empty(M, **f32),
           "dh": torch.empty((M, d), **b16), "dW": torch.empty((V, d), **f32),
           "wpartials": torch.empty((TW, d), **f32), "dgamma": torch.empty(d, **f32)}
    nws = int(coda._lib.load().coda_wgrad_tok_workspace_bytes(V, d, M, V, d))
    out["wws"] = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws > 0 else None
    stream = torch.cuda.current_stream()
    stages = [
        ("gemm_ce_bwd", "k_gemm_rowscale_swiglu",
         lambda: coda.gemm_ce_bwd(h, Wp, r, tgt, lse, gw, out["dz"], out["partials"])),
        ("rmsnorm_bwd_reduce", "k_rmsnorm_bwd_reduce",
         lambda: coda.rmsnorm_bwd_reduce(out["partials"], r, d, V, out["q"])),
        ("gemm_rmsnorm_bwd", "k_gemm_rmsnorm_bwd",
         lambda: coda.gemm_rmsnorm_bwd(out["dz"], Wpt, h, out["q"], None, out["dh"])),
        ("gemm_wgrad", "k_gemm_wgrad",
         lambda: coda.gemm_wgrad_tok(out["dz"], h, gamma, W, out["dW"], out["wpartials"], out["wws"])),
        ("colsum_reduce", "k_colsum_reduce", lambda: coda.colsum_reduce(out["wpartials"], out["dgamma"]))]
    names = [x[0] for x in stages]
    kern = [x[1] for x in stages]

    def step(ev=None):
        for i, (_, _, call) in enumerate(stages):
            if ev is not None:
                ev[i].record(stream)
            call()
        if ev is not None:
            ev[len(stages)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    k_ms = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i in range(len(names))]
    g_flops = 2 * M * d * V
    gemm_fl = {names.index("gemm_ce_bwd"): g_flops, names.index("gemm_rmsnorm_bwd"): g_flops,
               names.index("gemm_wgrad"): g_flops}
    value = w.gemm_flops / (ms_per_step * 1e-3) / 1e12
    dom = max(gemm_fl, key=lambda i: k_ms[i])
    byt = {"gemm_ce_bwd": M * d * 2 + V * d * 2 + 4 * M * 4 + M * V * 2 + M * T * 4,
           "rmsnorm_bwd_reduce": M * T * 4 + 2 * M * 4,
           "gemm_rmsnorm_bwd": M * V * 2 + d * V * 2 + M * d * 2 + M * 4 + M * d * 2,
           "gemm_wgrad": M * V * 2 + M * d * 2 + d * 4 + V * d * 2 + V * d * 4 + TW * d * 4,
           "colsum_reduce": TW * d * 4 + d * 4}
    achieved = gemm_fl[dom] / (k_ms[dom] * 1e-3) / 1e12
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "M": M, "d": d, "V": V, "loss": "mean cross-entropy",
                   "direction": "backward of the LM-head block (dh, dW, dgamma)", "eps": w.eps, "seed": w.seed},
        "note": "FLOPs of the executed GEMMs: the recomputed logits product, the input-gradient product and "
                "the weight-gradient product",
        "kernels_ms": {n: round(t, 4) for n, t in zip(names, k_ms)},
        "gemm_tflops": {names[i]: round(gemm_fl[i] / (k_ms[i] * 1e-3) / 1e12, 1) for i in gemm_fl},
        "hbm_bytes_algorithmic": {"fused": sum(byt[n] for n in names)},
        "prep_ms": round(prep_ms, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": load_traffic(w.name, kern[dom]), "kernel": kern[dom],
                     "kernel_ms": round(k_ms[dom], 4), "algorithmic_bytes": byt[names[dom]],
                     "kernel_source_hash": kernel_source_hash(kern[dom])},
        "kernel_source_hash": kernel_source_hash(),
    }
    if args.unfused:
        # torch autograd of the unfused forward (bf16 GEMM writing the logits, element-wise
        # RMSNorm, torch's cross_entropy on fp32 logits, mean) for the same gradients
        for k in ("dz", "dW", "wws"):
            out[k] = None
        torch.cuda.empty_cache()
        hh = h.clone().requires_grad_(True)
        Wl = W.clone().requires_grad_(True)
        gl = gamma.clone().requires_grad_(True)
        hf = hh.float()
        n = (hf * torch.rsqrt(hf.pow(2).mean(-1, keepdim=True) + w.eps)).to(torch.bfloat16) * gl.to(torch.bfloat16)
        z = n @ Wl.t()
        loss = torch.nn.functional.cross_entropy(z.float(), tgt.long())

        def ubwd():
            torch.autograd.grad((loss,), (hh, Wl, gl), retain_graph=True)

        for _ in range(2):
            ubwd()
        torch.cuda.synchronize()
        s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nu = max(1, min(args.steps, 10))
        s2.record(stream)
        for _ in range(nu):
            ubwd()
        e2.record(stream)
        torch.cuda.synchronize()
        ums = s2.elapsed_time(e2) / nu
        rec["unfused_torch"] = {"ms_per_step": round(ums, 4), "speedup_of_fused": round(ums / ms_per_step, 3),
                                "note": f"torch autograd of the same gradients from saved activations (2 GEMMs, "
                                        f"fp32 logits), {nu} steps"}
    if not args.no_cpu_baseline:
        import oracle

        rng = np.random.default_rng(0)
        Wp_ref = oracle.fold_bf16(inp["W_t"], inp["gamma"])
        n_rows = 2
        while True:
            rows = np.sort(rng.choice(M, size=min(n_rows, M), replace=False))
            t1 = time.perf_counter()
            oracle.lmhead_ce_bwd(inp["h"], inp["gamma"], Wp_ref, 1.0, inp["W_t"], inp["targets"], inp["g"], w.eps,
                                 rows=rows)
            dt = time.perf_counter() - t1
            if dt >= args.cpu_seconds / 2 or n_rows >= M:
                break
            n_rows *= 2
        done = rows.size * 2 * (2 * V * d)                 # the recomputed logits and dh per row
        rec["cpu_baseline"] = {"value": round(done / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": f"{rows.size} random rows of dh (their logits recomputed) of the {M}-token "
                                         f"workload in one oracle call (fp64), {dt:.1f} s; the weight gradient, "
                                         f"which needs every token's softmax, is not sampled"}
    return rec


class ClockSampler:
    """The GPU's graphics clock (MHz) from the firmware's metrics table (amdsmi gpu
    metrics: ``average_gfxclk_frequency``, and the mean over the XCDs of
    ``current_gfxclks``), sampled in a background thread while a loop runs;
    ``result()`` gives mean / min / max of the samples, or the reason none could be
    read.  (The DPM "current clock" amdsmi also reports shows the selected level, not the
    clock the chip holds under its power limit.)"""

    def __init__(self, interval_s: float = 0.005):
        import threading

        self.samples, self.cur_samples, self.error, self.handle = [], [], None, None
        self._stop = threading.Event()
        self._thread = None
        self._interval = interval_s
        try:
            import amdsmi
            import torch

            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            bus = torch.cuda.get_device_properties(0).pci_bus_id
            handles = amdsmi.amdsmi_get_processor_handles()
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # dddd:bb:dd.f
                if int(bdf.split(":")[1], 16) == bus:
                    self.handle = h
            if self.handle is None and len(handles) == 1:
                self.handle = handles[0]
            if self.handle is None:
                self.error = f"no amdsmi device on PCI bus {bus:#x}"
        except Exception as e:  # noqa: BLE001 -- a missing clock is reported, not fatal
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        avg = m.get("average_gfxclk_frequency")
        cur = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        ok = lambda v: isinstance(v, (int, float)) and 0 < v < 10000  # noqa: E731
        return (float(avg) if ok(avg) else None), (sum(cur) / len(cur) if cur else None)

    def _run(self):
        while not self._stop.is_set():
            try:
                avg, cur = self._read()
                if avg is not None:
                    self.samples.append(avg)
                if cur is not None:
                    self.cur_samples.append(cur)
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self._interval)

    def __enter__(self):
        import threading

        if self.handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def result(self) -> dict:
        import numpy as np

        out = {}
        for key, smp in (("average_gfxclk", self.samples), ("current_gfxclks_xcd_mean", self.cur_samples)):
            if smp:
                a = np.array(smp)
                # consecutive equal readings are one firmware update
                distinct = [float(v) for i, v in enumerate(smp) if i == 0 or v != smp[i - 1]]
                out[key] = {"mhz_mean": round(float(a.mean()), 1), "mhz_min": round(float(a.min()), 1),
                            "mhz_max": round(float(a.max()), 1), "samples": int(a.size),
                            "readings": [round(v, 1) for v in distinct[:12]]}
        if not out:
            return {"mhz_mean": None, "error": self.error or "no samples"}
        out["source"] = ("amdsmi gpu metrics (firmware-reported graphics clock), sampled every 5 ms during "
                         "the loop; readings below ~500 MHz are idle moments between dispatches")
        return out


def timing_stats(ms: list) -> dict:
    import numpy as np

    a = np.array(ms, dtype=np.float64)
    return {"n": int(a.size), "median_ms": round(float(np.median(a)), 4), "min_ms": round(float(a.min()), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4), "mean_ms": round(float(a.mean()), 4)}


def numerics_o1(w, inp, y_fused, y_unfused, h_fused, rows) -> dict:
    """Error of the fused chain and of the unfused torch chain against the chain as a
    model defines it (raw second weight, gamma inside RMSNorm, unrounded residual
    stream, fp64: oracle.chain_textbook), on the sampled rows.  Per output y: max and
    rms of |y - ref| / (1 + |ref|) and rms of |y - ref| / rms(ref)."""
    import numpy as np
    import torch

    import oracle

    ref = oracle.chain_textbook(inp, w.act, w.eps, rows=rows)
    dec = lambda t: oracle.bf16_decode(t.view(torch.int16).cpu().numpy().view(np.uint16))  # noqa: E731
    out = {"rows": int(rows.size), "reference": "fp64, raw second weight, gamma in RMSNorm, h unrounded"}
    yr = ref["y"]
    scale = float(np.sqrt(np.mean(yr * yr)))
    for name, y in (("fused", y_fused), ("unfused_torch", y_unfused)):
        if y is None:
            continue
        yg = dec(y)
        rel = np.abs(yg - yr) / (1 + np.abs(yr))
        out[name] = {"y_max_rel": float(f"{rel.max():.4e}"), "y_rms_rel": float(f"{np.sqrt(np.mean(rel ** 2)):.4e}"),
                     "y_rms_over_rms_ref": float(f"{np.sqrt(np.mean((yg - yr) ** 2)) / scale:.4e}")}
    if h_fused is not None:
        hr = ref["h"]
        eh = np.abs(dec(h_fused) - hr) / (1 + np.abs(hr))
        out["fused"]["h_max_rel"] = float(f"{eh.max():.4e}")
    return out


def forward_summary(w, inp, args, numerics_rows: int = 512) -> dict:
    """One forward workload (NONE or SwiGLU second GEMM), compact: each of
    ``args.stat_steps`` chains timed on its own with HIP events (median / min / p90, and
    per kernel the median), the GPU clock during that loop, the dominant kernel's
    roofline against its own dtype's dense MFMA peak, the algorithmic HBM bytes of the
    fused and the unfused chain, the unfused torch chain's time, and the O1 numerics
    diagnostic on sampled rows."""
    import numpy as np
    import torch

    import gemm_epilogue_transformer_amd as coda
    import synth_inputs as si

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    A, Wo, xr, W = dev(inp["A"]), dev(inp["Wo_t"]), dev(inp["x_res"]), dev(inp["W_t"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    if w.dtype == "bf16":
        Wp = coda.prepare_weight_bf16(W, gamma)
        a_in, wo_in, sa, so, sw = A, Wo, None, None, None
    else:
        a_in, sa2 = coda.quantize_e4m3(A)
        wo_in, so2 = coda.quantize_e4m3(Wo)
        Wp, sw2 = coda.quantize_e4m3(W, gamma)
        sa, so, sw = sa2[1:], so2[1:], sw2[1:]
    M, d = w.M, w.d
    out = {"h": torch.empty((M, d), dtype=torch.bfloat16, device="cuda"),
           "partials": torch.empty((M, coda.partials_per_row(d)), dtype=torch.float32, device="cuda"),
           "r": torch.empty(M, dtype=torch.float32, device="cuda"),
           "y": torch.empty((M, w.n_out), dtype=torch.bfloat16, device="cuda")}
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        coda.gemm_resid_partialrms(a_in, wo_in, xr, sa, so, out["h"], out["partials"])
        if ev is not None:
            ev[1].record(stream)
        coda.rowscale_reduce(out["partials"], d, w.eps, out["r"])
        if ev is not None:
            ev[2].record(stream)
        coda.gemm_rowscale_swiglu(out["h"], Wp, out["r"], w.act, sw, out["y"])
        if ev is not None:
            ev[3].record(stream)

    for _ in range(max(args.warmup, 3)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    # at least stat_steps chains, and at least a second of them (the firmware's clock
    # readings change only every few hundred ms)
    n = max(args.stat_steps, int(1.0 / max(time.perf_counter() - t0, 1e-4)))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    with ClockSampler() as clk:
        for i in range(n):
            step(evs[i])
        torch.cuda.synchronize()
    chain_ms = [e[0].elapsed_time(e[3]) for e in evs]
    k_ms = [[e[j].elapsed_time(e[j + 1]) for e in evs] for j in range(3)]
    med = [float(np.median(k)) for k in k_ms]
    g1 = 2 * M * w.K1 * d
    g2 = 2 * M * d * w.N2w
    # the first GEMM runs on the 8-bit MFMA for the e4m3 workload, the second always on bf16
    kern = [("gemm_resid_partialrms", g1, "e4m3" if w.dtype == "e4m3" else "bf16"),
            ("gemm_rowscale_swiglu", g2, "bf16")]
    dom = 0 if med[0] > med[2] else 1
    name, fl, dt = kern[dom]
    kms = med[0] if dom == 0 else med[2]
    ach = fl / (kms * 1e-3) / 1e12
    byt = algorithmic_bytes(w)
    rec = {"workload": w.name, "M": M, "K1": w.K1, "d": d, "N2w": w.N2w,
           "act": "swiglu" if w.act == si.ACT_SWIGLU else "none", "dtype": w.dtype,
           "timing": timing_stats(chain_ms),
           "tflops_median": round(w.gemm_flops / (np.median(chain_ms) * 1e-3) / 1e12, 2),
           "frac_of_bf16_peak_median": round(w.gemm_flops / (np.median(chain_ms) * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
                                             4),
           "kernels_ms_median": {"gemm_resid_partialrms": round(med[0], 4), "rowscale_reduce": round(med[1], 4),
                                 "gemm_rowscale_swiglu": round(med[2], 4)},
           "gemm1_tflops_median": round(g1 / (med[0] * 1e-3) / 1e12, 1),
           "gemm2_tflops_median": round(g2 / (med[2] * 1e-3) / 1e12, 1),
           "roofline": {"bound": "mfma", "kernel": name, "dtype": dt, "achieved": round(ach, 1),
                        "peak": PEAK_TFLOPS[dt], "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[dt], 4),
                        "kernel_ms_median": round(kms, 4)},
           "clock": clk.result(),
           "hbm_bytes_algorithmic": {"fused": byt["total"], "unfused": algorithmic_bytes(w, False)["total"]}}

    # the unfused torch chain (hipBLASLt GEMMs, element-wise residual, RMSNorm, SwiGLU),
    # on the same bf16 inputs (the 8-bit workload: its bf16 source tensors)
    def unfused():
        t = A @ Wo.t()
        hh = xr + t
        hf = hh.float()
        nn_ = (hf * torch.rsqrt(hf.pow(2).mean(-1, keepdim=True) + w.eps)).to(torch.bfloat16) \
            * gamma.to(torch.bfloat16)
        z = nn_ @ W.t()
        if w.act == si.ACT_SWIGLU:
            return torch.nn.functional.silu(z[:, : w.n_out]) * z[:, w.n_out:]
        return z

    y_unf = unfused()
    torch.cuda.synchronize()
    if w.dtype == "bf16":
        ue = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(min(n, 30))]
        for e in ue:
            e[0].record(stream)
            unfused()
            e[1].record(stream)
        torch.cuda.synchronize()
        ums = float(np.median([e[0].elapsed_time(e[1]) for e in ue]))
        rec["unfused_torch"] = {"median_ms": round(ums, 4), "speedup_of_fused": round(ums / np.median(chain_ms), 3),
                                "steps": len(ue)}
        # the vendor library's plain product of each GEMM's shape (torch.matmul on the same
        # operands, hipBLASLt on ROCm), timed alternately with the library's kernel on the
        # same machine: the GEMM-only reference the fused kernels are held against
        hbuf = out["h"]
        vend = {}
        for name, fn_ours, fn_vendor, fl in (
                ("gemm_resid_partialrms", lambda: coda.gemm_resid_partialrms(A, Wo, xr, None, None, out["h"],
                                                                             out["partials"]),
                 lambda: torch.matmul(A, Wo.t()), g1),
                ("gemm_rowscale_swiglu", lambda: coda.gemm_rowscale_swiglu(hbuf, Wp, out["r"], w.act, sw, out["y"]),
                 lambda: torch.matmul(hbuf, Wp.t()), g2)):
            ts = {"ours": [], "vendor": []}
            for _ in range(3):
                fn_ours()
                fn_vendor()
            torch.cuda.synchronize()
            for _ in range(20):
                for key, fn in (("ours", fn_ours), ("vendor", fn_vendor)):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    fn()
                    e1.record(stream)
                    ts[key].append((e0, e1))
            torch.cuda.synchronize()
            med = {k: float(np.median([a.elapsed_time(b) for a, b in v])) for k, v in ts.items()}
            vend[name] = {"ours_ms": round(med["ours"], 4), "vendor_matmul_ms": round(med["vendor"], 4),
                          "ours_tflops": round(fl / (med["ours"] * 1e-3) / 1e12, 1),
                          "vendor_tflops": round(fl / (med["vendor"] * 1e-3) / 1e12, 1)}
        vend["note"] = ("torch.matmul of the same operands (no residual, no row scale, no activation; it writes "
                        "the full [M, N2w] product), alternated with the library's kernel, 20 each, medians")
        rec["vendor_gemm"] = vend
    if numerics_rows > 0:
        rng = np.random.default_rng(w.seed)
        rows = np.sort(rng.choice(M, size=min(numerics_rows, M), replace=False))
        sel = torch.from_numpy(rows).cuda()
        rec["numerics_o1"] = numerics_o1(w, inp, out["y"][sel], y_unf[sel], out["h"][sel], rows)
    del A, Wo, xr, W, Wp, out, y_unf
    torch.cuda.empty_cache()
    return rec


def _oracle_path(oracle, prep, inp, w, rows):
    """The oracle's whole path for the rows: the chain, then RoPE or the loss."""
    import synth_inputs as si

    act = w.act if w.act in (si.ACT_NONE, si.ACT_SWIGLU) else si.ACT_NONE
    ref = oracle.chain(prep, inp["x_res"], inp["gamma"], act, w.eps, rows=rows)
    if w.act == si.ACT_ROPE:
        oracle.rope(ref["y"], inp["pos"][rows], w.rope_base, w.head_dim, w.rot_cols)
    elif w.act == si.ACT_CE:
        oracle.cross_entropy(ref["y"], inp["targets"][rows])
    return ref


def cpu_baseline(w, inp, target_s: float, rows_all: bool = True) -> dict:
    """The oracle timed on the host cores: on every row of the workload in one call
    (rows_all), else on a random row sample grown until one call takes about target_s."""
    import numpy as np

    import oracle

    prep = oracle.prepare(inp, w.dtype)
    per_row = 2 * (w.K1 * w.d + w.d * w.N2w)
    if rows_all:
        t0 = time.perf_counter()
        _oracle_path(oracle, prep, inp, w, np.arange(w.M, dtype=np.int64))
        dt = time.perf_counter() - t0
        return {"value": round(w.M * per_row / dt / 1e12, 6), "unit": "TFLOP/s",
                "cores": oracle.max_threads(), "kind": "oracle",
                "sample": f"all {w.M} rows of the workload in one oracle call (fp64, includes its weight "
                          f"decode), {dt:.1f} s"}
    rng = np.random.default_rng(0)
    # grow the sample until one call takes >= 1/4 of the target, then size it to the target
    n, dt = 8, 0.0
    while True:
        rows = np.sort(rng.choice(w.M, size=min(n, w.M), replace=False))
        t0 = time.perf_counter()
        _oracle_path(oracle, prep, inp, w, rows)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or n >= w.M:
            break
        n *= 4
    if dt < target_s / 2 and n < w.M:
        n = int(min(w.M, n * target_s / dt))
        rows = np.sort(rng.choice(w.M, size=n, replace=False))
        t0 = time.perf_counter()
        _oracle_path(oracle, prep, inp, w, rows)
        dt = time.perf_counter() - t0
    n = rows.size
    return {"value": round(n * per_row / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{n} random rows of the {w.M}-row workload in one oracle call "
                      f"(fp64, includes its weight decode), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="workload number (1-11)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-sample", action="store_true",
                    help="time the oracle on a row sample (about --cpu-seconds) instead of every row")
    ap.add_argument("--stat-steps", type=int, default=100,
                    help="forward workloads: chains timed one by one for median / min / p90 (after the K steps)")
    ap.add_argument("--numerics-rows", type=int, default=512,
                    help="rows sampled for the numerics diagnostic against the textbook definition (0: none)")
    ap.add_argument("--no-configs", action="store_true",
                    help="workload 2: skip the summaries of workloads 3, 4 and 5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="also time the unfused torch chain")
    ap.add_argument("--graph", action="store_true",
                    help="forward workloads: also time the step replayed from a captured HIP graph")
    ap.add_argument("--saved-z", action="store_true",
                    help="backward workloads: start from the pre-activation the forward saved (no recompute)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times): the "
                         "reference for scaling HBM byte counters, then exit")
    ap.add_argument("--ingest-traffic", nargs=4, metavar="DIR",
                    help="write profiles/traffic_*.json from rocprofv3 --pmc output dirs: "
                         "FETCH_SIZE run, WRITE_SIZE run, FETCH_SIZE copy run, WRITE_SIZE copy run")
    ap.add_argument("--ingest-command", default="",
                    help="command line recorded with --ingest-traffic / --summarize-trace")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("DIR", "WORKLOAD", "BENCH_LOG"),
                    help="write profiles/kernel_trace_<WORKLOAD>.txt from a rocprofv3 --kernel-trace csv "
                         "run in DIR whose stdout (with the bench line) is BENCH_LOG")
    ap.add_argument("--vendor-probe", action="store_true",
                    help="bf16 forward workloads: after the setup run --steps rounds of (the library's first "
                         "GEMM, torch.matmul of its operands, the library's second GEMM, torch.matmul of its "
                         "operands) and exit: counter runs of it compare each kernel with the vendor GEMM of "
                         "the same shape")
    ap.add_argument("--ingest-counters", nargs="+", metavar="DIR",
                    help="write profiles/counters_<workload>.txt from rocprofv3 --pmc runs of --vendor-probe "
                         "(one directory per counter pass)")
    ap.add_argument("--traffic-probe", choices=("fused", "unfused"), default=None,
                    help="forward bf16 workloads: after the setup run exactly --steps steps of one path "
                         "(no warm-up, no timing) and exit; two such runs under rocprofv3 --pmc at two "
                         "step counts give the HBM bytes of one step by difference")
    ap.add_argument("--ingest-step-traffic", nargs=12, metavar="ARG",
                    help="write profiles/step_traffic_<workload>.json: n_small n_big, then FETCH_SIZE "
                         "small / big and WRITE_SIZE small / big run dirs of the fused probe, the same "
                         "four of the unfused probe, then the FETCH_SIZE and WRITE_SIZE copy run dirs")
    args = ap.parse_args()
    if args.ingest_counters:
        import synth_inputs as si

        ingest_counters(args.ingest_counters, si.WORKLOADS[args.workload], args.ingest_command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.ingest_command)
        return
    if args.ingest_step_traffic:
        import synth_inputs as si

        ingest_step_traffic(args.ingest_step_traffic, si.WORKLOADS[args.workload].name,
                            (args.copy_calibration or 1024) << 20, args.ingest_command)
        return
    if args.ingest_traffic:
        import synth_inputs as si

        ingest_traffic(args.ingest_traffic, si.WORKLOADS[args.workload].name + ("_saved_z" if args.saved_z else ""),
                       (args.copy_calibration or 1024) << 20, args.ingest_command)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on ONE GPU; --gpus {args.gpus} is not supported "
              "(the chain shards along tokens with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
        return

    import gemm_epilogue_transformer_amd as coda
    import synth_inputs as si

    w = si.WORKLOADS[args.workload]
    if w.act in (si.ACT_SWIGLU_BWD, si.ACT_CHAIN_BWD):
        print(json.dumps(bench_backward(w, args)), flush=True)
        return
    if w.act == si.ACT_ROPE_BWD:
        print(json.dumps(bench_rope_backward(w, args)), flush=True)
        return
    if w.act == si.ACT_CE_BWD:
        print(json.dumps(bench_ce_backward(w, args)), flush=True)
        return
    inp = si.generate(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    A, Wo, xr, W = dev(inp["A"]), dev(inp["Wo_t"]), dev(inp["x_res"]), dev(inp["W_t"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()

    # weight / activation preparation (once), timed separately
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if w.dtype == "bf16":
        Wp = coda.prepare_weight_bf16(W, gamma)
        a_in, wo_in, sa, so, sw = A, Wo, None, None, None
    else:
        a_in, sa2 = coda.quantize_e4m3(A)
        wo_in, so2 = coda.quantize_e4m3(Wo)
        Wp, sw2 = coda.quantize_e4m3(W, gamma)
        sa, so, sw = sa2[1:], so2[1:], sw2[1:]
    torch.cuda.synchronize()
    prep_ms = (time.perf_counter() - t0) * 1e3

    ce_in = None
    if w.act == si.ACT_CE:
        T_ce = coda.ce_partials_per_row(w.N2w)
        ce_in = {"targets": torch.from_numpy(inp["targets"]).cuda(),
                 "partials": torch.empty((w.M, T_ce, 2), dtype=torch.float32, device="cuda"),
                 "tgt": torch.empty(w.M, dtype=torch.float32, device="cuda"),
                 "lse": torch.empty(w.M, dtype=torch.float32, device="cuda"),
                 "loss": torch.empty(w.M, dtype=torch.float32, device="cuda")}
    rope_in = None
    if w.act == si.ACT_ROPE:              # angle table and positions: once, like the weights
        cos_t, sin_t = coda.rope_table(w.seq_len, w.rope_base)
        rope_in = (torch.from_numpy(inp["pos"]).cuda(), cos_t, sin_t)
        torch.cuda.synchronize()

    M, d = w.M, w.d
    out = {"h": torch.empty((M, d), dtype=torch.bfloat16, device="cuda"),
           "partials": torch.empty((M, coda.partials_per_row(d)), dtype=torch.float32, device="cuda"),
           "r": torch.empty(M, dtype=torch.float32, device="cuda"),
           "y": None if ce_in else torch.empty((M, w.n_out), dtype=torch.bfloat16, device="cuda")}
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        h, P = coda.gemm_resid_partialrms(a_in, wo_in, xr, sa, so, out["h"], out["partials"])
        if ev is not None:
            ev[1].record(stream)
        r = coda.rowscale_reduce(P, d, w.eps, out["r"])
        if ev is not None:
            ev[2].record(stream)
        if ce_in is not None:
            coda.gemm_rowscale_ce(h, Wp, r, ce_in["targets"], sw, ce_in["partials"], ce_in["tgt"])
        elif rope_in is None:
            coda.gemm_rowscale_swiglu(h, Wp, r, w.act, sw, out["y"])
        else:
            coda.gemm_rowscale_rope(h, Wp, r, *rope_in, w.rot_cols, sw, out["y"])
        if ev is not None:
            ev[3].record(stream)
        if ce_in is not None:
            coda.ce_reduce(ce_in["partials"], ce_in["targets"], ce_in["tgt"], w.N2w, ce_in["lse"], ce_in["loss"])
            if ev is not None:
                ev[4].record(stream)

    # the unfused chain in torch (hipBLASLt GEMMs, element-wise RMSNorm / activation kernels)
    def unfused():
        t = A @ Wo.t()
        hh = xr + t
        hf = hh.float()
        n = (hf * torch.rsqrt(hf.pow(2).mean(-1, keepdim=True) + w.eps)).to(torch.bfloat16) \
            * gamma.to(torch.bfloat16)
        z = n @ W.t()
        if w.act == si.ACT_SWIGLU:
            F_ = w.n_out
            return torch.nn.functional.silu(z[:, :F_]) * z[:, F_:]
        if w.act == si.ACT_CE:
            return torch.nn.functional.cross_entropy(z.float(), ce_in["targets"].long(), reduction="none")
        if w.act == si.ACT_ROPE:
            pos_t, cos_t, sin_t = rope_in
            q = z[:, : w.rot_cols].view(M, -1, 64)
            c, s_ = cos_t[pos_t].unsqueeze(1), sin_t[pos_t].unsqueeze(1)
            x1, x2 = q[..., :32], q[..., 32:]
            rq = torch.cat([x1 * c - x2 * s_, x2 * c + x1 * s_], -1).to(torch.bfloat16)
            return torch.cat([rq.view(M, -1), z[:, w.rot_cols:]], 1)
        return z

    if args.vendor_probe:
        if w.dtype != "bf16" or w.act not in (si.ACT_NONE, si.ACT_SWIGLU):
            print("bench.py: --vendor-probe covers the bf16 forward workloads", file=sys.stderr)
            sys.exit(2)
        hbuf = out["h"]
        coda.gemm_resid_partialrms(A, Wo, xr, None, None, hbuf, out["partials"])
        coda.rowscale_reduce(out["partials"], d, w.eps, out["r"])
        for _ in range(args.steps):
            coda.gemm_resid_partialrms(A, Wo, xr, None, None, hbuf, out["partials"])
            torch.matmul(A, Wo.t())
            coda.gemm_rowscale_swiglu(hbuf, Wp, out["r"], w.act, None, out["y"])
            torch.matmul(hbuf, Wp.t())
        torch.cuda.synchronize()
        print(json.dumps({"vendor_probe": w.name, "rounds": args.steps}), flush=True)
        return

    if args.traffic_probe:
        if w.dtype != "bf16":
            print("bench.py: --traffic-probe covers the bf16 workloads", file=sys.stderr)
            sys.exit(2)
        run = step if args.traffic_probe == "fused" else unfused
        for _ in range(args.steps):
            run()
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": args.traffic_probe, "workload": w.name, "steps": args.steps}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K chains, per-kernel HIP events on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    k1_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    k2_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    k3_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    k4_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in evs])) if ce_in is not None else None

    # the same step captured once in a HIP graph and replayed K times (no per-kernel
    # events inside): what a launch-bound caller would run
    graph_ms = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g, stream=gs):
                step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        gstart, gend = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gstart.record(stream)
        for _ in range(args.steps):
            g.replay()
        gend.record(stream)
        torch.cuda.synchronize()
        graph_ms = gstart.elapsed_time(gend) / args.steps

    flops = w.gemm_flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    g1_flops = 2 * M * w.K1 * d
    g2_flops = 2 * M * d * w.N2w
    k2_dtype = "bf16"  # the second GEMM runs on the bf16 MFMA (8-bit weights decoded exactly)
    achieved = g2_flops / (k3_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[k2_dtype]
    byt = algorithmic_bytes(w)
    # on bf16 weights the library runs the forward SwiGLU and the plain row-scaled product
    # as persistent kernels whose epilogues overlap the next tile's first k-tile when K
    # spans more than 2 k-tiles (the SwiGLU one in a plain persistent form below that)
    if w.dtype == "bf16" and w.act in (si.ACT_SWIGLU, si.ACT_NONE) and d > 128:
        k3_name = "k_gemm_rowscale_ovl"
    elif w.dtype == "bf16" and w.act == si.ACT_SWIGLU:
        k3_name = "k_gemm_swiglu_persistent"
    else:
        k3_name = "k_gemm_rowscale_swiglu"
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": load_traffic(w.name, k3_name),
            "kernel": k3_name, "kernel_ms": round(k3_ms, 4),
            "algorithmic_bytes": byt["gemm2"], "kernel_source_hash": kernel_source_hash(k3_name)}

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "e4m3/bf16", "data": "synthetic",
        "config": {"workload": w.name, "M": M, "K1": w.K1, "d": d, "N2w": w.N2w,
                   "act": {si.ACT_SWIGLU: "swiglu", si.ACT_ROPE: "rope", si.ACT_CE: "cross_entropy"}.get(
                       w.act, "none"), "eps": w.eps,
                   "seed": w.seed, **({"rot_cols": w.rot_cols, "seq_len": w.seq_len, "rope_base": w.rope_base}
                                      if w.act == si.ACT_ROPE else {})},
        "frac_of_peak_chain": round(value / PEAK_TFLOPS["bf16"], 4),
        "kernels_ms": {"gemm_resid_partialrms": round(k1_ms, 4), "rowscale_reduce": round(k2_ms, 4),
                       "gemm_rowscale_swiglu": round(k3_ms, 4),
                       **({"ce_reduce": round(k4_ms, 4)} if k4_ms is not None else {})},
        "gemm1_tflops": round(g1_flops / (k1_ms * 1e-3) / 1e12, 2),
        "hbm_bytes_algorithmic": {"fused": byt["total"], "unfused": algorithmic_bytes(w, False)["total"]},
        "hbm_bytes_measured": load_step_traffic(w.name),
        "prep_ms": round(prep_ms, 3),
        "roofline": roof,
        "kernel_source_hash": kernel_source_hash(),
    }

    if graph_ms is not None:
        rec["graph"] = {"ms_per_step": round(graph_ms, 4), "value": round(flops / (graph_ms * 1e-3) / 1e12, 2),
                        "note": "the same step replayed from a captured HIP graph"}
    if args.unfused and w.dtype == "bf16":
        for _ in range(3):
            unfused()
        torch.cuda.synchronize()
        s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s2.record(stream)
        for _ in range(args.steps):
            unfused()
        e2.record(stream)
        torch.cuda.synchronize()
        ums = s2.elapsed_time(e2) / args.steps
        rec["unfused_torch"] = {"ms_per_step": round(ums, 4),
                                "tflops": round(flops / (ums * 1e-3) / 1e12, 2),
                                "speedup_of_fused": round(ums / ms_per_step, 3)}

    if w.act in (si.ACT_NONE, si.ACT_SWIGLU) and args.stat_steps > 0:
        # the same workload, each chain timed on its own, with the clock and the numerics
        # diagnostic; then (default workload) the other 16K-token forward configurations
        del out
        torch.cuda.empty_cache()
        summ = forward_summary(w, inp, args, args.numerics_rows)
        for k in ("timing", "clock", "numerics_o1", "kernels_ms_median", "vendor_gemm"):
            if k in summ:
                rec[k] = summ[k]
        if "unfused_torch" in summ:
            rec.setdefault("unfused_torch", summ["unfused_torch"])
        if args.workload == 2 and not args.no_configs:
            rec["configs"] = {}
            for c in (3, 4, 5):
                wc = si.WORKLOADS[c]
                print(f"bench.py: summary of workload {c} ({wc.name})", file=sys.stderr, flush=True)
                inp_c = inp if (wc.seed == w.seed and wc.M == w.M and wc.K1 == w.K1 and wc.d == w.d
                                and wc.N2w == w.N2w) else si.generate(wc)
                rec["configs"][wc.name] = forward_summary(wc, inp_c, args, args.numerics_rows)
                del inp_c

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, rows_all=not args.cpu_sample)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
