#!/usr/bin/env python3
"""Throughput of the MoE-layer forward pass on one MI355X (gfx950).

A step is one whole layer: route, dispatch, grouped gate/up GEMM with the
SwiGLU epilogue, grouped down GEMM (routed and shared experts), combine, with
inputs already resident in HBM.  After an untimed device warm-up of at least
0.5 s (the GPU's clocks ramp up after the host-side set-up), it is timed in
three passes of the same number of steps:
- all on one stream through ``moe_layer_fwd``, called directly and, as a
  second timing, recorded once into a HIP graph and replayed;
- with the shared experts on a second stream through ``moe_layer_fwd_overlap``
  (only for layers that have shared experts);
- on one stream through ``moe_layer_fwd_timed``, which records HIP events
  between the stages.
``value`` is the fastest of the uninstrumented timings (direct, graph replay,
second stream); all are reported.  For workloads with duplicated rows (or with
``--condense COS``) a fourth pass times ``moe_layer_fwd_condensed``, token
condensation, an approximation of the layer: it is reported under
``condensed`` with the rows it keeps, never as ``value``.  The default
workload is the largest one-GPU configuration, the prefill-scale layer
(T=32768 tokens as 8 sequences of 4096, d=2048, 64 experts top-6 + 2 shared,
I=1408, 30% near-duplicate token rows), bf16 inputs with fp32 accumulation,
synthetic seeded data.  The DeepSeek-V2-Lite-shaped layer (T=4096, same
experts) is timed too, more briefly, under ``other_workloads`` (``--also``).

Prints one JSON line.  Per-stage times come from the third pass: HIP events
that the library records on the layer's stream between its kernels, averaged
over its timed steps.  ``cold`` times the layer again with a 1 GiB write
between calls (no input left in the 256 MB MALL); ``grouped_roofline`` is each
GEMM launch's ideal time, the sum over experts of max(FLOP / bf16 peak, bytes /
HBM peak) for this input's expert loads, and its fraction of the measured
time.  The oracle (fp64 NumPy on the host cores) is timed on a bounded token
sample of the same workload as a CPU baseline.
"""
import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + grouped-GEMM % bf16 MFMA peak, 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
STAGES = ("route", "dispatch", "gate_up", "down", "combine")
GATE_UP_KERNEL = "grouped_gemm_bf16_kernel<true, true, false>"  # gate/up, buffer-load variant
PROFILES = os.path.join(ROOT, "profiles")
# sources of the gate/up kernel: a change to any of them voids stored counter readings
GEMM_SOURCES = ("gemm_bf16.hip", "grouped_gemm.h", "kernels.h", "common.h")


def gemm_source_sha():
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "expert_routing_grouped_route_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_summary_path(workload):
    return os.path.join(PROFILES, f"hbm_traffic_gate_up_{workload}.md")


def load_traffic(workload):
    """HBM bytes per gate/up launch from the committed counter summary; None
    when there is none or it was taken on other kernel sources."""
    path = traffic_summary_path(workload)
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha") != gemm_source_sha():
        return None
    return rec["traffic_bytes_per_launch"]


def _dispatches(csv_path, counter):
    """[(dispatch id, kernel name, value)] of one counter in a rocprofv3 counter CSV."""
    out = []
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(out)


def summarize_pmc(fetch_csv, write_csv, copy_mib, workload, command):
    """Write the HBM-traffic summary of the gate/up kernel from a FETCH_SIZE and
    a WRITE_SIZE run (KiB per dispatch), each scaled by what the same counter
    reads for the plain device copy of copy_mib MiB at the end of the run."""
    rec = {"kernel": GATE_UP_KERNEL, "workload": workload, "kernel_source_sha": gemm_source_sha(),
           "copy_calibration_mib": copy_mib}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _dispatches(path, name)
        gu = [v for _, k, v in rows if GATE_UP_KERNEL in k]
        last_moe = max(i for i, k, _ in rows if "moe" in k)
        cp = sum(v for i, k, v in rows if i > last_moe and "copyBuffer" in k)
        scale = copy_mib * 1024.0 / cp
        rec[name] = {"kib_per_launch": sum(gu) / len(gu), "launches": len(gu),
                     "copy_kib": cp, "scale": scale}
    rec["traffic_bytes_per_launch"] = round(
        (rec["FETCH_SIZE"]["kib_per_launch"] * rec["FETCH_SIZE"]["scale"] +
         rec["WRITE_SIZE"]["kib_per_launch"] * rec["WRITE_SIZE"]["scale"]) * 1024)
    path = traffic_summary_path(workload)
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of the gate/up grouped GEMM, {workload}\n\n")
        fh.write("Commands (one counter per run, from the repository root):\n\n")
        for c in command:
            fh.write(f"    {c}\n")
        fh.write("\nFETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by "
                 f"(copy size) / (the counter's reading for the {copy_mib} MiB device copy "
                 "at the end of the run).\n\n")
        fh.write("```json\n" + json.dumps(rec, indent=1) + "\n```\n")
    print(path)


# kernels of the layer path by role (regular expressions on demangled names)
KERNEL_ROLES = (
    ("route", r"route_bf16_kernel|route_resident_bf16_kernel|route_f32_kernel"),
    ("dispatch_count", r"dispatch_count_kernel"),
    ("dispatch_rank", r"dispatch_rank_kernel"),
    ("row_scatter", r"scatter_rows_kernel"),
    ("gate_up", r"grouped_gemm_bf16_kernel<true"),
    ("down", r"grouped_gemm_bf16_kernel<false"),
    ("combine", r"combine_k_kernel|combine_kernel"),
)
SIMD_NUM = 1024  # MI355X: 256 CUs x 4 SIMDs


def kernel_role(name):
    for role, rx in KERNEL_ROLES:
        if re.search(rx, name):
            return role
    return None


def algorithmic_bytes(cfg, counts):
    """(read, write) bytes each kernel of the layer path has to move at the
    least: every input it needs read once, every output written once.  The
    gate/up kernel reads each routed assignment's token row once (R rows) and
    only the weights of experts that received tokens; the gather (standalone
    dispatch) reads x once, with the ids and inv_perm."""
    es = 2 if cfg.dtype == "bf16" else 4
    T, d, E, k, I, ns, Is = cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.I_shared
    R = T * k
    nz = int(sum(1 for c in counts if c > 0))
    return {
        "route": (T * d * es + E * d * es + E * 4, R * 8),
        "dispatch_count": (R * 4, 0),
        "dispatch_rank": (R * 4, R * 8 + (2 * E + 1) * 4),
        "row_scatter": (T * d * es + R * 8, R * d * es),
        "gate_up": (nz * 2 * I * d * es + ns * 2 * Is * d * es + R * d * es + (T * d * es if ns else 0),
                    R * I * es + T * ns * Is * es),
        "down": (nz * d * I * es + ns * d * Is * es + R * I * es + T * ns * Is * es,
                 R * d * 4 + (T * d * 4 if ns else 0)),
        "combine": (R * d * 4 + R * 8 + (T * d * 4 if ns else 0), T * d * 4),
    }


def _counter_rows(csv_path):
    with open(csv_path) as fh:
        return list(csv.DictReader(fh))


def summarize_counters(trace_csv, counter_csvs, bench_log, copy_mib, workload, command):
    """Per-kernel table of the layer path from one kernel-trace run and
    counter runs (rocprofv3 CSV): average duration (trace), HBM-side bytes
    from FETCH_SIZE and WRITE_SIZE (KiB per dispatch, each scaled by what it
    reads for the copy_mib MiB device copy at the end of its run) against the
    algorithmic bytes, the MFMA utilisation (MfmaUtil: MFMA-busy cycles over
    GUI-active cycles x SIMDs), the MFMA work executed (bf16 MOPS x 512) and
    the clock (GUI-active cycles over the traced duration).  Writes
    profiles/counters_<workload>.md."""
    import moe_synth
    cfg = moe_synth.CONFIGS[workload]
    info = None
    for line in open(bench_log):
        if line.startswith("{"):
            info = json.loads(line)
    counts = info["counts"]
    last = int(info["profile_steps"])  # the profiled calls: the last ones of each kernel
    alg = algorithmic_bytes(cfg, counts)
    fl_gu, fl_dn = gemm_flops(cfg)
    flops = {"gate_up": fl_gu, "down": fl_dn}
    # durations per role from the kernel trace
    dur = {}
    for r in _counter_rows(trace_csv):
        role = kernel_role(r["Kernel_Name"])
        if role:
            dur.setdefault(role, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    vals = {}   # role -> counter -> [per-dispatch values]
    cdur = {}   # role -> [duration of each dispatch in the counter runs]
    copy = {}   # counter -> KiB read for the calibration copy
    for path in counter_csvs:
        rows = _counter_rows(path)
        last_id = max((int(r["Dispatch_Id"]) for r in rows if kernel_role(r["Kernel_Name"])), default=-1)
        for r in rows:
            role = kernel_role(r["Kernel_Name"])
            name, v = r["Counter_Name"], float(r["Counter_Value"])
            if role:
                vals.setdefault(role, {}).setdefault(name, []).append(v)
                if name == "GRBM_GUI_ACTIVE":
                    cdur.setdefault(role, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            elif "copyBuffer" in r["Kernel_Name"] and int(r["Dispatch_Id"]) > last_id:
                copy[name] = copy.get(name, 0.0) + v
    scale = {n: copy_mib * 1024.0 / copy[n] for n in ("FETCH_SIZE", "WRITE_SIZE") if copy.get(n)}
    mean = lambda xs: sum(xs[-last:]) / len(xs[-last:])
    table = {}
    for role, _ in KERNEL_ROLES:
        if role not in dur:
            continue
        us = mean(dur[role]) / 1e3
        c = {n: mean(v) for n, v in vals.get(role, {}).items()}
        rd, wr = alg[role]
        e = {"calls": min(last, len(dur[role])), "avg_us": round(us, 2),
             "alg_read_MB": round(rd / 1e6, 2), "alg_write_MB": round(wr / 1e6, 2),
             "alg_GB/s": round((rd + wr) / (us * 1e-6) / 1e9, 1)}
        if "FETCH_SIZE" in c and "FETCH_SIZE" in scale:
            f = c["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
            e["fetch_MB"] = round(f / 1e6, 2)
            e["fetch_over_alg_read"] = round(f / rd, 3) if rd else None
        if "WRITE_SIZE" in c and "WRITE_SIZE" in scale:
            w = c["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
            e["write_MB"] = round(w / 1e6, 2)
            e["write_over_alg_write"] = round(w / wr, 3) if wr else None
        if "fetch_MB" in e and "write_MB" in e:
            e["traffic_GB/s"] = round((e["fetch_MB"] + e["write_MB"]) * 1e6 / (us * 1e-6) / 1e9, 1)
        if "MfmaUtil" in c:
            e["mfma_util_pct"] = round(c["MfmaUtil"], 1)
        if "GRBM_GUI_ACTIVE" in c and role in cdur and us > 100:  # summed over the 8 XCDs
            e["clock_GHz"] = round(c["GRBM_GUI_ACTIVE"] / 8 / mean(cdur[role]), 3)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c and role in flops:
            ex = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            e["mfma_flop_executed_over_alg"] = round(ex / flops[role], 3)
        if role in flops:
            e["alg_TFLOP/s"] = round(flops[role] / (us * 1e-6) / 1e12, 1)
            e["frac_bf16_peak"] = round(flops[role] / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)
        for n in ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY",
                  "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "TCC_HIT_sum", "TCC_MISS_sum",
                  "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_DRAM_sum"):
            if n in c:
                e[n] = c[n]
        table[role] = e
    rec = {"workload": workload, "copy_calibration_mib": copy_mib, "scale": scale,
           "kernel_source_sha": gemm_source_sha(), "kernels": table}
    path = os.path.join(PROFILES, f"counters_{workload}.md")
    with open(path, "w") as fh:
        fh.write(f"# Counters of the layer path, {workload}\n\n")
        fh.write("Commands (from the repository root; one counter set per run):\n\n")
        for cmd in command:
            fh.write(f"    {cmd}\n")
        fh.write("\nDurations from the kernel trace. FETCH_SIZE and WRITE_SIZE (KiB per dispatch) "
                 "are scaled by the copy size over what each counter reads for the "
                 f"{copy_mib} MiB device copy at the end of its run; `alg` bytes are what the "
                 "kernel has to move at the least. MfmaUtil is MFMA-busy cycles over "
                 "GUI-active cycles times the 1024 SIMDs; clock = GUI-active cycles (summed over the 8 XCDs) / 8 / the dispatch's duration in the same counter run (kernels over 100 us only).\n\n")
        cols = ["calls", "avg_us", "alg_read_MB", "fetch_MB", "fetch_over_alg_read", "alg_write_MB",
                "write_MB", "alg_GB/s", "traffic_GB/s", "mfma_util_pct", "clock_GHz",
                "frac_bf16_peak", "mfma_flop_executed_over_alg"]
        fh.write("| kernel | " + " | ".join(cols) + " |\n|" + "---|" * (len(cols) + 1) + "\n")
        for role, e in table.items():
            fh.write(f"| {role} | " + " | ".join(str(e.get(k_, "")) for k_ in cols) + " |\n")
        fh.write("\n```json\n" + json.dumps(rec, indent=1) + "\n```\n")
    print(path)


def kernel_label(name, limit=120):
    """Demangled kernel name without return type, anonymous namespace and
    arguments, cut to `limit` characters."""
    name = re.sub(r"^void ", "", name).replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(name):  # cut at the argument list (first '(' outside template brackets)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            name = name[:i]
            break
    return name if len(name) <= limit else name[:limit] + "..."


def summarize_trace(trace_csv, workload, command, bench_log=None):
    """Kernel time from a rocprofv3 --kernel-trace CSV of a bench.py run,
    grouped by kernel and grid size (so the launches of the headline workload
    and of the other workloads timed in the same run stay apart): calls,
    average and total time, share.  With the run's JSON line (bench_log), the
    same run's HIP-event stage times and roofline are appended for comparison.
    Writes profiles/kernels_<workload>.md."""
    groups = {}
    for r in _counter_rows(trace_csv):
        key = (kernel_label(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    total = sum(sum(v) for v in groups.values())
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    path = os.path.join(PROFILES, f"kernels_{workload}.md")
    with open(path, "w") as fh:
        fh.write(f"# Kernel time, bench.py run on {workload} (rocprofv3 --kernel-trace)\n\n")
        fh.write("Command (from the repository root):\n\n")
        for c in command:
            fh.write(f"    {c}\n")
        fh.write("\nEvery launch of the run (warm-up, the timed passes, the other workloads, the "
                 "backward pass), grouped by kernel and grid (workgroups).\n\n")
        fh.write("| kernel | workgroups | calls | average us | total ms | share |\n|---|---|---|---|---|---|\n")
        for (name, grid), d in rows:
            if sum(d) < 1e-4 * total:
                continue
            fh.write(f"| `{name}` | {grid} | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | "
                     f"{sum(d) / 1e6:.3f} | {100.0 * sum(d) / total:.1f}% |\n")
        if bench_log:
            for line in open(bench_log):
                if line.startswith("{"):
                    rec = json.loads(line)
                    fh.write("\nThe same run's JSON line: HIP-event stage times (ms per layer call) " +
                             ", ".join(f"{k} {v}" for k, v in rec["stages_ms"].items()) +
                             f"; roofline kernel `{rec['roofline']['kernel']}` average launch "
                             f"{rec['roofline']['avg_launch_ms']} ms, {rec['roofline']['achieved']} "
                             f"TFLOP/s.\n")
    print(path)


def summarize_stats(stats_csv, workload, command, bench_log=None, part="layer"):
    """Write the rocprofv3 --stats kernel summary (name, calls, average and total
    time), with the stage times that bench.py measured with HIP events in the
    same profiled run when its log is given.  part "backward" names the summary
    of a run that also timed the backward pass."""
    rows = list(csv.DictReader(open(stats_csv)))
    name = f"kernels_{workload}.md" if part == "layer" else f"kernels_{part}_{workload}.md"
    path = os.path.join(PROFILES, name)
    with open(path, "w") as fh:
        fh.write(f"# Kernel time, {workload} {part} (rocprofv3 --kernel-trace --stats)\n\n")
        fh.write("Command (from the repository root):\n\n")
        for c in command:
            fh.write(f"    {c}\n")
        fh.write("\n| kernel | calls | average us | total ms | share |\n|---|---|---|---|---|\n")
        for r in rows:
            fh.write(f"| `{kernel_label(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f}% |\n")
        if bench_log:
            for line in open(bench_log):
                if line.startswith("{"):
                    rec = json.loads(line)
                    fh.write("\nThe same profiled run's HIP-event stage times (ms per layer call, "
                             "averaged over the timed steps): " +
                             ", ".join(f"{k} {v}" for k, v in rec["stages_ms"].items()) + ".\n")
                    if part == "backward" and rec.get("backward"):
                        b = rec["backward"]
                        fh.write(f"\nBackward pass (moe_layer_bwd, HIP events over {b['calls_timed']} "
                                 f"calls): {b['ms']} ms per call, {b['roofline']['achieved']} "
                                 f"TFLOP/s of algorithmic work.\n")
    print(path)


def stage_bytes(cfg):
    """Algorithmic HBM bytes of the bandwidth-bound stages of the layer path.

    In moe_layer_fwd the row gather of x is part of the gate/up GEMM's operand
    loads, so the dispatch kernels move index data only: the ids in, perm and
    inv_perm out (the standalone moe_dispatch also writes x_sorted)."""
    es = 2 if cfg.dtype == "bf16" else 4
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    R = T * k
    return {
        # x and W_r read, bias read, ids and weights written
        "route": T * d * es + E * d * es + E * 4 + R * 8,
        # ids read, perm and inv_perm written, counts and offsets written
        "dispatch": R * 4 + 2 * R * 4 + (2 * E + 1) * 4,
        # y_sorted gathered, inv_perm and weights read, shared output read, out written
        "combine": R * d * 4 + R * 8 + (T * d * 4 if cfg.n_shared else 0) + T * d * 4,
    }


def gather_dispatch_bytes(cfg):
    """Algorithmic bytes of the standalone dispatch: x and the ids read, every
    assignment's row written to x_sorted, perm and inv_perm written."""
    es = 2 if cfg.dtype == "bf16" else 4
    R = cfg.T * cfg.k
    return cfg.T * cfg.d * es + R * 4 + R * cfg.d * es + 2 * R * 4


PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector peak (packed FMA: 2 per lane per clock)
# without packed fp32 instructions (not generated here): 256 CUs x 64 lanes x
# one FMA (2 FLOP) per lane per clock x 2.4 GHz
PEAK_FP32_UNPACKED_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12


def backward_flops(cfg):
    """FLOPs of the backward pass.  Algorithmic: the gradient products of the
    experts (dA, dW_down, dW_gate and dW_up, dx: 12 d I per routed row and
    12 d n_s I_s per token); executed adds the recomputed forward products
    G and U (4 d I per row).  The hi/lo parts of fp32 operands are not
    counted."""
    rows = cfg.T * cfg.k * cfg.d * cfg.I + cfg.T * cfg.d * cfg.n_shared * cfg.I_shared
    return 12 * rows, 16 * rows


def time_backward(cfg, dev, d, wdt, stream, warm=2, timed=5):
    import torch

    import expert_routing_grouped_route_amd as moe

    f = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")
    g = dict(dx=f(cfg.T, cfg.d), dw_router=f(cfg.E, cfg.d), dbias=f(cfg.E),
             dw_gate=f(cfg.E, cfg.I, cfg.d), dw_up=f(cfg.E, cfg.I, cfg.d),
             dw_down=f(cfg.E, cfg.d, cfg.I))
    sh = cfg.n_shared > 0
    g["dwsh_gate"] = f(cfg.n_shared, cfg.I_shared, cfg.d) if sh else None
    g["dwsh_up"] = f(cfg.n_shared, cfg.I_shared, cfg.d) if sh else None
    g["dwsh_down"] = f(cfg.n_shared, cfg.d, cfg.I_shared) if sh else None
    wsb = moe.moe_backward_workspace_bytes(d)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    dout = torch.randn(cfg.T, cfg.d, generator=torch.Generator(device="cuda").manual_seed(cfg.seed),
                       device="cuda", dtype=torch.float32)

    def call(variant=0):
        args = (d, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"],
                dev["w_down"], dev["wsh_gate"], dev["wsh_up"], dev["wsh_down"], dout, g["dx"],
                g["dw_router"], g["dbias"], g["dw_gate"], g["dw_up"], g["dw_down"],
                g["dwsh_gate"], g["dwsh_up"], g["dwsh_down"], ws, wsb)
        if variant:
            moe.moe_layer_bwd_variant(*args, variant, stream)
        else:
            moe.moe_layer_bwd(*args, stream)

    def timed_ms(variant=0):
        for _ in range(warm):
            call(variant)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(timed)]
        for a_, b_ in ev:
            a_.record(stream)
            call(variant)
            b_.record(stream)
        torch.cuda.synchronize()
        return sum(a_.elapsed_time(b_) for a_, b_ in ev) / timed

    print(f"[bench] timing {timed} calls of the backward pass", file=sys.stderr, flush=True)
    ms = timed_ms()  # products on the matrix cores (the library's default)
    fa, fe = backward_flops(cfg)
    tf = fa / (ms * 1e-3) / 1e12
    valu = None
    if cfg.dtype == "f32":
        # fp32 layers run every product on the grouped GEMM with free strides;
        # the vector-ALU variant puts it on the VALU in fp32
        ms_valu = timed_ms(moe.MOE_VARIANT_BWD_VALU)
        tf_v = fa / (ms_valu * 1e-3) / 1e12
        valu = {"ms": round(ms_valu, 3), "achieved_tflops": round(tf_v, 2),
                "frac_of_unpacked_fp32_fma_peak": round(tf_v / PEAK_FP32_UNPACKED_TFLOPS, 4),
                "peak_unpacked_fma": round(PEAK_FP32_UNPACKED_TFLOPS, 1)}
    return {"entry_point": "moe_layer_bwd", "calls_timed": timed, "ms": round(ms, 3),
            "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
            "flops_algorithmic": fa, "flops_executed": fe,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "executed_tflops": round(fe / (ms * 1e-3) / 1e12, 2),
                         "note": "algorithmic FLOPs over the whole call; products on bf16 MFMA, "
                                 "each fp32 operand as bf16 hi + lo parts"},
            "vector_alu_variant": valu}


def gemm_flops(cfg):
    R = cfg.T * cfg.k
    gate_up = 4 * R * cfg.d * cfg.I + 4 * cfg.T * cfg.d * cfg.n_shared * cfg.I_shared
    down = 2 * R * cfg.d * cfg.I + 2 * cfg.T * cfg.d * cfg.n_shared * cfg.I_shared
    return gate_up, down


def grouped_roofline_ms(cfg, counts):
    """Ideal time of each grouped GEMM launch at the bf16 peak and the HBM
    peak: the sum over experts (and the shared experts) of max(FLOP / peak,
    bytes / bandwidth), with bytes = the expert's weights, its input rows and
    its output rows.  Returns (gate_up_ms, down_ms)."""
    es = 2 if cfg.dtype == "bf16" else 4
    pk, bw = PEAK_BF16_TFLOPS * 1e12, PEAK_HBM_GBS * 1e9
    groups = [(int(n), cfg.I) for n in counts if n > 0]
    if cfg.n_shared:
        groups.append((cfg.T, cfg.n_shared * cfg.I_shared))
    gu = dn = 0.0
    for n, width in groups:
        gu += max(4.0 * n * cfg.d * width / pk,
                  (2 * width * cfg.d * es + n * cfg.d * es + n * width * es) / bw)
        dn += max(2.0 * n * cfg.d * width / pk,
                  (width * cfg.d * es + n * width * es + n * cfg.d * 4) / bw)
    return gu * 1e3, dn * 1e3


def cpu_baseline(cfg, arrays, budget_s=10.0, max_runs=7):
    """Time the oracle on the first Ts tokens, doubling Ts until one run takes
    at least budget_s or covers the whole workload; when the whole workload
    takes less than budget_s, repeat it until budget_s of work is done and
    report the median run."""
    import oracle
    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))

    def run(Ts):
        t0 = time.perf_counter()
        oracle.moe_layer(arrays["x"][:Ts], arrays["w_router"], arrays["bias"], arrays["w_gate"],
                         arrays["w_up"], arrays["w_down"], cfg.k, arrays["wsh_gate"],
                         arrays["wsh_up"], arrays["wsh_down"], round_a=cfg.dtype == "bf16")
        return time.perf_counter() - t0

    Ts = min(512, cfg.T)
    with threadpool_limits(limits=cores):
        while True:
            el = run(Ts)
            if el >= budget_s or Ts >= cfg.T:
                break
            Ts = min(cfg.T, Ts * 2)
        times = [el]
        while sum(times) < budget_s and len(times) < max_runs:
            times.append(run(Ts))
    med = sorted(times)[len(times) // 2]
    return {"value": Ts / med, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {Ts} of {cfg.T} tokens, all {cfg.E} experts"
                      f"{' + shared' if cfg.n_shared else ''}, fp64 NumPy oracle; median of "
                      f"{len(times)} run(s) of {med:.2f} s",
            "cpu_model": cpu_model(), "blas": blas_info(cores)}


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_info(cores):
    """The BLAS library NumPy runs on (threadpoolctl's view, under the same
    thread limit as the timed runs)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    with threadpool_limits(limits=cores):
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    return [{"library": i.get("internal_api"), "version": i.get("version"),
             "threads": i.get("num_threads"), "architecture": i.get("architecture")}
            for i in libs]


def quick_workload(cfg, args):
    """Another workload's layer, timed more briefly than the headline one: the
    one-stream call, the two-stream call (layers with shared experts) and a
    pass with stage events, each args.warmup untimed and args.steps timed
    calls after a 0.3 s device warm-up.  Reports the faster uninstrumented
    timing, the stage times, the gate/up fraction of the bf16 peak and the
    bandwidth stages' rates over their algorithmic bytes."""
    import torch

    import expert_routing_grouped_route_amd as moe
    import moe_synth

    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    arrays = moe_synth.generate(cfg, workers=min(16, len(os.sched_getaffinity(0))))
    wdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = {n: (None if v is None else torch.from_numpy(v).to(
        torch.float32 if n == "bias" else wdt).cuda()) for n, v in arrays.items()}
    del arrays
    d = moe.dims(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.I_shared, cfg.dtype)
    ws_bytes = moe.moe_workspace_bytes(d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(cfg.T, cfg.d, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    lay = (d, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"],
           dev["wsh_gate"], dev["wsh_up"], dev["wsh_down"], out, None, None, None, None, None, ws,
           ws_bytes)
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()
    fork.record(stream)
    join.record(stream)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for ev in events:
        for e in ev:
            e.record(stream)

    def passes(label, fn):
        for _ in range(args.warmup):
            fn(0)
        torch.cuda.synchronize()
        print(f"[bench] timing {args.steps} steps: {cfg.name} {label}", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.3:
        for _ in range(10):
            moe.moe_layer_fwd(*lay, stream)
        torch.cuda.synchronize()
    walls = {"single_stream": passes("moe_layer_fwd", lambda i: moe.moe_layer_fwd(*lay, stream))}
    if cfg.n_shared:
        walls["shared_on_second_stream"] = passes(
            "moe_layer_fwd_overlap",
            lambda i: moe.moe_layer_fwd_overlap(*lay, side, fork, join, stream))
    passes("moe_layer_fwd_timed", lambda i: moe.moe_layer_fwd_timed(
        *lay, [e.cuda_event for e in events[i]], stream))
    stage_ms = {s_: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / args.steps
                for j, s_ in enumerate(STAGES)}
    best = min(walls, key=walls.get)
    ms = walls[best] * 1e3 / args.steps
    fl_gu, fl_dn = gemm_flops(cfg)
    gu_tf = fl_gu / (stage_ms["gate_up"] * 1e-3) / 1e12
    sb = stage_bytes(cfg)
    return {"config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "top_k": cfg.k,
                       "I": cfg.I, "n_shared": cfg.n_shared, "I_shared": cfg.I_shared,
                       "dtype": cfg.dtype},
            "ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
            "value_from": best,
            "layer_variants_ms": {k_: round(v * 1e3 / args.steps, 4) for k_, v in walls.items()},
            "stages_ms": {k_: round(v, 4) for k_, v in stage_ms.items()},
            "gate_up": {"achieved_tflops": round(gu_tf, 1),
                        "frac_bf16_peak": round(gu_tf / PEAK_BF16_TFLOPS, 4)},
            "down_tflops": round(fl_dn / (stage_ms["down"] * 1e-3) / 1e12, 1),
            "hbm": {s_: {"GB/s": round(sb[s_] / (stage_ms[s_] * 1e-3) / 1e9, 1),
                         "frac_of_8TB/s": round(sb[s_] / (stage_ms[s_] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "bytes": sb[s_]} for s_ in sb}}


def profile_run(cfg, args, d, dev, wdt, out, ws, ws_bytes, stream):
    """A short run for counter collection: 0.2 s of untimed layer calls, then
    args.profile_steps calls of moe_layer_fwd and of the standalone
    moe_dispatch (row gather included), then the copy calibration if asked.
    Prints the expert counts (for the algorithmic bytes) as one JSON line."""
    import torch

    import expert_routing_grouped_route_amd as moe

    lay = (d, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"],
           dev["wsh_gate"], dev["wsh_up"], dev["wsh_down"], out)
    R = cfg.T * cfg.k
    ids = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")
    cnt = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.2:
        moe.moe_layer_fwd(*lay, ids, None, cnt, None, None, ws, ws_bytes, stream)
        torch.cuda.synchronize()
    i32 = lambda *sh: torch.empty(sh, dtype=torch.int32, device="cuda")
    d_cnt, d_off, d_perm, d_inv = i32(cfg.E), i32(cfg.E + 1), i32(R), i32(R)
    x_sorted = torch.empty(R, cfg.d, dtype=wdt, device="cuda")
    print(f"[bench] profiling {args.profile_steps} calls of moe_layer_fwd and moe_dispatch",
          file=sys.stderr, flush=True)
    for _ in range(args.profile_steps):
        moe.moe_layer_fwd(*lay, None, None, None, None, None, ws, ws_bytes, stream)
    for _ in range(args.profile_steps):
        moe.moe_dispatch(d, dev["x"], ids, d_cnt, d_off, d_perm, d_inv, x_sorted, ws, ws_bytes,
                         stream)
    torch.cuda.synchronize()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps({"workload": cfg.name, "profile_steps": args.profile_steps,
                      "counts": cnt.cpu().tolist()}), flush=True)


def main():
    import moe_synth

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_stress", choices=list(moe_synth.CONFIGS))
    ap.add_argument("--also", default="deepseek_v2_lite",
                    help="comma-separated workloads timed briefly after the headline one "
                         "(one-stream and two-stream layer, stage events), reported under "
                         "other_workloads; empty for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--condense", type=float, default=None, metavar="COS",
                    help="also time moe_layer_fwd_condensed with this cosine threshold (the "
                         "default for workloads with duplicated rows: 0.9)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the timing of the backward pass (moe_layer_bwd)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="time only the one-stream layer (for profiling runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (HBM counter scale)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the gate/up HBM-traffic summary from two rocprofv3 counter CSVs")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="write the kernel-time summary from a rocprofv3 kernel_stats CSV")
    ap.add_argument("--bench-log", help="bench.py output of the profiled run (for --summarize-stats)")
    ap.add_argument("--summary-part", default="layer", choices=("layer", "backward"),
                    help="which summary --summarize-stats writes")
    ap.add_argument("--profile-steps", type=int, default=0, metavar="N",
                    help="profiling run: after a short warm-up, N calls of moe_layer_fwd and N "
                         "of the standalone moe_dispatch, then the copy calibration if asked; "
                         "prints the expert counts as JSON and skips every timing pass")
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="write profiles/kernels_<workload>.md from a rocprofv3 kernel-trace CSV")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="write profiles/counters_<workload>.md from a kernel-trace CSV followed "
                         "by counter-collection CSVs (needs --bench-log of the profiling run)")
    ap.add_argument("--command", action="append", default=[],
                    help="command line recorded in a summary (repeatable)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.command, args.bench_log)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:], args.bench_log,
                           args.copy_calibration_mib, args.workload, args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.copy_calibration_mib, args.workload, args.command)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.workload, args.command, args.bench_log,
                        args.summary_part)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of tokens; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import expert_routing_grouped_route_amd as moe

    moe.lib()
    torch.cuda.set_device(0)
    cfg = moe_synth.CONFIGS[args.workload]
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    arrays = moe_synth.generate(cfg, workers=min(16, len(os.sched_getaffinity(0))))
    wdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = {n: (None if v is None else torch.from_numpy(v).to(
        torch.float32 if n == "bias" else wdt).cuda()) for n, v in arrays.items()}
    d = moe.dims(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.I_shared, cfg.dtype)
    ws_bytes = moe.moe_workspace_bytes(d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(cfg.T, cfg.d, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    if args.profile_steps:
        profile_run(cfg, args, d, dev, wdt, out, ws, ws_bytes, stream)
        return

    n_ev = 6
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
              for _ in range(args.steps)]
    for step_ev in events:
        for e in step_ev:
            e.record(stream)  # creates the underlying hipEvent_t

    def step_timed(ev):
        moe.moe_layer_fwd_timed(d, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"],
                                dev["w_down"], dev["wsh_gate"], dev["wsh_up"], dev["wsh_down"], out,
                                None, None, None, None, None, ws, ws_bytes,
                                [e.cuda_event for e in ev], stream)

    def step_single(st=None):
        moe.moe_layer_fwd(d, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"],
                          dev["w_down"], dev["wsh_gate"], dev["wsh_up"], dev["wsh_down"], out,
                          None, None, None, None, None, ws, ws_bytes, stream if st is None else st)

    # the same layer with the shared experts on a second stream (moe_layer_fwd_overlap)
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()
    fork.record(stream)
    join.record(stream)

    def step_overlap():
        moe.moe_layer_fwd_overlap(d, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"],
                                  dev["w_up"], dev["w_down"], dev["wsh_gate"], dev["wsh_up"],
                                  dev["wsh_down"], out, None, None, None, None, None, ws, ws_bytes,
                                  side, fork, join, stream)

    def timed(label, fn):
        # args.warmup untimed calls, then args.steps calls between two synchronisations
        for _ in range(args.warmup):
            fn(0)
        torch.cuda.synchronize()
        print(f"[bench] timing {args.steps} steps: {label}", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # The GPU's clocks ramp up over tens of milliseconds after the host-side set-up,
    # so the passes start from a steady state: the layer runs untimed for at least
    # 0.5 s first (each pass still does its own W warm-up steps).
    print("[bench] device warm-up (0.5 s of layer calls, untimed)", file=sys.stderr, flush=True)
    n_dev_warm, t_w = 0, time.perf_counter()
    while time.perf_counter() - t_w < 0.5:
        for _ in range(10):
            step_single()
        torch.cuda.synchronize()
        n_dev_warm += 10

    # 1. the layer on one stream, no instrumentation
    wall = timed("moe_layer_fwd", lambda i: step_single())
    # 1b. the same call recorded once into a HIP graph and replayed (no launch
    #     overhead per kernel; the library records no memset and no host sync)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        step_single(cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step_single(torch.cuda.current_stream())
    torch.cuda.synchronize()
    wall_graph = timed("moe_layer_fwd, HIP graph replay", lambda i: graph.replay())

    # 2. shared experts on a second stream (only where there are shared experts:
    #    otherwise the two entry points do the same work)
    wall_overlap = float("inf")
    if not args.no_overlap and cfg.n_shared:
        wall_overlap = timed("moe_layer_fwd_overlap", lambda i: step_overlap())
    # 3. one stream with HIP events between the stages (stage times, roofline)
    wall_timed = timed("moe_layer_fwd_timed (stage events)", lambda i: step_timed(events[i]))

    # cold: each call after a 1 GiB scrub write, so that no input sits in the
    # 256 MB MALL; the layer alone is timed by its own first and last events
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    for step_ev in cold_ev:
        for e in step_ev:
            e.record(stream)
    print(f"[bench] timing {args.steps} cold steps (scrub between calls)", file=sys.stderr, flush=True)
    for i in range(args.steps):
        scrub.fill_(i & 255)
        step_timed(cold_ev[i])
    torch.cuda.synchronize()
    cold_ms = sum(ev[0].elapsed_time(ev[n_ev - 1]) for ev in cold_ev) / args.steps
    cold_stage_ms = {s_: round(sum(ev[j].elapsed_time(ev[j + 1]) for ev in cold_ev) / args.steps, 4)
                     for j, s_ in enumerate(STAGES)}
    del scrub

    # expert loads of this input, for the grouped roofline (outside every timed region)
    cnt = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    moe.moe_layer_fwd(d, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"],
                      dev["w_down"], dev["wsh_gate"], dev["wsh_up"], dev["wsh_down"], out, None,
                      None, cnt, None, None, ws, ws_bytes, stream)
    counts_np = cnt.cpu().numpy()

    # the standalone dispatch with its row gather (x_sorted written), timed by HIP events
    # on the stream it runs on; its bytes are the full dispatch of the method
    ids_t = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")
    moe.moe_layer_fwd(d, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"],
                      dev["w_down"], dev["wsh_gate"], dev["wsh_up"], dev["wsh_down"], out, ids_t,
                      None, None, None, None, ws, ws_bytes, stream)
    R = cfg.T * cfg.k
    d_cnt = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    d_off = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
    d_perm = torch.empty(R, dtype=torch.int32, device="cuda")
    d_inv = torch.empty(R, dtype=torch.int32, device="cuda")
    x_sorted = torch.empty(R, cfg.d, dtype=wdt, device="cuda")
    disp_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for _ in range(args.warmup):
        moe.moe_dispatch(d, dev["x"], ids_t, d_cnt, d_off, d_perm, d_inv, x_sorted, ws, ws_bytes,
                         stream)
    for a_, b_ in disp_ev:
        a_.record(stream)
        moe.moe_dispatch(d, dev["x"], ids_t, d_cnt, d_off, d_perm, d_inv, x_sorted, ws, ws_bytes,
                         stream)
        b_.record(stream)
    torch.cuda.synchronize()
    disp_ms = sum(a_.elapsed_time(b_) for a_, b_ in disp_ev) / args.steps
    del x_sorted

    # the layer's backward pass (moe_layer_bwd), a few calls timed by HIP events
    backward = None
    if not args.no_backward:
        backward = time_backward(cfg, dev, d, wdt, stream)

    # 4. token condensation (an approximation of the layer: reported apart, never as value)
    condensed = None
    cos_thr = args.condense if args.condense is not None else (0.9 if cfg.dup_frac > 0 else None)
    if cos_thr is not None:
        hyper = torch.from_numpy(moe_synth.condense_hyperplanes(cfg)).to(wdt).cuda()
        cws_bytes = moe.moe_condensed_workspace_bytes(d)
        cws = torch.empty(cws_bytes, dtype=torch.uint8, device="cuda")
        c_off = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")

        def step_condensed():
            moe.moe_layer_fwd_condensed(d, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"],
                                        dev["w_up"], dev["w_down"], dev["wsh_gate"], dev["wsh_up"],
                                        dev["wsh_down"], hyper, cos_thr, out, None, None, None,
                                        c_off, None, None, cws, cws_bytes, stream)

        wall_cond = timed(f"moe_layer_fwd_condensed (cos >= {cos_thr})", lambda i: step_condensed())
        rows = int(c_off[-1].item())
        condensed = {"cos_threshold": cos_thr, "ms_per_step": round(wall_cond * 1e3 / args.steps, 4),
                     "tokens_per_s": round(cfg.T / (wall_cond / args.steps), 1),
                     "rows": rows, "rows_of": cfg.T * cfg.k,
                     "rows_frac": round(rows / (cfg.T * cfg.k), 4),
                     "speedup_vs_exact": round(min(wall, wall_graph, wall_overlap) / wall_cond, 4)}

    stage_ms = {s: 0.0 for s in STAGES}
    for ev in events:
        for j, s in enumerate(STAGES):
            stage_ms[s] += ev[j].elapsed_time(ev[j + 1]) / args.steps
    def rate(w):
        return {"ms_per_step": round(w * 1e3 / args.steps, 4),
                "tokens_per_s": round(cfg.T / (w / args.steps), 1)}
    single = rate(wall)
    graphed = rate(wall_graph)
    overlap = rate(wall_overlap) if wall_overlap < float("inf") else None
    best, best_name = single, "single_stream"
    if wall_graph < wall:
        best, best_name = graphed, "single_stream_graph"
    if overlap and wall_overlap < min(wall, wall_graph):
        best, best_name = overlap, "shared_on_second_stream"
    ms_per_step = best["ms_per_step"]
    tokens_per_s = best["tokens_per_s"]

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    fl_gu, fl_dn = gemm_flops(cfg)
    grl = grouped_roofline_ms(cfg, counts_np)
    gu_s, dn_s = stage_ms["gate_up"] * 1e-3, stage_ms["down"] * 1e-3
    gu_tflops = fl_gu / gu_s / 1e12
    gemm_tflops = (fl_gu + fl_dn) / (gu_s + dn_s) / 1e12
    sb = stage_bytes(cfg)
    hbm = {s: {"GB/s": round(sb[s] / (stage_ms[s] * 1e-3) / 1e9, 1),
               "frac_of_8TB/s": round(sb[s] / (stage_ms[s] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               "bytes": sb[s]} for s in sb}
    gb = gather_dispatch_bytes(cfg)
    hbm["dispatch_with_row_gather"] = {
        "entry_point": "moe_dispatch", "ms": round(disp_ms, 4),
        "GB/s": round(gb / (disp_ms * 1e-3) / 1e9, 1),
        "frac_of_8TB/s": round(gb / (disp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bytes": gb}

    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "top_k": cfg.k,
                   "I": cfg.I, "n_shared": cfg.n_shared, "I_shared": cfg.I_shared,
                   "router_bias": cfg.bias, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": GATE_UP_KERNEL,
                     "achieved": round(gu_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic(cfg.name),
                     "flops_per_launch": fl_gu, "avg_launch_ms": round(stage_ms["gate_up"], 4)},
        "grouped_roofline": {
            "gate_up_ideal_ms": round(grl[0], 4), "down_ideal_ms": round(grl[1], 4),
            "gate_up_frac": round(grl[0] / stage_ms["gate_up"], 4),
            "down_frac": round(grl[1] / stage_ms["down"], 4)},
        "cold": {"ms_per_layer": round(cold_ms, 4), "tokens_per_s": round(cfg.T / (cold_ms * 1e-3), 1),
                 "stages_ms": cold_stage_ms},
        "grouped_gemm": {"tflops": round(gemm_tflops, 1),
                         "frac_bf16_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                         "down_tflops": round(fl_dn / dn_s / 1e12, 1)},
        "device_warmup_steps": n_dev_warm,
        "layer_variants": {"single_stream": single, "single_stream_graph": graphed,
                           "shared_on_second_stream": overlap,
                           "single_stream_with_stage_events": rate(wall_timed),
                           "value_from": best_name},
        "stages_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "condensed": condensed,
        "backward": backward,
        "hbm": hbm,
    }
    others = {}
    for name in [n for n in args.also.split(",") if n and n != cfg.name]:
        others[name] = quick_workload(moe_synth.CONFIGS[name], args)
    rec["other_workloads"] = others
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host cores", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, arrays)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
