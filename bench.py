"""SS2D forward benchmark on one MI355X.

Default workload: VMamba-T stage-1 SS2D (B=32, D=192, H=W=56, N=16, fp32), the
configuration the headline metric is quoted on.  One step = one full forward
(CrossScan + selective scan + CrossMerge) over one batch of seeded synthetic
inputs that are resident in HBM before timing starts.

Prints ONE JSON line with the throughput in state updates/s (B*4*D*L*N per step),
the roofline of the dominant kernel (measured live with HIP events on the launch
stream), achieved algorithmic HBM bandwidth, a parity check against the fp64
oracle and the oracle's own CPU throughput (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ss2d_inputs  # noqa: E402

# MI355X peaks (vendor figures: 256 CUs, 2.4 GHz, 8 TB/s HBM3E).
CUS, CLOCK_HZ = 256, 2.4e9
HBM_PEAK_GBPS = 8000.0
# FP32 VALU issue: 128 lanes/clk/CU (157.3 TFLOP/s fp32 vector = 256 CU x 2.4 GHz x 128 FMA x 2).
VALU_LANES_PER_CLK = 128
# Transcendentals run at a quarter of that rate and take the same issue slots.
TRANS_SLOTS = 4
# Minimal work of one state update: exp2(delta*A) plus 4 VALU (delta*A, du*B, h fma, y fma).
SLOTS_PER_UPDATE = 4 + TRANS_SLOTS
PEAK_UPDATES_PER_S = CUS * CLOCK_HZ * VALU_LANES_PER_CLK / SLOTS_PER_UPDATE  # 9.83e12
FP32_MFMA_PEAK = 157.3e12  # dense fp32 matrix FLOP/s

_CSRC = os.path.join("selective_scan_crossscan_amd", "csrc")
# The sources that define each profiled kernel and its launch (a counter record is
# valid while these are unchanged).
KERNEL_SOURCES = {
    "ss2d_forward_kernel": ["ss2d_kernels.h", "ss2d_plan.hip", "ss2d_f32_t16.hip", "ss2d_f32_t8.hip",
                            "ss2d_bf16_t16.hip", "ss2d_bf16_t8.hip"],
    "project_kernel": ["ss2d_kernels.h", "ss2d_project.hip"],
    "bwd_chunk_kernel": ["ss2d_kernels.h", "ss2d_backward.hip"],
    "channel_last_kernel": ["ss2d_kernels.h", "ss2d_epilogue.hip"],
}
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_PREFIX = "ss2d_forward_kernel"
# Kernels that one forward may launch besides the scan (transposes of x and of the merge plane).
STEP_KERNELS = {"ss2d_forward_kernel", "transpose_small", "transpose_planes", "project_kernel", "bwd_chunk_kernel",
                "bwd_seg_carry", "bwd_reduce_bc", "bwd_merge", "bwd_params", "channel_last_kernel"}


def traffic_file(workload: str, kernel: str = KERNEL_PREFIX) -> str:
    return os.path.join(PROFILES, f"{kernel}_{workload}_hbm_traffic.md")


def kernel_source_hash(kernel: str = "ss2d_forward_kernel") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, _CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str = KERNEL_PREFIX):
    """HBM bytes per launch of `kernel` from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, scaled by the copy-kernel calibration; None when absent or the kernel
    changed since."""
    try:
        with open(traffic_file(workload, kernel)) as f:
            text = f.read()
        m = re.search(r"```json\n(.*?)\n```", text, re.S)
        rec = json.loads(m.group(1)) if m else {}
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel) or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# The profiling commands whose output --summarize-profile turns into the text summaries under profiles/.
# Each runs from the repository root; {d} is the output folder and {c} the workload index.
PROFILE_COMMANDS = {
    "stats": "rocprofv3 --kernel-trace --stats -f csv -d {d} -o stats -- "
             "python bench.py --config {c}{x} --steps 20 --warmup 5 --no-cpu-baseline > {d}/stats_bench.json",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d {d} -o fetch -- "
             "python bench.py --config {c}{x} --steps 3 --warmup 1 --no-cpu-baseline --flush-steps 0 --no-peaks "
             "--copy-probe-mib 512",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d {d} -o write -- "
             "python bench.py --config {c}{x} --steps 3 --warmup 1 --no-cpu-baseline --flush-steps 0 --no-peaks "
             "--copy-probe-mib 512",
}
COPY_PROBE_MIB = 512

# Shader counters of the step's kernels, two passes of at most eight SQ counters each
# (one counter block per pass: the hardware takes no more).
SQ_PASSES = {
    "sq1": "SQ_WAVES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_SALU SQ_INSTS_LDS "
           "SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR",
    "sq2": "SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_WAIT_ANY SQ_WAIT_INST_LDS "
           "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INST_LEVEL_LDS",
}
SQ_COMMAND = ("rocprofv3 --pmc {counters} -f csv -d {d} -o {name} -- python bench.py --config {c}{x} --steps 3 "
              "--warmup 1 --no-cpu-baseline --flush-steps 0 --no-peaks")


def summarize_counters(folder: str, cfg: int, path: str = "scan") -> int:
    """Write the SQ-counter summary of the step's dominant kernel into profiles/: the
    instruction mix per state update and the VALU's share of the CUs' busy cycles."""
    shape = ss2d_inputs.CONFIGS[cfg]
    bwd = path == "backward"
    kernel = "bwd_chunk_kernel" if bwd else KERNEL_PREFIX
    workload = shape.name + ("_backward" if bwd else "")
    extra = " --path backward" if bwd else ""
    cmds = [SQ_COMMAND.format(counters=SQ_PASSES[n], d=folder, name=n, c=cfg, x=extra) for n in SQ_PASSES]
    vals = {}  # counter -> summed over the kernel's template instances, averaged over dispatches
    for name in SQ_PASSES:
        inst = {}
        for r in _counter_rows(folder, name):
            if _is_kernel(r["Kernel_Name"], kernel):
                inst.setdefault((r["Counter_Name"], r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        for (cn, _), v in inst.items():
            vals[cn] = vals.get(cn, 0.0) + sum(v) / len(v)
    upd = shape.updates
    lines = [f"# {kernel} — {workload} — shader counters (rocprofv3)", "",
             f"Workload: {shape}.  State updates per step: {upd:.4e}"
             + (" ((b,k,d,n,l) terms; the backward runs more work per term)." if bwd else "."), "",
             "Two counter runs, from the repository root:", "", "```", *cmds, "```", "",
             "Per step, summed over the kernel's template instances and averaged over its dispatches:", "",
             "| counter | value |", "|---|---|"]
    for cn in sorted(vals):
        lines.append(f"| {cn} | {vals[cn]:.4e} |")
    valu = vals.get("SQ_INSTS_VALU", 0.0)
    trans = vals.get("SQ_INSTS_VALU_TRANS_F32", 0.0)
    busy = vals.get("SQ_BUSY_CU_CYCLES", 0.0)
    lines += ["", "Derived:", "",
              f"* VALU instructions per state update: {valu * 64 / upd:.2f} (SQ_INSTS_VALU x 64 lanes / updates), "
              f"{trans * 64 / upd:.2f} of them transcendental (SQ_INSTS_VALU_TRANS_F32);",
              f"* LDS instructions per update: {vals.get('SQ_INSTS_LDS', 0.0) * 64 / upd:.3f}; vector memory "
              f"reads {vals.get('SQ_INSTS_VMEM_RD', 0.0) * 64 / upd:.3f}, writes "
              f"{vals.get('SQ_INSTS_VMEM_WR', 0.0) * 64 / upd:.3f};"]
    if busy > 0:
        act = vals.get("SQ_ACTIVE_INST_VALU", 0.0)
        lines.append(f"* VALU issue share of the SIMDs: SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES = {act / busy:.3f}. "
                     "SQ_ACTIVE_INST_VALU counts 4-cycle units (one per wave64 VALU instruction, two per "
                     f"transcendental: here {act / max(valu + trans, 1.0):.3f} of SQ_INSTS_VALU + "
                     "SQ_INSTS_VALU_TRANS_F32), summed over the waves; SQ_BUSY_CU_CYCLES counts cycles summed "
                     "over the CUs, so the ratio is the fraction of the four SIMDs' cycles spent issuing VALU "
                     "instructions;")
    if vals.get("SQ_LDS_IDX_ACTIVE", 0.0) > 0:
        lines.append(f"* LDS bank-conflict cycles per LDS-active cycle: "
                     f"{vals.get('SQ_LDS_BANK_CONFLICT', 0.0) / vals['SQ_LDS_IDX_ACTIVE']:.3f}.")
    lines.append("")
    out = os.path.join(PROFILES, f"{kernel}_{workload}_sq_counters.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out}: {valu * 64 / upd:.2f} VALU per update")
    return 0


def _is_kernel(name: str, kernel: str) -> bool:
    """Whether a rocprofv3 kernel name is `kernel` (a template instance or a plain function)."""
    return f"::{kernel}<" in name or f"::{kernel}(" in name


def _find(folder: str, suffix: str) -> str:
    import glob
    hits = sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {folder}")
    return hits[0]


def _counter_rows(folder: str, prefix: str):
    import csv
    with open(_find(folder, f"{prefix}_counter_collection.csv")) as f:
        return list(csv.DictReader(f))


def summarize_profile(folder: str, cfg: int, path: str = "scan") -> int:
    """Write the rocprofv3 summaries of one workload into profiles/ (text only).
    path "scan": the scan kernel of the forward; "from_x": the projection kernel of
    the forward from x and the projection weights."""
    import csv
    shape = ss2d_inputs.CONFIGS[cfg]
    os.makedirs(PROFILES, exist_ok=True)
    from_x, bwd, epi = path == "from_x", path == "backward", path == "epilogue"
    kernel = ("project_kernel" if from_x else "bwd_chunk_kernel" if bwd else "channel_last_kernel" if epi
              else KERNEL_PREFIX)
    workload = shape.name + ("" if path == "scan" else "_" + path)
    extra = " --epilogue" if epi else f" --path {path}" if path != "scan" else ""
    cmds = {k: v.format(d=folder, c=cfg, x=extra) for k, v in PROFILE_COMMANDS.items()}

    # Kernel-trace statistics, next to the bench line printed by the same run.
    with open(_find(folder, "stats_kernel_stats.csv")) as f:
        stats = list(csv.DictReader(f))
    with open(os.path.join(folder, "stats_bench.json")) as f:
        bench_line = [ln for ln in f.read().splitlines() if ln.startswith("{")][-1]
    bench = json.loads(bench_line)
    if from_x:
        alg_bytes, alg_flops = projection_work(shape)
        work = (f"Projection per launch: {alg_flops:.4e} FLOP (fp32 MFMA), algorithmic bytes {alg_bytes:.4e} "
                "(x read once; dt, Bs, Cs written once; weights).")
    elif epi:
        alg_bytes = 2 * shape.elem_bytes * shape.B * shape.D * shape.L + 8 * shape.D
        work = (f"Epilogue per launch: algorithmic bytes {alg_bytes:.4e} (y read once, the channel-last output "
                "written once, gamma and beta).")
    elif bwd:
        alg_bytes = 4 * shape.B * shape.L * (11 * shape.D + 16 * shape.N)
        work = (f"Backward per launch: {shape.updates:.4e} (b,k,d,n,l) terms; algorithmic bytes {alg_bytes:.4e} "
                "(x, dy, dt, Bs, Cs read once; dx, ddt, dBs, dCs written once).")
    else:
        alg_bytes = shape.algorithmic_bytes
        work = f"Updates per launch: {shape.updates:.4e}; algorithmic bytes per launch: {alg_bytes:.4e}."
    lines = [f"# {kernel} — {workload} — rocprofv3 kernel trace", "", f"Workload: {shape}.  {work}", "",
             "Command (from the repository root):", "", "```", cmds["stats"], "```", "",
             "| kernel | calls | average µs | min µs | max µs | share |", "|---|---|---|---|---|---|"]
    # Each template instance of the kernel runs once per step (a segmented backward
    # runs two: its two passes), so its time per step is the sum of their averages.
    kern_avg = None
    per_step = 0.0  # fused plans launch each of a forward's kernels once per step
    present = []
    for r in stats:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        avg = float(r["AverageNs"]) / 1e3
        if _is_kernel(r["Name"], kernel):
            kern_avg = (kern_avg or 0.0) + avg
        for k in STEP_KERNELS:
            if _is_kernel(r["Name"], k):
                per_step += avg
                present.append(k)
        lines.append(f"| `{name}` | {r['Calls']} | {avg:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    lines += ["", f"bench.py's own HIP-event average over the timed steps of this run: "
                  f"{bench['kernel_us']:.1f} µs per step (roofline frac {bench['roofline']['frac']:.3f}).",
              f"rocprofv3 average over all launches (warm-up included): {kern_avg:.1f} µs for {kernel}; "
              f"{per_step:.1f} µs per step as the sum of the average durations of the step's kernels, one launch each "
              f"({', '.join(sorted(present))}).", ""]
    if epi:
        ej = bench["epilogue"]
        lines += [f"The epilogue timed by bench.py with HIP events: {ej['us']:.1f} µs; {kernel} by rocprofv3: "
                  f"{kern_avg:.1f} µs, i.e. {alg_bytes / (kern_avg * 1e-6) / 1e9:.0f} GB/s of algorithmic bytes "
                  f"({alg_bytes / (kern_avg * 1e-6) / 1e9 / HBM_PEAK_GBPS:.3f} of 8 TB/s).", ""]
    if from_x:
        pj = bench["projection"]
        lines += [f"The projection alone, timed by bench.py with HIP events (transpose of x + {kernel}): "
                  f"{pj['us']:.1f} µs; {kernel} by rocprofv3: {kern_avg:.1f} µs, i.e. "
                  f"{alg_flops / (kern_avg * 1e-6) / 1e12:.1f} TFLOP/s "
                  f"({alg_flops / (kern_avg * 1e-6) / FP32_MFMA_PEAK:.3f} of the fp32 MFMA peak) and "
                  f"{alg_bytes / (kern_avg * 1e-6) / 1e9:.0f} GB/s of algorithmic bytes "
                  f"({alg_bytes / (kern_avg * 1e-6) / 1e9 / HBM_PEAK_GBPS:.3f} of 8 TB/s).", ""]
    lines += ["Bench line of this run:", "", "```json", bench_line, "```", ""]
    with open(os.path.join(PROFILES, f"{kernel}_{workload}_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines))

    # HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), calibrated on a plain device copy
    # (the runtime's copy kernel; the largest of its dispatches is the probe).
    per = {}
    for counter, prefix in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        rows = [r for r in _counter_rows(folder, prefix) if r["Counter_Name"] == counter]
        inst = {}  # template instance -> its dispatches' values
        for r in rows:
            if _is_kernel(r["Kernel_Name"], kernel):
                inst.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        copies = [(float(r["Counter_Value"]), r["Kernel_Name"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        probe_kib, probe_name = max(copies)
        expected_kib = COPY_PROBE_MIB * 1024.0
        per[counter] = {"kernel_kib_per_dispatch": sum(sum(v) / len(v) for v in inst.values()),
                        "dispatches": sum(len(v) for v in inst.values()), "instances": len(inst),
                        "copy_probe_kib": probe_kib, "copy_probe_kernel": probe_name,
                        "copy_expected_kib": expected_kib, "scale": expected_kib / probe_kib}
    fetch_b = per["FETCH_SIZE"]["kernel_kib_per_dispatch"] * 1024 * per["FETCH_SIZE"]["scale"]
    write_b = per["WRITE_SIZE"]["kernel_kib_per_dispatch"] * 1024 * per["WRITE_SIZE"]["scale"]
    rec = {"workload": workload, "kernel": kernel, "kernel_source_hash": kernel_source_hash(kernel),
           "kernel_sources": KERNEL_SOURCES[kernel],
           "hbm_bytes_per_launch": fetch_b + write_b, "fetch_bytes": fetch_b, "write_bytes": write_b,
           "algorithmic_bytes": alg_bytes, "counters": per}
    lines = [f"# {kernel} — {workload} — HBM traffic (rocprofv3 counters)", "",
             "Two counter runs, one counter each, from the repository root:", "", "```", cmds["fetch"],
             cmds["write"], "```", "",
             f"Each run also performs one {COPY_PROBE_MIB} MiB device-to-device copy; the scale factor is the "
             "copy's known size divided by what the same counter reads for it.  Where the kernel has several "
             "template instances in a step (the two passes of a segmented backward), the per-dispatch figure "
             "is the sum of the instances' averages.", "",
             "| counter | kernel KiB / dispatch | copy probe KiB | copy expected KiB | scale | kernel bytes |",
             "|---|---|---|---|---|---|"]
    for counter, b in (("FETCH_SIZE", fetch_b), ("WRITE_SIZE", write_b)):
        c = per[counter]
        lines.append(f"| {counter} | {c['kernel_kib_per_dispatch']:.0f} | {c['copy_probe_kib']:.0f} | "
                     f"{c['copy_expected_kib']:.0f} | {c['scale']:.4f} | {b / 1e6:.1f} MB |")
    lines += ["", f"HBM traffic per launch: {(fetch_b + write_b) / 1e6:.1f} MB against "
                  f"{alg_bytes / 1e6:.1f} MB algorithmic "
                  f"(ratio {(fetch_b + write_b) / alg_bytes:.2f}).", "",
              "Record read by bench.py (valid only while the kernel sources hash to the value below):", "",
              "```json", json.dumps(rec, indent=1), "```", ""]
    with open(traffic_file(workload, kernel), "w") as f:
        f.write("\n".join(lines))
    print(f"wrote profiles for {workload}: {kernel} avg {kern_avg:.1f} us, step {per_step:.1f} us, "
          f"traffic {(fetch_b + write_b) / 1e6:.1f} MB")
    return 0


def projection_work(shape, R=None):
    """Algorithmic bytes and FLOP of the projections of one forward: x read once, dt, Bs, Cs
    written once (storage type), fp32 weights; 2 FLOP per multiply-add of x_proj and the dt map."""
    R = ss2d_inputs.default_rank(shape.D) if R is None else R
    C = R + 2 * shape.N
    flops = 2.0 * shape.B * 4 * shape.L * (C * shape.D + shape.D * R)
    nbytes = (shape.elem_bytes * shape.B * shape.L * (shape.D + 4 * (shape.D + 2 * shape.N))
              + 4 * 4 * (C * shape.D + shape.D * R))
    return nbytes, flops


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload index (0..4); 1 = VMamba-T stage-1")
    ap.add_argument("--path", choices=["scan", "from_x", "backward"], default="scan",
                    help="scan: the forward from x, dt, Bs, Cs (the headline); from_x: the forward from x and the "
                         "projection weights (projections on the matrix cores, then the scan); backward: the "
                         "gradients of the forward given dy (fp32 workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing and parity")
    ap.add_argument("--lanes", type=int, default=0, help="force lanes per sequence chunk (16/32/64; 0 = auto)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    ap.add_argument("--flush-steps", type=int, default=10,
                    help="extra steps timed one by one with a 1 GiB fill between them (0 = skip)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the on-device roofline probes")
    ap.add_argument("--epilogue", action="store_true",
                    help="also time the channel-last LayerNorm epilogue on the forward's output")
    ap.add_argument("--summarize-kind", choices=["scan", "from_x", "backward", "epilogue"], default=None,
                    help="which kernel --summarize-profile summarises (default: --path)")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="write the SQ-counter summary (two rocprofv3 --pmc runs in DIR) into profiles/ and exit")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="turn the rocprofv3 output of PROFILE_COMMANDS in DIR into the summaries under profiles/")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.config, args.path)
    if args.summarize_profile:
        return summarize_profile(args.summarize_profile, args.config, args.summarize_kind or args.path)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the SS2D forward shards by (batch, channel) with no exchange; see the design notes)",
              file=sys.stderr)
        return 2

    import torch

    import selective_scan_crossscan_amd as ss2d

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    if args.lanes:
        ss2d.set_lanes_per_seq(args.lanes)
    shape = ss2d_inputs.CONFIGS[args.config]
    print(f"[bench] workload {shape}", file=sys.stderr, flush=True)
    from_x = args.path == "from_x"
    bwd = args.path == "backward"
    inp = ss2d_inputs.generate_projected(shape, seed=0) if from_x else ss2d_inputs.generate(shape, seed=0)
    tdt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    d = {}
    for k, v in inp.items():
        t = torch.from_numpy(v)
        if k in ("x", "dt", "Bs", "Cs"):
            t = t.to(tdt)
        d[k] = t.to(dev)
    y = torch.empty((shape.B, shape.D, shape.H, shape.W), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev)

    if bwd:
        dy = torch.from_numpy(np.random.default_rng(1).standard_normal((shape.B, shape.D, shape.H, shape.W))
                              .astype(np.float32)).to(tdt).to(dev)
        grads = {}

        def step():
            grads.update(ss2d.backward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"], dy,
                                       stream=stream))
    elif from_x:
        def step():
            ss2d.forward_from_x(d["x"], d["x_proj_weight"], d["dt_projs_weight"], d["A_log"], d["dt_bias"],
                                d["Ds"], out=y, stream=stream)
    else:
        def step():
            ss2d.forward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"], out=y,
                         stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    print(f"[bench] {args.steps} steps: events {ev_ms:.3f} ms, wall {wall * 1e3:.3f} ms", file=sys.stderr,
          flush=True)

    # Cold-cache timing, outside the contract's timed region: each step is timed alone
    # after a 1 GiB fill has pushed its inputs out of L2 and the 256 MB MALL.
    flushed = None
    if args.flush_steps > 0:
        junk = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        per_us = []
        for i in range(args.flush_steps):
            junk.fill_(float(i))
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            step()
            a1.record(stream)
            torch.cuda.synchronize()
            per_us.append(a0.elapsed_time(a1) * 1e3)
        del junk
        flushed = {"steps": args.flush_steps, "median_us": float(np.median(per_us)), "min_us": float(min(per_us)),
                   "flush": "1 GiB fill before each step"}

    proj = None
    if from_x:
        # the projections alone (transpose of x + the MFMA projection kernel), into preallocated outputs
        R = d["dt_projs_weight"].shape[2]
        C = R + 2 * shape.N
        pdt = torch.empty((shape.B, 4, shape.D, shape.L), dtype=tdt, device=dev)
        pB = torch.empty((shape.B, 4, shape.N, shape.L), dtype=tdt, device=dev)
        pC = torch.empty_like(pB)
        code = 1 if shape.dtype == "bf16" else 0

        def proj_step():
            rc = ss2d.ss2d_project(d["x"].data_ptr(), d["x_proj_weight"].data_ptr(), d["dt_projs_weight"].data_ptr(),
                                   pdt.data_ptr(), pB.data_ptr(), pC.data_ptr(), shape.B, shape.D, shape.H,
                                   shape.W, shape.N, R, code, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"ss2d_project failed: {rc}")

        for _ in range(args.warmup):
            proj_step()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        p0.record(stream)
        for _ in range(args.steps):
            proj_step()
        p1.record(stream)
        torch.cuda.synchronize()
        proj_s = p0.elapsed_time(p1) * 1e-3 / args.steps
        nbytes, flops = projection_work(shape, R)
        proj = {"us": proj_s * 1e6, "kernels": "transpose of x + MFMA projection", "R": R,
                "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                "achieved_TFLOPs": flops / proj_s / 1e12, "frac_fp32_mfma_peak": flops / proj_s / FP32_MFMA_PEAK,
                "achieved_GBps": nbytes / proj_s / 1e9, "frac_hbm_peak": nbytes / proj_s / 1e9 / HBM_PEAK_GBPS,
                "bound": "hbm" if nbytes / (HBM_PEAK_GBPS * 1e9) > flops / FP32_MFMA_PEAK else "mfma"}
        del pdt, pB, pC

    epi = None
    if args.epilogue:
        gamma = torch.linspace(0.5, 1.5, shape.D, device=dev)
        beta = torch.linspace(-0.1, 0.1, shape.D, device=dev)
        eout = torch.empty((shape.B, shape.H, shape.W, shape.D), dtype=tdt, device=dev)
        for _ in range(args.warmup):
            ss2d.channel_last(y, gamma, beta, out=eout, stream=stream)
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        q0.record(stream)
        for _ in range(args.steps):
            ss2d.channel_last(y, gamma, beta, out=eout, stream=stream)
        q1.record(stream)
        torch.cuda.synchronize()
        epi_s = q0.elapsed_time(q1) * 1e-3 / args.steps
        ebytes = 2 * shape.elem_bytes * shape.B * shape.D * shape.L + 8 * shape.D
        epi = {"us": epi_s * 1e6, "kernel": "channel_last_kernel (LayerNorm over D, channel-last out)",
               "algorithmic_bytes": ebytes, "achieved_GBps": ebytes / epi_s / 1e9,
               "frac_hbm_peak": ebytes / epi_s / 1e9 / HBM_PEAK_GBPS, "bound": "hbm"}
        del eout

    peaks = None
    if not args.no_peaks:
        peaks = ss2d.measure_peaks(1 << 30, stream.cuda_stream)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    plan = dict(kv.split("=") for kv in ss2d.describe(shape.B, shape.D, shape.H, shape.W, shape.N,
                                                       1 if shape.dtype == "bf16" else 0).split())
    nseg = int(plan["segments"])
    launches = int(plan["x_transposed"]) + (1 if nseg == 1 else 5 + int(plan["plane_transposed"]))
    if bwd:
        # two transposes, the chunked scan (or, on a segmented map, its two passes
        # and the segment carry), the dBs/dCs sum, the dx merge, the parameter sums
        launches = 6 if int(plan["backward_segments"]) == 1 else 8
    if from_x:
        launches += 1 + (1 - int(plan["x_transposed"]))  # the projection, and its own transpose of x
    ms_per_step = wall * 1e3 / args.steps
    kernel_s = ev_ms * 1e-3 / args.steps  # one kernel launch per step, same stream
    updates = shape.updates
    value = updates * args.steps / wall
    achieved = updates / kernel_s
    hbm_gbps = shape.algorithmic_bytes / kernel_s / 1e9
    # the counters of the step's dominant kernel: the scan (forward, from_x) or the
    # chunked backward kernel
    traffic = (measured_traffic(shape.name + "_backward", "bwd_chunk_kernel") if bwd
               else measured_traffic(shape.name))

    result = {
        "metric": "SS2D state-updates/s (B·4·D·L·N) and achieved HBM GB/s % of peak",
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (seeded numpy PCG64, VMamba-shaped value recipe)",
        "config": {"workload": shape.name + ("_from_x" if from_x else "_backward" if bwd else ""), "path": args.path, "B": shape.B, "D": shape.D, "H": shape.H, "W": shape.W,
                   "N": shape.N, "K": 4, "L": shape.L, "io_dtype": shape.dtype,
                   "plan": ss2d.describe(shape.B, shape.D, shape.H, shape.W, shape.N,
                                         1 if shape.dtype == "bf16" else 0)},
        "roofline": {
            "bound": "alu",
            "achieved": achieved / 1e9,
            "peak": PEAK_UPDATES_PER_S / 1e9,
            "unit": "Gupdates/s (1 exp2 + 4 fp32 VALU per update = 8 of 128 issue slots/clk/CU)",
            "frac": achieved / PEAK_UPDATES_PER_S,
            "traffic": traffic,
            "timed": f"HIP events around each step on the launch stream: {launches} launch(es) " + (
                     "(transposes of x and dy, the chunked backward kernel, the dBs/dCs sum, the dx merge, the "
                     "parameter sums; traffic is the chunked kernel's own)" if bwd else
                     "(the scan kernel, after a transpose of x on maps of 2048+ pixels; traffic is the scan "
                     "kernel's own)"),
        },
        "hbm": {"algorithmic_bytes": shape.algorithmic_bytes, "achieved_GBps": hbm_gbps,
                "frac_of_peak": hbm_gbps / HBM_PEAK_GBPS, "peak_GBps": HBM_PEAK_GBPS},
        "kernel_us": kernel_s * 1e6,
    }
    if bwd:
        result["roofline"]["unit"] += ("; backward: each (b,k,d,n,l) counted once, though the backward recomputes "
                                       "the forward twice and adds the adjoint walk")
    if epi is not None:
        result["epilogue"] = epi
    if proj is not None:
        result["projection"] = proj
        result["roofline"]["unit"] += "; from_x: the whole path (transpose, projection, scan) per step"
    if flushed is not None:
        flushed["frac_of_roofline_peak"] = updates / (flushed["median_us"] * 1e-6) / PEAK_UPDATES_PER_S
        result["flushed"] = flushed
    if peaks is not None:
        result["measured_peaks"] = {
            "update_mix_Gps": peaks["update_mix_per_s"] / 1e9, "exp_Gps": peaks["exp_per_s"] / 1e9,
            "fma_Gps": peaks["fma_per_s"] / 1e9, "hbm_read_GBps": peaks["hbm_read_Bps"] / 1e9,
            "hbm_copy_GBps": peaks["hbm_copy_Bps"] / 1e9, "lds_read_GBps": peaks["lds_read_Bps"] / 1e9,
            "compute_units": peaks["compute_units"]}
        result["roofline_measured"] = {
            "bound": "alu", "achieved": achieved / 1e9, "peak": peaks["update_mix_per_s"] / 1e9,
            "unit": "Gupdates/s (peak = the probe kernel running the update's exp2 + 4 VALU mix on this device)",
            "frac": achieved / peaks["update_mix_per_s"],
            "hbm_frac_of_measured_copy": hbm_gbps * 1e9 / peaks["hbm_copy_Bps"]}

    if not args.no_cpu_baseline:
        import oracle

        x64 = {k: np.ascontiguousarray(v, dtype=np.float64) for k, v in inp.items()}
        threads = oracle.threads()
        t0 = time.perf_counter()
        if bwd:
            # a bounded sample: the float64 backward oracle on the first batch element
            from oracle import backward as obwd
            x1 = {k: (v[:1] if k in ("x", "dt", "Bs", "Cs") else v) for k, v in x64.items()}
            refs = obwd.ss2d_backward_f64(**x1, dy=dy[:1].double().cpu().numpy())
            cpu_s = (time.perf_counter() - t0) * shape.B
            ref = refs["dx"]
        elif from_x:
            from oracle import projection
            ref = projection.ss2d_from_x_f64(**x64)
            cpu_s = time.perf_counter() - t0
        else:
            ref = oracle.ss2d_f64(**x64)
            cpu_s = time.perf_counter() - t0
        got = (grads["dx"][:1] if bwd else y).double().cpu().numpy()
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        max_abs = float(np.max(np.abs(got - ref)))
        result["cpu_baseline"] = {
            "value": updates / cpu_s,
            "unit": "state-updates/s",
            "cores": 1 if bwd else threads,
            "kind": "oracle",
            "sample": (f"the float64 numpy backward oracle on 1 of {shape.B} batch elements, scaled by {shape.B}; "
                       f"{cpu_s / shape.B:.2f} s for the sample on {cpu_model()}") if bwd else
                      (f"the whole workload ({shape.B}x{shape.D} planes, {updates:.3e} updates), "
                       + ("numpy float64 projections (einsum), then " if from_x else "")
                       + f"fp64 C loops, OpenMP over (b,d) planes; {cpu_s:.2f} s on {cpu_model()}"),
        }
        result["parity"] = {"rel_l2": rel, "max_abs": max_abs, "max_abs_y": float(np.max(np.abs(ref))),
                            "vs": "fp64 backward oracle, dx of batch element 0" if bwd else
                            "fp64 oracle, whole output"}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
