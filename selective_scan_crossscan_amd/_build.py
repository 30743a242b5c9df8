"""Build libss2d.so (HIP, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libss2d.so")
# The kernel templates (ss2d_kernels.h) are instantiated in one unit per storage
# type and steps per lane, compiled in parallel.
SOURCES = ["ss2d_api.hip", "ss2d_plan.hip", "ss2d_f32_t16.hip", "ss2d_f32_t8.hip", "ss2d_bf16_t16.hip",
           "ss2d_bf16_t8.hip", "ss2d_peaks.hip", "ss2d_project.hip",
           "ss2d_epilogue.hip", "ss2d_backward.hip"]

# -packed-fp32-ops: no packed FP32 instructions are generated (plain VALU only).
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libss2d.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source into selective_scan_crossscan_amd/libss2d.so; returns its path."""
    tag = f".tmp{os.getpid()}"
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o")) + tag
        objs.append(obj)
        cmds.append([hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, os.path.join(CSRC, src)])
    jobs = jobs or min(len(cmds), os.cpu_count() or 1)
    try:
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + tag
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
