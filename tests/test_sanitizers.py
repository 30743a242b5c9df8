"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The C oracle (oracle/ss2d_oracle.c), built with gcc and both sanitizers into a
  small driver (tests/sanitize/oracle_driver.c), runs on seeded inputs and must
  give the same y as the ordinary build.
* libss2d.so's host code (argument validation, planning, the per-device set-up
  up to the device query), built with hipcc with the sanitizers on the host side
  only, runs tests/sanitize/abi_driver.c: every entry point with arguments that
  validation rejects and with valid arguments on a machine without a GPU, and
  the plan of many shapes.  Skipped where a GPU is present (valid calls would
  then launch kernels on the driver's fake addresses) or hipcc is missing.
Any sanitizer report aborts the driver (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import ss2d_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "selective_scan_crossscan_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
# host-side only: the sanitizers do not apply to GPU code
HIPCC_HOST_SAN = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=all".split()
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _no_device_here():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.parametrize("shape", [(1, 2, 1, 1, 1), (2, 3, 3, 5, 4), (1, 2, 7, 4, 16), (2, 1, 4, 4, 20)])
def test_oracle_under_sanitizers(shape, tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_san"
    subprocess.check_call([gcc, "-O1", "-g", "-std=c99", "-fopenmp", *SAN, "-o", str(exe),
                           os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "ss2d_oracle.c"),
                           "-lm"])
    B, D, H, W, N = shape
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=sum(shape))
    f64 = {k: np.ascontiguousarray(v, dtype=np.float64) for k, v in inp.items()}
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        np.array([B, D, H, W, N], dtype=np.int64).tofile(f)
        for k in ("x", "dt", "A_log", "dt_bias", "Bs", "Cs", "Ds"):
            f64[k].tofile(f)
    dst = tmp_path / "out.bin"
    res = subprocess.run([str(exe), str(src), str(dst)], env=ENV, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr[-2000:]
    y = np.fromfile(dst, dtype=np.float64).reshape(B, D, H, W)
    np.testing.assert_allclose(y, oracle.ss2d_f64(**f64), rtol=1e-13, atol=1e-14)


@pytest.mark.skipif(not _no_device_here(), reason="valid calls would launch kernels on fake addresses")
def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    flags = ["-O1", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", *HIPCC_HOST_SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(name):
        obj = tmp_path / name.replace(".hip", ".o")
        subprocess.run([hipcc, *flags, "-c", "-o", str(obj), os.path.join(CSRC, name)], check=True,
                       capture_output=True, text=True)
        return str(obj)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = tmp_path / "abi_san"
    # the driver is plain C; clang links it with the host objects, the sanitizer
    # runtimes and the HIP runtime
    clang = "/opt/rocm/llvm/bin/clang++"
    drv = tmp_path / "abi_driver.o"
    subprocess.run([clang, "-x", "c", "-O1", *SAN, "-I", os.path.join(ROOT, "include"), "-c", "-o", str(drv),
                    os.path.join(HERE, "abi_driver.c")], check=True, capture_output=True, text=True)
    subprocess.run([clang, *SAN, "-o", str(exe), str(drv), *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], env=ENV, capture_output=True, text=True, timeout=300)
    print(res.stdout[-3000:])
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-3000:])
    assert "failures: 0" in res.stdout
