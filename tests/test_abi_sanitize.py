"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library's sources with the sanitizers on the host code only (the
gfx950 device code is compiled as usual), links the C driver
tests/abi_sanitize.c against them and runs it on the CPU.  The driver only
makes calls that fail validation before any launch (invalid dims, null and
misaligned pointers, short workspaces, oversized allocation-free dispatches,
random dims around every documented limit), so no GPU is involved; any
out-of-bounds access, overflow or other undefined behaviour on those paths
aborts the run.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routing_dispatch_grouped_moe_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
# host-only sanitizers: each flag goes to the host compilation alone
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs hipcc and clang from ROCm")
def test_abi_validation_under_asan_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INCLUDE,
               "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result", "-w", *HOST_SAN, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"hipcc failed on {src}:\n{r.stderr[-2000:]}"
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv_o = str(tmp_path / "abi_sanitize.o")
    r = subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-Wall", "-Werror",
                        "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-I", INCLUDE,
                        "-c", os.path.join(ROOT, "tests", "abi_sanitize.c"), "-o", drv_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "abi_sanitize")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *HOST_SAN[:4], *objs, drv_o, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "abi_sanitize: ok" in r.stdout, r.stdout + r.stderr
    shutil.rmtree(tmp_path, ignore_errors=True)
