"""The library's host logic under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libmoe is compiled with the sanitizers on its host code only
(device code is built as usual and never runs here), linked with the C++
driver tests/host_checks.cpp, and run on the CPU: argument validation of
every entry point, workspace and packed-weight sizing, the 4 GiB operand
limit, the allocation-free entry point's scratch limit and the placement
planner. Any sanitizer report aborts the driver and fails the test.
"""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_10_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

# sanitizers on the host pass only (each flag after -Xarch_host)
HOST_SAN = []
for flag in ("address", "undefined"):
    HOST_SAN += ["-Xarch_host", "-fsanitize=" + flag]
HOST_SAN += ["-Xarch_host", "-fno-sanitize-recover=all"]
LINK_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_host_logic_under_asan_and_ubsan(tmp_path):
    common = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++20", "-fPIC", "-I", INCLUDE]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        extra = ["-ffp-contract=off"] if src.endswith("route.hip") else []
        _run([HIPCC, "--offload-arch=gfx950", *common, *HOST_SAN, *extra,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "host_checks.o")
    _run([CLANG, *common, *LINK_SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-c",
          os.path.join(ROOT, "tests", "host_checks.cpp"), "-o", drv])
    exe = str(tmp_path / "host_checks")
    _run([CLANG, *LINK_SAN, "-o", exe, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env, timeout=600)
    assert "host checks passed" in r.stdout
