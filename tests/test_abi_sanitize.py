"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every library source is compiled with the sanitizers on its host code only
(device code is built as usual and never runs here), linked with the
checker tests/abi_check.cpp into one executable under _build/, and run twice:
plainly and with the library's debug-sync mode on.  The checker drives
validation, sizes, launch names and error text (see its header); any
sanitizer report aborts it, which fails the test.  Where a GPU is visible the
checker skips the calls that would launch kernels.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_switch_amd", "csrc")
OUT = os.path.join(ROOT, "sparse_mixture_experts_switch_amd", "_build", "abi_sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"

# sanitizers on the host side of each hipcc compile only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
# the checker and the link are host-only clang++ steps
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


@pytest.fixture(scope="module")
def checker():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not installed")
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", *HOST_SAN, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(6, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = os.path.join(OUT, "abi_check.o")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN, "-c",
          os.path.join(ROOT, "tests", "abi_check.cpp"), "-o", drv])
    exe = os.path.join(OUT, "abi_check")
    _run([CLANGXX, *SAN, *objs, drv, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    yield exe
    shutil.rmtree(OUT, ignore_errors=True)


@pytest.mark.parametrize("mode", ["plain", "debug"])
def test_abi_host_code_under_sanitizers(checker, mode):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("SMX_DEBUG_SYNC", None)
    r = subprocess.run([checker] + (["debug"] if mode == "debug" else []), capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, f"abi_check failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    assert "abi_check ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
