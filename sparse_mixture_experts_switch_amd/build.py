"""Build libswitchmoe.so (all HIP sources in csrc/) for gfx950 with hipcc.

Sources compile in parallel to objects under _build/, then link into one
shared library next to this file.  Each compile also records the compiler's
per-kernel resource report (registers, scratch, LDS, occupancy) in
_build/<source>.resources.txt; kernel_resources() parses them.  Run as a
module to build:
    python -m sparse_mixture_experts_switch_amd.build
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libswitchmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    with open(os.path.join(BUILD, os.path.basename(src) + ".resources.txt"), "w") as fh:
        fh.write(r.stderr)
    return obj


def kernel_resources(build_dir: str = BUILD) -> dict:
    """Per-kernel resource report of the last build: {mangled kernel name:
    {"ScratchSize [bytes/lane]": int, "VGPRs Spill": int, "VGPRs": int, ...}}
    from the compiler's kernel-resource-usage remarks."""
    out: dict = {}
    for path in sorted(glob.glob(os.path.join(build_dir, "*.resources.txt"))):
        cur = None
        with open(path) as fh:
            for line in fh:
                m = re.search(r"remark: Function Name: (\S+) \[", line)
                if m:
                    cur = out.setdefault(m.group(1), {})
                    continue
                m = re.search(r"remark:\s+([^:]+): (\S+) \[-Rpass-analysis", line)
                if m and cur is not None:
                    v = m.group(2)
                    cur[m.group(1).strip()] = int(v) if v.lstrip("-").isdigit() else v
    return out


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
