"""The compiler's resource report of every kernel in the library (recorded by
the build): no kernel keeps values in scratch memory, except the router
variants for more than 128 experts, whose logits live in a global scratch
buffer and which keep seven row pointers in scratch (reloaded once per
128-expert chunk).  A value that the compiler moves to scratch costs a
memory round trip at each use: the top-2 router's epilogue once held its
four running values there and took 31 us instead of 22."""

import glob
import os
import re

import pytest

from sparse_mixture_experts_switch_amd import build as B

# router for N > 128 (logits in a [T][N] buffer, template argument kLds =
# false): forward top-1 / top-2, the backward's recompute, the single-pass
# routing
ALLOWED = (
    re.compile(r"^_ZN3smx22router_fwd_bf16_kernelILb0ELi[12]E"),
    re.compile(r"^_ZN3smx22router_bwd_bf16_kernelILb0EE"),
    re.compile(r"^_ZN3smx23route_fused_bf16_kernelILb0EE"),
)


def allowed(name: str) -> bool:
    return any(p.match(name) for p in ALLOWED)


@pytest.fixture(scope="module")
def resources():
    srcs = glob.glob(os.path.join(B.CSRC, "*.hip"))
    recs = glob.glob(os.path.join(B.BUILD, "*.resources.txt"))
    if len(recs) < len(srcs):
        B.build(verbose=False)
    r = B.kernel_resources()
    assert r, "no kernel resource report"
    return r


def test_every_source_reports(resources):
    # one report per source, and the layer's kernels are in it
    assert len(glob.glob(os.path.join(B.BUILD, "*.resources.txt"))) >= len(glob.glob(os.path.join(B.CSRC, "*.hip")))
    for part in ("router_fwd_bf16_kernel", "assign_one_kernel", "ffn_gemm_bf16_kernel", "ffn_fused_bf16_kernel",
                 "add_norm_kernel", "topk_sum_kernel", "bwd_gemm_bf16_kernel"):
        assert any(part in k for k in resources), part


def test_no_scratch(resources):
    bad = {k: v.get("ScratchSize [bytes/lane]") for k, v in resources.items()
           if not allowed(k) and (v.get("ScratchSize [bytes/lane]", 0) != 0 or v.get("Dynamic Stack") == "True")}
    assert not bad, f"kernels using scratch memory: {bad}"


def test_allowed_spills_stay_small(resources):
    names = [k for k in resources if allowed(k)]
    assert len(names) == 4, names
    for k in names:
        assert resources[k]["ScratchSize [bytes/lane]"] <= 128, (k, resources[k])
