"""GPU parity of the single-pass routing + dispatch (switch_route_dispatch).

Its routing outputs and dispatch rows must equal those of switch_route
followed by switch_dispatch bit for bit (both are deterministic and share
the router's arithmetic), its aux loss must agree with switch_route's to
1e-6 relative (P sums in 2^-31 fixed point instead of fp32) and with the
oracle to the layer's 1e-4, and the routing must pass the same oracle checks
as the layer.  Shapes span one and many router blocks (up to 2048 blocks, far
more than run at once, so later blocks wait on earlier ones), the LDS and
scratch-row logit paths, drops, bias and the degenerate cases.
"""

import numpy as np
import pytest
import torch

import oracle.switch_oracle as so
import sparse_mixture_experts_switch_amd as smx
from parity_lib import AUX_REL, check_routing, f64, gpu_outputs_numpy, oracle_run, say
from sparse_mixture_experts_switch_amd.inputs import CONFIGS, LayerConfig, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SMALL = LayerConfig("small", 1000, 128, 256, 16, 1.0, "bf16")
CASES = {
    "ragged_tokens": SMALL,
    "one_block": SMALL.with_(tokens=64),
    "one_token": SMALL.with_(tokens=1, num_experts=8),
    "65_tokens": SMALL.with_(tokens=65, num_experts=3),
    "one_expert": SMALL.with_(num_experts=1, tokens=333),
    "drops_cf_quarter": SMALL.with_(capacity_factor=0.25, tokens=4000),
    "no_drops_cf_eq_N": SMALL.with_(capacity_factor=16.0),
    "zipf_bias": SMALL.with_(zipf_s=1.1, tokens=5000, num_experts=32),
    "scratch_logits_200_experts": SMALL.with_(num_experts=200, tokens=3000, capacity_factor=2.0),
    "2048_experts": SMALL.with_(tokens=10000, num_experts=2048, d_model=64, d_ff=64, capacity_factor=2.0),
    "2048_blocks": SMALL.with_(tokens=2048 * 64 - 17, num_experts=64, d_model=64, d_ff=64),
    "fp32_ragged": SMALL.with_(dtype="f32", tokens=531, num_experts=5, d_model=64, d_ff=192),
    "fp32_many_experts": SMALL.with_(dtype="f32", tokens=400, num_experts=300, d_model=128, d_ff=128,
                                     capacity_factor=3.0),
}


def _both(cfg: LayerConfig):
    say(f"case {cfg}")
    inp = make_inputs(cfg, device=DEV)
    N, d = cfg.num_experts, cfg.d_model
    C = smx.capacity(cfg.tokens, N, cfg.capacity_factor)
    r = smx.route(inp["x"], inp["w_router"], inp["router_bias"], C)
    ref = torch.zeros(N, C, d, dtype=inp["x"].dtype, device=DEV)
    if C > 0:
        smx.dispatch(inp["x"], r["expert_idx"], r["slot"], r["dropped"], N, C, out=ref)
    disp = torch.zeros(N, C, d, dtype=inp["x"].dtype, device=DEV)
    f = smx.route_dispatch(inp["x"], inp["w_router"], inp["router_bias"], C, dispatched=disp)
    torch.cuda.synchronize()
    say("  gpu done")
    return inp, C, r, ref, f


def _check_against_stages(r, ref, f, label):
    for k in ("expert_idx", "gate", "slot", "dropped", "expert_count"):
        assert torch.equal(r[k], f[k]), f"{label}: {k} differs from switch_route"
    # every kept row written exactly, padding rows untouched (zero)
    assert torch.equal(ref, f["dispatched"]), f"{label}: dispatched differs from switch_dispatch"
    a, b = float(r["aux_loss"][0]), float(f["aux_loss"][0])
    assert np.isfinite(b), f"{label}: aux loss {b}"
    assert abs(a - b) <= 1e-6 * abs(a) + 1e-12, f"{label}: aux {b} vs switch_route {a}"


@pytest.mark.parametrize("name", sorted(CASES))
def test_route_dispatch_matches_stages_and_oracle(name):
    cfg = CASES[name]
    inp, C, r, ref, f = _both(cfg)
    _check_against_stages(r, ref, f, name)
    g = gpu_outputs_numpy({k: v for k, v in f.items() if k != "dispatched"})
    own = oracle_run(inp, C, experts=[])
    fed = oracle_run(inp, C, expert_idx=g["expert_idx"], experts=[])
    rep = check_routing(g, own, fed, name)
    assert abs(g["aux_loss"] - fed["aux_loss"]) <= AUX_REL * abs(fed["aux_loss"]), name
    # dispatched rows against the oracle's layout of the GPU's routing
    if C > 0:
        buf, filled = so.dispatch(f64(inp["x"]), g["expert_idx"].astype(np.int64), g["slot"], g["dropped"],
                                  cfg.num_experts, C)
        assert np.array_equal(f64(f["dispatched"])[filled], buf[filled]), name
    say(f"  {name}: C={C} {rep}")


def test_route_dispatch_capacity_zero_and_empty():
    cfg = SMALL.with_(tokens=300)
    inp = make_inputs(cfg, device=DEV)
    f = smx.route_dispatch(inp["x"], inp["w_router"], None, 0)
    torch.cuda.synchronize()
    assert bool(f["dropped"].all()) and int(f["expert_count"].sum()) == 300
    empty = make_inputs(cfg.with_(tokens=0), device=DEV)
    f = smx.route_dispatch(empty["x"], empty["w_router"], None, 4)
    torch.cuda.synchronize()
    assert int(f["expert_count"].abs().sum()) == 0 and float(f["aux_loss"][0]) == 0.0


def test_route_dispatch_deterministic_and_reusable_workspace():
    """Two calls on one workspace (the second with fewer tokens) and a third
    on the first shape give identical results: the call clears its own
    ordering state."""
    cfg = SMALL.with_(tokens=6000, num_experts=64)
    inp = make_inputs(cfg, device=DEV)
    N, d = cfg.num_experts, cfg.d_model
    C = smx.capacity(cfg.tokens, N, cfg.capacity_factor)
    ws = torch.empty(smx.workspace_bytes(smx.binding.make_shape(cfg.tokens, d, 64, N, 0, inp["x"].dtype)),
                     dtype=torch.uint8, device=DEV)
    a = smx.route_dispatch(inp["x"], inp["w_router"], None, C, workspace=ws,
                           dispatched=torch.zeros(N, C, d, dtype=inp["x"].dtype, device=DEV))
    part = inp["x"][:2500].contiguous()
    Cp = smx.capacity(2500, N, cfg.capacity_factor)
    p = smx.route_dispatch(part, inp["w_router"], None, Cp, workspace=ws,
                           dispatched=torch.zeros(N, Cp, d, dtype=inp["x"].dtype, device=DEV))
    b = smx.route_dispatch(inp["x"], inp["w_router"], None, C, workspace=ws,
                           dispatched=torch.zeros(N, C, d, dtype=inp["x"].dtype, device=DEV))
    rp = smx.route(part, inp["w_router"], None, Cp)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    for k in ("expert_idx", "gate", "slot", "dropped", "expert_count"):
        assert torch.equal(p[k], rp[k]), k


@pytest.mark.parametrize("name", ["base", "large"])
def test_route_dispatch_full_config(name):
    """Full-size workloads: equal to the stage calls, and the routing passes
    the oracle's checks."""
    inp, C, r, ref, f = _both(CONFIGS[name])
    _check_against_stages(r, ref, f, name)
    g = gpu_outputs_numpy({k: v for k, v in f.items() if k != "dispatched"})
    own = oracle_run(inp, C, experts=[])
    fed = oracle_run(inp, C, expert_idx=g["expert_idx"], experts=[])
    rep = check_routing(g, own, fed, name)
    assert abs(g["aux_loss"] - fed["aux_loss"]) <= AUX_REL * abs(fed["aux_loss"]), name
    say(f"  {name}: C={C} {rep}")
