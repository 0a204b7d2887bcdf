"""GPU parity of switch_layer_forward_add_norm: the Switch layer and the
block's Add + Normalize ("The Architecture in Place") in one call, against
the oracle's layer normalisation of x + y_bare (y_bare from the oracle fed
the GPU's routing), on shapes where the normalization is the fused expert
kernel's epilogue (bf16, d_model 128 or 256) and on shapes that take the bare
layer followed by the add_norm kernel (fp32; bf16 d_model 192 to 768, with
ragged tiles, several row tiles per expert and more tiles than workgroups),
with and without drops; the full base workload; and against the unfused
calls.

Tolerance (end to end), per element of row t:
    |out - ref| <= 2 rstd_t |gamma| dy_t + 2 u |ref| + 1e-5,
with dy_t = max over the row of (tol rms(y) + r |y|), the layer's own bound
on y (parity_lib: tol 2e-2 / r 2^-8 in bf16, 1e-4 / 2^-24 in fp32), carried
through the normalization (a change dv of the row moves the output by at most
~2 rstd |gamma| max|dv| to first order), u = 2^-8 (bf16) or 2^-24 (fp32) for
the output's own rounding, and rstd_t = 1 / sqrt(var(x_t + y_t) + eps).
Dropped rows are the normalization of x alone (dy = 0 there).
"""

import numpy as np
import pytest
import torch

import oracle.switch_oracle as so
import sparse_mixture_experts_switch_amd as smx
from parity_lib import Y_ROUND, Y_TOL, check_routing, f64, gpu_outputs_numpy, oracle_run, report, say
from sparse_mixture_experts_switch_amd.inputs import CONFIGS, LayerConfig, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SMALL = LayerConfig("ln", 1000, 128, 256, 16, 1.0, "bf16")
CASES = {
    "fused_d128": SMALL,
    "fused_d256_drops": SMALL.with_(d_model=256, d_ff=384, tokens=1500, capacity_factor=0.5),
    "fused_two_tiles": SMALL.with_(d_model=256, d_ff=256, tokens=2000, num_experts=16, capacity_factor=1.25),
    "unfused_d768_ragged": SMALL.with_(d_model=768, d_ff=512, tokens=777, num_experts=8, capacity_factor=1.25),
    # Zipf-skewed router bias: drops (capacity 100)
    "unfused_d512_drops": SMALL.with_(d_model=512, d_ff=256, tokens=1600, num_experts=16, capacity_factor=1.0,
                                   zipf_s=1.1),
    "unfused_d384": SMALL.with_(d_model=384, d_ff=256, tokens=1900, num_experts=13, capacity_factor=1.0),
    # three row tiles per expert (capacity 375)
    "unfused_d768_row_tiles": SMALL.with_(d_model=768, d_ff=256, tokens=3000, num_experts=8, capacity_factor=1.0),
    # 512 down-projection tiles: two per workgroup of the persistent grid
    "unfused_two_tiles_per_workgroup": SMALL.with_(d_model=768, d_ff=256, tokens=25600, num_experts=256,
                                                capacity_factor=1.0),
    "unfused_fp32": SMALL.with_(dtype="f32", d_model=64, d_ff=192, tokens=531, num_experts=5),
    "unfused_d192": SMALL.with_(d_model=192, d_ff=256, tokens=901, capacity_factor=0.5),
    "unfused_capacity_above_160": SMALL.with_(d_model=128, d_ff=128, tokens=700, num_experts=2, capacity_factor=1.0),
}


def _affine(d, seed):
    gen = torch.Generator().manual_seed(seed)
    gamma = (1.0 + 0.1 * torch.randn(d, generator=gen)).to(DEV)
    beta = (0.1 * torch.randn(d, generator=gen)).to(DEV)
    return gamma, beta


def _check(cfg, eps=1e-6, seed=3):
    say(f"layer add_norm case {cfg}")
    inp = make_inputs(cfg, device=DEV)
    C = smx.capacity(cfg.tokens, cfg.num_experts, cfg.capacity_factor)
    gamma, beta = _affine(cfg.d_model, seed)
    o = smx.layer_forward_add_norm(inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"], C,
                                   gamma, beta, eps)
    again = smx.layer_forward_add_norm(inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"],
                                       C, gamma, beta, eps)
    bare = smx.layer_forward(inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"], C)
    unfused = smx.add_norm(inp["x"], bare["y"], gamma, beta, eps)
    torch.cuda.synchronize()
    assert torch.equal(o["y"], again["y"]), "repeat run differs"
    for k in ("expert_idx", "gate", "slot", "dropped", "expert_count", "aux_loss"):
        assert torch.equal(o[k], bare[k]), f"routing output {k} differs from switch_layer_forward"
    g = gpu_outputs_numpy(o)
    own = oracle_run(inp, C, experts=[])
    fed = oracle_run(inp, C, expert_idx=g["expert_idx"])
    check_routing(g, own, fed, cfg.name)
    x, yb, ga = f64(inp["x"]), fed["y_bare"], f64(gamma)
    ref = so.add_normalize(x, yb, ga, f64(beta), eps)
    rnd = 2.0 ** -8 if cfg.dtype == "bf16" else 2.0 ** -24
    got = g["y"]
    err = np.abs(got - ref)
    kept = ~fed["dropped"]
    rms = float(np.sqrt(np.mean(yb[kept] ** 2))) if kept.any() else 0.0
    dy = np.where(kept[:, None], Y_TOL[cfg.torch_dtype] * rms + Y_ROUND[cfg.torch_dtype] * np.abs(yb), 0.0)
    rstd = 1.0 / np.sqrt((x + yb).var(axis=1) + eps)
    lim = 2 * rstd[:, None] * np.abs(ga)[None, :] * dy.max(axis=1)[:, None] + 2 * rnd * np.abs(ref) + 1e-5
    worst = np.unravel_index(np.argmax(err - lim), err.shape)
    assert np.all(err <= lim), f"{cfg.name}: err {err[worst]:.3e} > {lim[worst]:.3e} at {worst}"
    # the unfused path rounds y to the activation dtype before the sum: the
    # two differ by at most that rounding, carried through the normalization
    diff = np.abs(f64(unfused) - got)
    assert np.all(diff <= 2 * lim), f"{cfg.name}: fused and unfused differ by {diff.max():.3e}"
    nd = int(g["dropped"].sum())
    report(f"layer_add_norm_{cfg.name}", {"capacity": C, "dropped": nd, "max_err": float(err.max())})
    say(f"  {cfg.name}: C={C} dropped={nd} max err {err.max():.3e}")
    return g


@pytest.mark.parametrize("name", sorted(CASES))
def test_layer_add_norm(name):
    g = _check(CASES[name].with_(name=name))
    if "drops" in name or name == "unfused_d192":
        assert g["dropped"].any(), "the case is meant to drop tokens"


def test_layer_add_norm_base_workload():
    """The full base workload (16384 tokens, d_model 768, d_ff 3072, 128
    experts, capacity 160) at the benchmarked shape, end to end against the
    oracle."""
    _check(CONFIGS["base"], eps=1e-5)


def test_layer_add_norm_empty_and_capacity_zero():
    cfg = SMALL.with_(tokens=300)
    inp = make_inputs(cfg, device=DEV)
    gamma, beta = _affine(cfg.d_model, 1)
    o = smx.layer_forward_add_norm(inp["x"], inp["w_router"], None, inp["w_in"], inp["w_out"], 0, gamma, beta,
                                   1e-6)
    torch.cuda.synchronize()
    g = gpu_outputs_numpy(o)
    assert g["dropped"].all()
    ref = so.add_normalize(f64(inp["x"]), np.zeros((cfg.tokens, cfg.d_model)), f64(gamma), f64(beta), 1e-6)
    assert np.all(np.abs(g["y"] - ref) <= 1e-5 + 2 * 2.0 ** -8 * np.abs(ref))
    with pytest.raises(smx.SwitchError):
        smx.layer_forward_add_norm(inp["x"], inp["w_router"], None, inp["w_in"], inp["w_out"], 4, gamma, beta,
                                   float("nan"))
