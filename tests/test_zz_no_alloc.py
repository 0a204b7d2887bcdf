"""GPU check of switch_layer_forward_noalloc, the layer forward on the
library's static workspace, against switch_layer_forward on a caller
workspace: two calls in a row (the second with a smaller input and the
residual), every output equal bit for bit to the ordinary call's on the same
inputs (the same kernels run on the same data)."""

import pytest
import torch

import sparse_mixture_experts_switch_amd as smx
from parity_lib import say
from sparse_mixture_experts_switch_amd.inputs import CONFIGS, LayerConfig, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _compare(cfg: LayerConfig, add_residual: bool) -> None:
    say(f"no-alloc case {cfg} residual={add_residual}")
    inp = make_inputs(cfg, device=DEV)
    C = smx.capacity(cfg.tokens, cfg.num_experts, cfg.capacity_factor)
    args = (inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"], C)
    ref = smx.layer_forward(*args, add_residual=add_residual)
    out = smx.binding._route_outputs(cfg.tokens, cfg.num_experts, torch.device(DEV))
    out["y"] = torch.empty(cfg.tokens, cfg.d_model, dtype=cfg.torch_dtype, device=DEV)
    got = smx.layer_forward_noalloc(*args, add_residual=add_residual, out=out)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k], got[k]), f"{cfg.name}: {k} differs from switch_layer_forward"
    say(f"  {cfg.name}: equal ({int(got['dropped'].sum())} dropped)")


def test_noalloc_matches_layer_forward_twice():
    need = smx.workspace_bytes(smx.binding.make_shape(16384, 768, 3072, 128, 160, torch.bfloat16))
    assert need <= smx.noalloc_scratch_bytes()  # the base layer fits the static workspace
    _compare(CONFIGS["base"].with_(name="noalloc_base"), add_residual=False)
    _compare(LayerConfig("noalloc_small", 1000, 256, 512, 16, 0.75, "bf16"), add_residual=True)
