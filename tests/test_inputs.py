"""Host checks of the seeded input generator (no GPU, no method arithmetic)."""

import math

import torch

from sparse_mixture_experts_switch_amd.inputs import CONFIGS, make_inputs, zipf_router_bias


def test_tiny_shapes_dtypes_and_determinism():
    cfg = CONFIGS["tiny"]
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    assert a["x"].shape == (512, 64) and a["x"].dtype == torch.float32
    assert a["w_router"].shape == (8, 64) and a["w_router"].dtype == torch.float32
    assert a["w_in"].shape == (8, 256, 64) and a["w_out"].shape == (8, 64, 256)
    assert a["router_bias"] is None
    for k in ("x", "w_router", "w_in", "w_out"):
        assert torch.equal(a[k], b[k])
    c = make_inputs(cfg.with_(seed=1))
    assert not torch.equal(a["x"], c["x"])


def test_truncation_and_scale():
    cfg = CONFIGS["tiny"].with_(num_experts=4, d_model=128, d_ff=512)
    inp = make_inputs(cfg)
    for k, fan in (("w_router", 128), ("w_in", 128), ("w_out", 512)):
        std = math.sqrt(0.1 / fan)
        w = inp[k].double()
        assert w.abs().max() <= 2 * std * (1 + 1e-6)
        # std of N(0, s^2) truncated at +-2s is 0.8796 s
        assert abs(w.std().item() / std - 0.8796) < 0.03


def test_bf16_rounding_and_chunking():
    cfg = CONFIGS["base"].with_(tokens=64, num_experts=3, d_model=64, d_ff=128)
    a = make_inputs(cfg)
    b = make_inputs(cfg, chunk_elems=100)  # one expert per chunk, same stream
    assert a["x"].dtype == torch.bfloat16 and a["w_in"].dtype == torch.bfloat16
    assert torch.equal(a["w_in"], b["w_in"]) and torch.equal(a["w_out"], b["w_out"])


def test_zipf_bias_shape():
    b = zipf_router_bias(128, 1024, 1.1, seed=0)
    assert b.shape == (128,) and b.dtype == torch.float32
    assert b.max().item() == 0.0
    # one expert per Zipf rank: sorted biases decrease like log r^-1.1
    s = torch.sort(b, descending=True).values.double()
    ratio = (s[0] - s[9]) / (s[0] - s[99])
    assert abs(ratio.item() - math.log(10) / math.log(100)) < 1e-6
