"""GPU checks of the tiled weight layout (switch_tile_weights /
switch_untile_weights, switch_tile_router, and every layer call with
weight_layout tiled).

* The conversion against the layout's definition in include/switch_moe.h,
  computed here in numpy element by element: bit-exact; and the round trip
  untile(tile(w)) == w.
* The router's planes: in numpy, each piece's 8 values at the position the
  header defines, each plane a bf16 value with at most 8 significant bits
  of the remainder left by the planes before it, hi + mid + lo == W_r
  exactly (in float64), zeros for the padding experts.
* The layer with tiled weights against the same call with row-major weights
  on the same inputs: every output bit-identical (the tiled layout only moves
  each weight to where the same matrix-core operand lane reads it), on the
  streaming expert kernels (d_model 768, capacity 160 and above 160, ragged
  tokens, residual) and on the fused kernel (d_model 128 / 256, drops), for
  switch_layer_forward, _train, _add_norm, _noalloc, the top-2 layer and the
  stage call switch_expert_ffn; and one case against the oracle directly.
"""

import numpy as np
import pytest
import torch

import sparse_mixture_experts_switch_amd as smx
from parity_lib import check_routing, check_y, f64, gpu_outputs_numpy, oracle_run, say
from sparse_mixture_experts_switch_amd.inputs import CONFIGS, LayerConfig, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def tiled_positions(count: int, rows: int, cols: int) -> np.ndarray:
    """Flat position in the tiled layout of element (m, r, k), from the
    header's formula: ((m R/16 + r/16) K/32 + k/32) 512 + (16 ((k%32)/8) +
    r%16) 8 + k%8."""
    m = np.arange(count, dtype=np.int64)[:, None, None]
    r = np.arange(rows, dtype=np.int64)[None, :, None]
    k = np.arange(cols, dtype=np.int64)[None, None, :]
    return (((m * (rows // 16) + r // 16) * (cols // 32) + k // 32) * 512 + (16 * ((k % 32) // 8) + r % 16) * 8
            + k % 8)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("shape", [(1, 16, 32), (3, 48, 96), (2, 64, 64), (5, 256, 128), (4, 3072, 768),
                                   (2, 768, 3072)])
def test_tile_matches_definition(shape):
    count, rows, cols = shape
    say(f"tile {shape}")
    gen = torch.Generator().manual_seed(rows * 7 + cols)
    w = torch.randn(shape, generator=gen).to(torch.bfloat16).to(DEV)
    t = smx.tile_weights(w)
    back = smx.untile_weights(t)
    torch.cuda.synchronize()
    want = np.empty(count * rows * cols, dtype=np.int16)
    want[tiled_positions(count, rows, cols).ravel()] = bits(w).ravel()
    assert np.array_equal(bits(t).ravel(), want)
    assert torch.equal(back.view(torch.int16), w.view(torch.int16))


def test_tile_round_trip_full_size_and_out():
    """The base workload's W_in (128 x 3072 x 768) through both directions,
    into caller-provided outputs; a conversion of zero matrices is a no-op."""
    inp = make_inputs(CONFIGS["base"], device=DEV)
    w = inp["w_in"]
    t = torch.empty_like(w)
    b = torch.empty_like(w)
    smx.tile_weights(w, out=t)
    smx.untile_weights(t, out=b)
    torch.cuda.synchronize()
    assert torch.equal(b.view(torch.int16), w.view(torch.int16))
    assert not torch.equal(t.view(torch.int16), w.view(torch.int16))
    # expert 77's matrix alone matches the definition (its pieces sit in expert 77's range)
    e = 77
    want = np.empty(3072 * 768, dtype=np.int16)
    want[tiled_positions(1, 3072, 768).ravel()] = bits(w[e]).ravel()
    assert np.array_equal(bits(t[e]).ravel(), want)
    empty = torch.empty(0, 16, 32, dtype=torch.bfloat16, device=DEV)
    assert smx.tile_weights(empty).numel() == 0


SMALL = LayerConfig("tl", 1000, 128, 256, 16, 1.0, "bf16")
CASES = {
    "base": CONFIGS["base"],                                       # streaming kernels, capacity 160
    "stream_capacity_above_160": SMALL.with_(d_model=768, d_ff=512, tokens=2500, num_experts=8,
                                             capacity_factor=1.0),  # capacity 313: two row tiles
    "stream_ragged": SMALL.with_(d_model=768, d_ff=384, tokens=777, num_experts=8, capacity_factor=1.25),
    "stream_d192_drops": SMALL.with_(d_model=192, d_ff=256, tokens=901, capacity_factor=0.5),
    "fused_d128": SMALL,
    "fused_d256_drops": SMALL.with_(d_model=256, d_ff=384, tokens=1500, capacity_factor=0.5),
    "fused_two_tiles": SMALL.with_(d_model=256, d_ff=256, tokens=2000, num_experts=16, capacity_factor=1.25),
}


def _tiled(inp):
    """The three weights in the tiled layout: W_r's planes, W_in, W_out."""
    return smx.tile_router(inp["w_router"]), smx.tile_weights(inp["w_in"]), smx.tile_weights(inp["w_out"])


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("N,d", [(1, 64), (16, 64), (20, 128), (128, 768), (2048, 2048)])
def test_tile_router_matches_definition(N, d):
    say(f"tile_router N={N} d={d}")
    gen = torch.Generator().manual_seed(N * 31 + d)
    w = torch.randn(N, d, generator=gen, dtype=torch.float64)
    # values across many binades, exact zeros and a few tiny magnitudes
    w = (w * torch.exp2(torch.randint(-30, 8, (N, d), generator=gen).double())).float()
    w[0, :5] = 0.0
    w = w.to(DEV)
    planes = smx.tile_router(w)
    torch.cuda.synchronize()
    assert tuple(planes.shape) == smx.tiled_router_shape(N, d)
    assert smx.tiled_router_bytes(N, d) == planes.numel() * 2
    b = planes.view(torch.int16).cpu().numpy().view(np.uint16)  # [tiles][d/32][3][64][8]
    # piece (m, g, plane, lane l) holds expert 16 m + l % 16, columns 32 g + 8 (l / 16) .. + 7
    tiles, steps = b.shape[0], b.shape[1]
    m = np.arange(tiles)[:, None, None, None]
    g = np.arange(steps)[None, :, None, None]
    lane = np.arange(64)[None, None, :, None]
    k = np.arange(8)[None, None, None, :]
    row = 16 * m + lane % 16
    col = 32 * g + 8 * (lane // 16) + k
    wr = w.double().cpu().numpy()
    want = np.where(row < N, wr[np.minimum(row, N - 1), col], 0.0)
    hi, mid, lo = (bf16_bits_to_f64(b[:, :, p]) for p in range(3))
    assert np.array_equal(hi + mid + lo, want)  # exact: each sum below is exact in float64
    # each plane holds the leading 8 significant bits of what the earlier planes left
    for part, rest in ((hi, want), (mid, want - hi), (lo, want - hi - mid)):
        nz = rest != 0
        _, ex = np.frexp(np.where(nz, rest, 1.0))
        # |rest - part| < one unit in the 8th significant bit of rest
        assert np.all(np.abs(rest - part)[nz] < np.ldexp(1.0, ex[nz] - 8))
        assert np.all(part[~nz] == 0)


def _same(a: dict, b: dict, keys, label):
    for k in keys:
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k]), f"{label}: {k} differs"


ROUTE_KEYS = ("expert_idx", "gate", "slot", "dropped", "expert_count", "aux_loss")


@pytest.mark.parametrize("name", sorted(CASES))
def test_layer_tiled_is_bit_identical(name):
    cfg = CASES[name]
    say(f"tiled layer {name}: {cfg}")
    inp = make_inputs(cfg, device=DEV)
    C = smx.capacity(cfg.tokens, cfg.num_experts, cfg.capacity_factor)
    wr, wi, wo = _tiled(inp)
    args = (inp["x"], inp["w_router"], inp["router_bias"])
    targs = (inp["x"], wr, inp["router_bias"])
    for res in (False, True):
        a = smx.layer_forward(*args, inp["w_in"], inp["w_out"], C, add_residual=res)
        b = smx.layer_forward(*targs, wi, wo, C, add_residual=res, tiled=True)
        torch.cuda.synchronize()
        _same(a, b, ROUTE_KEYS + ("y",), f"{name} residual={res}")
    if name.startswith("fused") or name == "stream_ragged":
        a = smx.layer_forward_train(*args, inp["w_in"], inp["w_out"], C)
        b = smx.layer_forward_train(*targs, wi, wo, C, tiled=True)
        gamma = torch.linspace(0.5, 1.5, cfg.d_model, device=DEV)
        beta = torch.linspace(-0.1, 0.1, cfg.d_model, device=DEV)
        c = smx.layer_forward_add_norm(*args, inp["w_in"], inp["w_out"], C, gamma, beta, 1e-5)
        d = smx.layer_forward_add_norm(*targs, wi, wo, C, gamma, beta, 1e-5, tiled=True)
        torch.cuda.synchronize()
        _same(a, b, ("y",), f"{name} train")
        _same(c, d, ("y",), f"{name} add_norm")
    if name in ("base", "fused_d256_drops"):
        C2 = smx.capacity(2 * cfg.tokens, cfg.num_experts, cfg.capacity_factor)
        a = smx.topk_layer_forward(*args, inp["w_in"], inp["w_out"], C2, top_k=2)
        b = smx.topk_layer_forward(*targs, wi, wo, C2, top_k=2, tiled=True)
        torch.cuda.synchronize()
        _same(a, b, ROUTE_KEYS + ("y",), f"{name} top-2")
    if name in ("base", "stream_d192_drops"):
        # the stage calls that route: the same outputs from W_r's planes
        N = cfg.num_experts
        a = smx.route(*args, C)
        b = smx.route(*targs, C, tiled=True, num_experts=N)
        c = smx.route_dispatch(*args, C)
        d = smx.route_dispatch(*targs, C, tiled=True, num_experts=N)
        torch.cuda.synchronize()
        _same(a, b, ROUTE_KEYS, f"{name} route")
        _same(c, d, ROUTE_KEYS, f"{name} route_dispatch")
        for e, n in enumerate(c["expert_count"].clamp(max=C).tolist()):  # live rows of the expert buffers
            assert torch.equal(c["dispatched"][e, :n].view(torch.int16), d["dispatched"][e, :n].view(torch.int16))


def test_expert_ffn_and_noalloc_tiled():
    cfg = CASES["stream_ragged"]
    inp = make_inputs(cfg, device=DEV)
    C = smx.capacity(cfg.tokens, cfg.num_experts, cfg.capacity_factor)
    wr, wi, wo = _tiled(inp)
    r = smx.route(inp["x"], inp["w_router"], inp["router_bias"], C)
    disp = smx.dispatch(inp["x"], r["expert_idx"], r["slot"], r["dropped"], cfg.num_experts, C)
    a = smx.expert_ffn(disp, r["expert_count"], inp["w_in"], inp["w_out"])
    b = smx.expert_ffn(disp, r["expert_count"], wi, wo, tiled=True)
    torch.cuda.synchronize()
    # live rows only: the expert buffers' padding rows are left unwritten
    for e, n in enumerate(r["expert_count"].clamp(max=C).tolist()):
        assert torch.equal(a[e, :n].view(torch.int16), b[e, :n].view(torch.int16)), f"expert {e}"
    if smx.noalloc_scratch_bytes() >= smx.workspace_bytes(smx.binding.make_shape(
            cfg.tokens, cfg.d_model, cfg.d_ff, cfg.num_experts, C, cfg.torch_dtype)):
        c = smx.layer_forward(inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"], C)
        d = smx.layer_forward_noalloc(inp["x"], wr, inp["router_bias"], wi, wo, C, tiled=True)
        torch.cuda.synchronize()
        _same(c, d, ROUTE_KEYS + ("y",), "noalloc")


def test_layer_tiled_against_oracle():
    """End to end against the oracle (row-major weights on the oracle's side)."""
    cfg = CASES["stream_d192_drops"]
    inp = make_inputs(cfg, device=DEV)
    C = smx.capacity(cfg.tokens, cfg.num_experts, cfg.capacity_factor)
    wr, wi, wo = _tiled(inp)
    o = smx.layer_forward(inp["x"], wr, inp["router_bias"], wi, wo, C, tiled=True)
    torch.cuda.synchronize()
    g = gpu_outputs_numpy(o)
    own = oracle_run(inp, C, experts=[])
    fed = oracle_run(inp, C, expert_idx=g["expert_idx"])
    check_routing(g, own, fed, "tiled")
    assert g["dropped"].any()
    check_y(g["y"], fed, cfg.torch_dtype, "tiled", expect_rows=int((~fed["dropped"]).sum()))
    assert f64(o["y"]).shape == (cfg.tokens, cfg.d_model)


@pytest.mark.parametrize("name,cfg,cap", [
    # capacity 160: one row tile per expert, weights and results streamed
    ("stream_capacity_160", SMALL.with_(d_model=768, d_ff=384, tokens=1280, num_experts=8), 160),
    # capacity 161: two row tiles, ordinary loads and stores
    ("stream_capacity_161", SMALL.with_(d_model=768, d_ff=384, tokens=1280, num_experts=8), 161),
    # the smallest tiled matrices: 4 column blocks, tiles wider than the matrix
    ("d64_f64", SMALL.with_(d_model=64, d_ff=64, tokens=333, num_experts=3), None),
    ("one_expert", SMALL.with_(d_model=192, d_ff=128, tokens=257, num_experts=1, capacity_factor=0.5), None),
])
def test_layer_tiled_edges(name, cfg, cap):
    """Edges of the tiled path, each bit-identical to row-major weights:
    the capacity where the expert kernels switch from streaming (one row
    tile per expert, nontemporal weights and results) to several row tiles,
    matrices narrower than one tile, and a single expert."""
    say(f"tiled edge {name}: {cfg} capacity {cap}")
    inp = make_inputs(cfg, device=DEV)
    C = cap if cap is not None else smx.capacity(cfg.tokens, cfg.num_experts, cfg.capacity_factor)
    wr, wi, wo = _tiled(inp)
    args = (inp["x"], inp["w_router"], inp["router_bias"])
    a = smx.layer_forward(*args, inp["w_in"], inp["w_out"], C, add_residual=True)
    b = smx.layer_forward(inp["x"], wr, inp["router_bias"], wi, wo, C, add_residual=True, tiled=True)
    torch.cuda.synchronize()
    _same(a, b, ROUTE_KEYS + ("y",), name)
    assert int(a["expert_count"].max()) > 0
