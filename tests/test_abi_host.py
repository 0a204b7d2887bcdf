"""Host-side checks of the C ABI (no GPU needed, nothing launched).

The library must load, export every function include/switch_moe.h declares,
and reject invalid arguments on the host before anything is enqueued.
Capacity and workspace arithmetic are checked against the oracle and the
hand-worked capacity table.
"""

import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle.switch_oracle as so
import sparse_mixture_experts_switch_amd as smx
from sparse_mixture_experts_switch_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "switch_moe.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*|size_t)\s*\**\s*(switch_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = smx.load_library()
    names = _declared()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in switch_moe.h but not exported"
    assert sorted(B.EXPORTED) == names


def test_capacity_matches_table_and_oracle():
    with open(os.path.join(ROOT, "tests", "golden", "capacity_table.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        assert smx.capacity(c["tokens"], c["experts"], c["cf"]) == c["capacity"], c
    for T in (1, 7, 100, 16384, 2 ** 31 - 1):
        for N in (1, 3, 128, 2048):
            for cf in (0.1, 0.5, 1.0, 1.1, 1.25, 2.0, 3.3, float(N)):
                want = so.expert_capacity(T, N, cf)
                if want > 2 ** 31 - 1:
                    with pytest.raises(smx.SwitchError):
                        smx.capacity(T, N, cf)
                else:
                    assert smx.capacity(T, N, cf) == want, (T, N, cf)


@pytest.mark.parametrize("args", [(-1, 8, 1.0), (10, 0, 1.0), (10, 8, 0.0), (10, 8, -1.0),
                                  (10, 8, float("nan")), (10, 8, float("inf"))])
def test_capacity_rejects(args):
    with pytest.raises(smx.SwitchError) as ei:
        smx.capacity(*args)
    assert ei.value.code == B.SWITCH_E_INVALID
    assert smx.load_library().switch_last_error().decode()


def test_workspace_bytes_layout():
    import torch
    s = B.make_shape(16384, 768, 3072, 128, 160, torch.bfloat16)
    ws = smx.workspace_bytes(s)
    nb = 16384 // 64
    # block counts, block offsets, P partials, P sums, ranks, W_r's three bf16 planes (bf16 layers), the
    # single-pass routing's ordering state (ticket, error word and one state word per block; then per
    # block and expert the aggregate and inclusive counts (4 bytes each) and P sums (8 bytes each)),
    # hidden, slot->token and slot->gate maps
    single_pass = (nb + 4) * 4 + nb * 128 * 24
    planes = 128 * 768 * 3 * 2
    expect_min = (3 * nb * 128 * 4 + 128 * 4 + 16384 * 4 + planes + single_pass + 128 * 160 * 3072 * 2
                  + 2 * 128 * 160 * 4)
    assert expect_min <= ws <= expect_min + 13 * 256
    # more experts than one router chunk adds the [T][N] logits scratch
    s2 = B.make_shape(1000, 64, 64, 300, 10, torch.float32)
    assert smx.workspace_bytes(s2) >= 1000 * 300 * 4
    # routing alone: the capacity-0 figure holds no expert buffers
    s3 = B.make_shape(16384, 768, 3072, 128, 0, torch.bfloat16)
    assert smx.workspace_bytes(s3) < 3 * nb * 128 * 4 + 16384 * 4 + planes + single_pass + 4096


@pytest.mark.parametrize("field,value,code", [
    ("tokens", -1, B.SWITCH_E_INVALID), ("d_model", 0, B.SWITCH_E_INVALID), ("d_ff", -64, B.SWITCH_E_INVALID),
    ("num_experts", 0, B.SWITCH_E_INVALID), ("capacity", -1, B.SWITCH_E_INVALID), ("dtype", 7, B.SWITCH_E_INVALID),
    ("d_model", 96, B.SWITCH_E_UNSUPPORTED), ("d_ff", 100, B.SWITCH_E_UNSUPPORTED),
    ("tokens", 2 ** 31, B.SWITCH_E_UNSUPPORTED), ("weight_layout", 2, B.SWITCH_E_INVALID),
    ("weight_layout", -1, B.SWITCH_E_INVALID), ("weight_layout", B.WEIGHTS_TILED, B.SWITCH_OK),
])
def test_shape_validation(field, value, code):
    import torch
    s = B.make_shape(1024, 128, 256, 8, 128, torch.bfloat16)
    setattr(s, field, value)
    out = ctypes.c_size_t()
    rc = smx.load_library().switch_workspace_bytes(ctypes.byref(s), ctypes.byref(out))
    assert rc == code


def test_entry_points_reject_before_launch():
    """Invalid pointers are caught on the host: the calls return an error code
    and text without touching a device (none exists here)."""
    import torch
    lib = smx.load_library()
    s = B.make_shape(64, 128, 256, 8, 16, torch.bfloat16)
    P = ctypes.c_void_p
    good = P(1 << 20)        # aligned stand-in pointer, never dereferenced on these paths
    odd = P((1 << 20) + 2)   # misaligned
    # route: NULL x
    rc = lib.switch_route(ctypes.byref(s), None, good, None, good, good, good, good, good, good, good, 1 << 30, None)
    assert rc == B.SWITCH_E_INVALID and b"x" in lib.switch_last_error()
    # route: misaligned w_router
    rc = lib.switch_route(ctypes.byref(s), good, odd, None, good, good, good, good, good, good, good, 1 << 30, None)
    assert rc == B.SWITCH_E_INVALID and b"aligned" in lib.switch_last_error()
    # route: workspace too small
    rc = lib.switch_route(ctypes.byref(s), good, good, None, good, good, good, good, good, good, good, 16, None)
    assert rc == B.SWITCH_E_WORKSPACE
    # layer forward: NULL shape
    rc = lib.switch_layer_forward(None, good, good, None, good, good, 0, good, good, good, good, good, good, good,
                                  good, 1 << 30, None)
    assert rc == B.SWITCH_E_INVALID
    # expert ffn: NULL expert_count
    rc = lib.switch_expert_ffn(ctypes.byref(s), good, None, good, good, good, good, 1 << 30, None)
    assert rc == B.SWITCH_E_INVALID
    # combine: misaligned y
    rc = lib.switch_combine(ctypes.byref(s), good, good, good, good, good, None, odd, None)
    assert rc == B.SWITCH_E_INVALID
    # dispatch: NULL dropped
    rc = lib.switch_dispatch(ctypes.byref(s), good, good, good, None, good, None)
    assert rc == B.SWITCH_E_INVALID
    # add_norm: negative / NaN eps, NULL gamma, misaligned out, d_model too large
    for eps in (-1.0, float("nan"), float("inf")):
        assert lib.switch_add_norm(ctypes.byref(s), good, good, good, good, eps, good, None) == B.SWITCH_E_INVALID
    assert lib.switch_add_norm(ctypes.byref(s), good, good, None, good, 1e-6, good, None) == B.SWITCH_E_INVALID
    assert lib.switch_add_norm(ctypes.byref(s), good, good, good, good, 1e-6, odd, None) == B.SWITCH_E_INVALID
    wide = B.make_shape(64, 8192, 256, 8, 16, torch.bfloat16)
    assert lib.switch_add_norm(ctypes.byref(wide), good, good, good, good, 1e-6, good, None) == \
        B.SWITCH_E_UNSUPPORTED
    # combine_add_norm: NULL x, misaligned out, non-finite eps
    rc = lib.switch_combine_add_norm(ctypes.byref(s), good, good, good, good, good, None, good, good, 1e-6, good, None)
    assert rc == B.SWITCH_E_INVALID
    rc = lib.switch_combine_add_norm(ctypes.byref(s), good, good, good, good, good, good, good, good, 1e-6, odd, None)
    assert rc == B.SWITCH_E_INVALID
    rc = lib.switch_combine_add_norm(ctypes.byref(s), good, good, good, good, good, good, good, good,
                                     float("inf"), good, None)
    assert rc == B.SWITCH_E_INVALID
    # route_dispatch: NULL dispatched, small workspace, more experts than the single pass supports
    rc = lib.switch_route_dispatch(ctypes.byref(s), good, good, None, good, good, good, good, good, good, None,
                                   good, 1 << 30, None)
    assert rc == B.SWITCH_E_INVALID and b"dispatched" in lib.switch_last_error()
    rc = lib.switch_route_dispatch(ctypes.byref(s), good, good, None, good, good, good, good, good, good, good,
                                   good, 16, None)
    assert rc == B.SWITCH_E_WORKSPACE
    many = B.make_shape(64, 128, 256, 4096, 16, torch.bfloat16)
    rc = lib.switch_route_dispatch(ctypes.byref(many), good, good, None, good, good, good, good, good, good, good,
                                   good, 1 << 40, None)
    assert rc == B.SWITCH_E_UNSUPPORTED
    # profiled: empty kernel range / times < 1
    for first, last, times in ((0, 0, 0), (2, 1, 1), (-1, 0, 1)):
        rc = lib.switch_layer_forward_profiled(ctypes.byref(s), good, good, None, good, good, 0, good, good, good,
                                               good, good, good, good, good, 1 << 30, None, first, last, times)
        assert rc == B.SWITCH_E_INVALID


def test_tiled_weights_validation():
    """The tiled expert-weight layout: bf16 only, and the conversion calls
    check sizes, pointers and overlap on the host; an empty conversion is a
    no-op that needs no pointers."""
    import torch
    lib = smx.load_library()
    out = ctypes.c_size_t()
    s = B.make_shape(1024, 128, 256, 8, 128, torch.float32, tiled=True)
    assert lib.switch_workspace_bytes(ctypes.byref(s), ctypes.byref(out)) == B.SWITCH_E_UNSUPPORTED
    assert b"bf16" in lib.switch_last_error()
    P = ctypes.c_void_p
    good, other, odd = P(1 << 20), P(1 << 30), P((1 << 20) + 8)
    for fn in (lib.switch_tile_weights, lib.switch_untile_weights):
        assert fn(-1, 64, 128, good, other, None) == B.SWITCH_E_INVALID
        assert fn(2, 24, 128, good, other, None) == B.SWITCH_E_UNSUPPORTED  # rows % 16
        assert fn(2, 64, 48, good, other, None) == B.SWITCH_E_UNSUPPORTED   # cols % 32
        assert fn(2, 64, 128, None, other, None) == B.SWITCH_E_INVALID
        assert fn(2, 64, 128, odd, other, None) == B.SWITCH_E_INVALID
        # dst starts inside src's 32 KB
        assert fn(2, 64, 128, good, P((1 << 20) + 16 * 1024), None) == B.SWITCH_E_INVALID
        assert b"overlap" in lib.switch_last_error()
        assert fn(0, 64, 128, None, None, None) == B.SWITCH_OK
        assert fn(3, 0, 128, None, None, None) == B.SWITCH_OK
    with pytest.raises(ValueError):
        smx.tile_weights(torch.zeros(2, 16, 32))  # fp32
    with pytest.raises(ValueError):
        smx.tile_weights(torch.zeros(2, 16, 32, dtype=torch.bfloat16))  # not on a GPU


def test_tiled_router_validation():
    """W_r's tiled form: its byte count from the header's definition, the
    conversion's host checks (sizes, pointers, overlap), and a tiled layer
    call's workspace without the split planes a row-major call keeps."""
    import torch
    lib = smx.load_library()
    out = ctypes.c_size_t()
    for N, d in ((1, 64), (16, 64), (17, 128), (128, 768), (2048, 2048)):
        assert lib.switch_tiled_router_bytes(N, d, ctypes.byref(out)) == B.SWITCH_OK
        assert out.value == -(-N // 16) * (d // 32) * 3 * 1024 == 2 * int(np.prod(smx.tiled_router_shape(N, d)))
    assert lib.switch_tiled_router_bytes(0, 64, ctypes.byref(out)) == B.SWITCH_E_INVALID
    assert lib.switch_tiled_router_bytes(8, 0, ctypes.byref(out)) == B.SWITCH_E_INVALID
    assert lib.switch_tiled_router_bytes(8, 96, ctypes.byref(out)) == B.SWITCH_E_UNSUPPORTED
    assert lib.switch_tiled_router_bytes(8, 64, None) == B.SWITCH_E_INVALID
    P = ctypes.c_void_p
    good, other, odd = P(1 << 20), P(1 << 30), P((1 << 20) + 8)
    fn = lib.switch_tile_router
    assert fn(0, 64, good, other, None) == B.SWITCH_E_INVALID
    assert fn(8, 96, good, other, None) == B.SWITCH_E_UNSUPPORTED
    assert fn(8, 64, None, other, None) == B.SWITCH_E_INVALID
    assert fn(8, 64, odd, other, None) == B.SWITCH_E_INVALID
    assert fn(8, 64, good, None, None) == B.SWITCH_E_INVALID
    # W_r of 8 x 64 fp32 is 2 KB; planes of one 16-expert tile 6 KB
    assert fn(8, 64, good, P((1 << 20) + 1024), None) == B.SWITCH_E_INVALID
    assert b"overlap" in lib.switch_last_error()
    assert fn(8, 64, P((1 << 20) + 4096), good, None) == B.SWITCH_E_INVALID  # W_r inside the planes
    with pytest.raises(ValueError):
        smx.tile_router(torch.zeros(8, 64, dtype=torch.bfloat16))  # not fp32
    with pytest.raises(ValueError):
        smx.tile_router(torch.zeros(8, 64))  # not on a GPU
    # the layer's workspace: the split planes only for row-major W_r
    rows = B.make_shape(16384, 768, 3072, 128, 160, torch.bfloat16)
    tiled = B.make_shape(16384, 768, 3072, 128, 160, torch.bfloat16, tiled=True)
    planes = -(-128 // 16) * (768 // 32) * 3 * 1024
    assert smx.workspace_bytes(rows) - smx.workspace_bytes(tiled) == planes
    # tiled layer calls check W_r's planes in the binding
    x = torch.zeros(64, 128, dtype=torch.bfloat16)
    w_in = torch.zeros(8, 64, 128, dtype=torch.bfloat16)
    w_out = torch.zeros(8, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="tiled"):
        smx.layer_forward(x, torch.zeros(8, 128), None, w_in, w_out, 16, tiled=True)  # fp32 W_r
    with pytest.raises(ValueError, match="num_experts"):
        smx.route(x, torch.zeros(smx.tiled_router_shape(8, 128), dtype=torch.bfloat16), None, 16, tiled=True)


def test_launch_names_follow_the_shape():
    import torch
    base = B.make_shape(16384, 768, 3072, 128, 160, torch.bfloat16)
    assert smx.launch_names(base) == ["router", "assign", "ffn_up", "ffn_down"]
    # bf16, d_model 128 or 256, capacity <= 160: the expert FFN is one kernel
    narrow = B.make_shape(16384, 256, 1024, 128, 160, torch.bfloat16)
    assert smx.launch_names(narrow) == ["router", "assign", "ffn"]
    deep = B.make_shape(16384, 256, 1024, 128, 161, torch.bfloat16)
    assert smx.launch_names(deep) == ["router", "assign", "ffn_up", "ffn_down"]
    # many router blocks x many experts: scan over blocks, then apply
    many = B.make_shape(32768, 2048, 6144, 2048, 16, torch.bfloat16)
    assert smx.launch_names(many) == ["router", "assign_scan", "assign_apply", "ffn_up", "ffn_down"]
    empty = B.make_shape(0, 64, 64, 8, 0, torch.float32)
    assert smx.launch_names(empty) == ["router", "assign", "ffn_up", "ffn_down"]
    bad = B.make_shape(16, 96, 64, 8, 2, torch.float32)
    with pytest.raises(smx.SwitchError):
        smx.launch_names(bad)


def test_topk_validation_and_workspace():
    """top_k outside 1..min(2, N) is rejected on the host; top_k = 1 needs the
    Switch layer's workspace; top_k = 2 doubles the per-block partials and
    ranks and adds the slot -> row map and the [2][T][d] buffer of routed
    outputs."""
    import torch
    lib = smx.load_library()
    s = B.make_shape(16384, 768, 3072, 128, 320, torch.bfloat16)
    assert smx.topk_workspace_bytes(s, 1) == smx.workspace_bytes(s)
    w2 = smx.topk_workspace_bytes(s, 2)
    nb = 16384 // 64
    single_pass = (2 * nb + 4) * 4 + 2 * nb * 128 * 24  # sized for k blocks per router block
    planes = 128 * 768 * 3 * 2                           # W_r's bf16 planes
    expect_min = (3 * 2 * nb * 128 * 4 + 128 * 4 + 2 * 16384 * 4 + planes + single_pass + 128 * 320 * 3072 * 2
                  + 3 * 128 * 320 * 4 + 2 * 16384 * 768 * 2)
    assert expect_min <= w2 <= expect_min + 15 * 256
    out = ctypes.c_size_t()
    for k, code in ((0, B.SWITCH_E_INVALID), (-1, B.SWITCH_E_INVALID), (3, B.SWITCH_E_UNSUPPORTED),
                    (129, B.SWITCH_E_INVALID)):
        assert lib.switch_topk_workspace_bytes(ctypes.byref(s), k, ctypes.byref(out)) == code, k
    one = B.make_shape(64, 128, 256, 1, 16, torch.bfloat16)
    assert lib.switch_topk_workspace_bytes(ctypes.byref(one), 2, ctypes.byref(out)) == B.SWITCH_E_INVALID
    big = B.make_shape(2 ** 30 + 1, 128, 256, 8, 16, torch.bfloat16)
    assert lib.switch_topk_workspace_bytes(ctypes.byref(big), 2, ctypes.byref(out)) == B.SWITCH_E_UNSUPPORTED
    P = ctypes.c_void_p
    good = P(1 << 20)
    small = B.make_shape(64, 128, 256, 8, 16, torch.bfloat16)
    rc = lib.switch_topk_layer_forward(ctypes.byref(small), 3, good, good, None, good, good, 0, good, good, good,
                                       good, good, good, good, good, 1 << 30, None)
    assert rc == B.SWITCH_E_UNSUPPORTED
    rc = lib.switch_topk_layer_forward(ctypes.byref(small), 2, None, good, None, good, good, 0, good, good, good,
                                       good, good, good, good, good, 1 << 30, None)
    assert rc == B.SWITCH_E_INVALID
    rc = lib.switch_topk_layer_forward(ctypes.byref(small), 2, good, good, None, good, good, 0, good, good, good,
                                       good, good, good, good, good, 64, None)
    assert rc == B.SWITCH_E_WORKSPACE


def test_backward_rejects_before_launch():
    """switch_layer_backward validates on the host (through the binding's
    argument types): NULL forward workspace, a forward workspace smaller than
    the forward's, a non-finite d_aux, misaligned dx, a short workspace."""
    import torch
    lib = smx.load_library()
    s = B.make_shape(64, 128, 256, 8, 16, torch.bfloat16)
    P = ctypes.c_void_p
    good, odd = P(1 << 20), P((1 << 20) + 2)
    fwd_need = smx.workspace_bytes(s)
    bwd_need = smx.backward_workspace_bytes(s)
    assert bwd_need > 0

    def call(fwd_ws=good, fwd_bytes=fwd_need, d_aux=0.5, dx=good, ws_bytes=bwd_need):
        return lib.switch_layer_backward(ctypes.byref(s), good, good, None, good, good, 0, good, good, good, fwd_ws,
                                         fwd_bytes, good, d_aux, dx, good, None, good, good, good, ws_bytes, None)

    assert call(fwd_ws=None) == B.SWITCH_E_INVALID
    assert call(fwd_bytes=fwd_need - 1) == B.SWITCH_E_WORKSPACE
    assert call(d_aux=float("nan")) == B.SWITCH_E_INVALID
    assert call(dx=odd) == B.SWITCH_E_INVALID
    assert call(ws_bytes=bwd_need - 1) == B.SWITCH_E_WORKSPACE
    # the backward reads row-major expert weights only
    s.weight_layout = B.WEIGHTS_TILED
    assert call() == B.SWITCH_E_UNSUPPORTED and b"row-major" in lib.switch_last_error()
    s.weight_layout = B.WEIGHTS_ROWS
    rc = lib.switch_layer_backward_profiled(ctypes.byref(s), good, good, None, good, good, 0, good, good, good, good,
                                            fwd_need, good, 0.5, good, good, None, good, good, good, bwd_need, None,
                                            2, 1, 1)
    assert rc == B.SWITCH_E_INVALID


def test_binding_rejects_mismatched_tensors():
    """The Python binding checks every tensor's dtype, shape and device (and
    each output buffer's) before calling the library, which takes raw pointers
    and could not tell: a bf16 router weight, a short bias, a transposed
    expert weight, a mistyped output, a host workspace or a tensor on another
    device is a ValueError, never a launch.  On this GPU-less host a call with
    every argument right stops at the stream lookup (no device)."""
    import torch
    T, d, f, N, C = 64, 128, 256, 8, 16
    x = torch.zeros(T, d, dtype=torch.bfloat16)
    wr = torch.zeros(N, d)
    w_in = torch.zeros(N, f, d, dtype=torch.bfloat16)
    w_out = torch.zeros(N, d, f, dtype=torch.bfloat16)

    def raises(fn, text):
        with pytest.raises(ValueError) as ei:
            fn()
        assert text in str(ei.value), str(ei.value)

    raises(lambda: smx.route(x, wr.to(torch.bfloat16), None, C), "w_router has dtype")
    raises(lambda: smx.route(x, wr[:, :64].contiguous(), None, C), "w_router has shape")
    raises(lambda: smx.route(x, wr, torch.zeros(N - 1), C), "router_bias has shape")
    raises(lambda: smx.layer_forward(x, wr, None, w_in.transpose(1, 2).contiguous(), w_out, C), "w_in has shape")
    raises(lambda: smx.layer_forward(x, wr, None, w_in, w_out.float(), C), "w_out has dtype")
    raises(lambda: smx.layer_forward(x, wr, None, w_in, w_out, C, workspace=torch.zeros(1 << 20, dtype=torch.int32)),
           "workspace has dtype")
    out = B._route_outputs(T, N, torch.device("cpu"))
    out["gate"] = torch.zeros(T, dtype=torch.float64)
    raises(lambda: smx.layer_forward(x, wr, None, w_in, w_out, C, out=out), "gate has dtype")
    out = B._route_outputs(T, N, torch.device("cpu"))
    out["y"] = torch.zeros(T, d + 64, dtype=torch.bfloat16)
    raises(lambda: smx.layer_forward(x, wr, None, w_in, w_out, C, out=out), "y has shape")
    raises(lambda: smx.layer_forward(x, wr, None, w_in.to("meta"), w_out, C), "w_in is on meta")
    raises(lambda: smx.layer_forward_noalloc(x, wr, None, w_in, w_out.to("meta"), C), "w_out is on meta")
    raises(lambda: smx.dispatch(x, torch.zeros(T, dtype=torch.int64), torch.zeros(T, dtype=torch.int32),
                                torch.zeros(T, dtype=torch.uint8), N, C), "expert_idx has dtype")
    raises(lambda: smx.add_norm(x, x, torch.ones(d + 1), torch.zeros(d), 1e-6), "gamma has shape")
    raises(lambda: smx.combine(torch.zeros(N, C, d, dtype=torch.bfloat16), torch.zeros(T, dtype=torch.int32),
                               torch.zeros(T, dtype=torch.int32), torch.zeros(T, dtype=torch.uint8),
                               torch.zeros(T, dtype=torch.float16)), "gate has dtype")
    # every argument right: the call stops where it would need the GPU
    raises(lambda: smx.layer_forward(x, wr, None, w_in, w_out, C), "cuda device")
    raises(lambda: smx.layer_forward_noalloc(x, wr, None, w_in, w_out, C), "cuda device")


def test_noalloc_rejects_shapes_beyond_its_workspace():
    """switch_layer_forward_noalloc refuses a shape whose workspace exceeds
    its static array (the XXL-shaped layer) with SWITCH_E_WORKSPACE and a
    message, before touching any pointer; the base layer fits."""
    import torch
    lib = smx.load_library()
    cap = smx.noalloc_scratch_bytes()
    assert cap == 1 << 27
    assert smx.workspace_bytes(B.make_shape(16384, 768, 3072, 128, 160, torch.bfloat16)) <= cap
    s = B.make_shape(8192, 4096, 10240, 64, 160, torch.bfloat16)
    assert smx.workspace_bytes(s) > cap
    rc = lib.switch_layer_forward_noalloc(ctypes.byref(s), None, None, None, None, None, 0, None, None, None, None,
                                          None, None, None, None)
    assert rc == B.SWITCH_E_WORKSPACE
    assert b"no-allocation" in lib.switch_last_error()
