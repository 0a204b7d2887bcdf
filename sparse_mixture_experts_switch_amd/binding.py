"""Python binding of libswitchmoe.so (ctypes).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory (outputs and workspace are torch
tensors) and the stream (torch's current stream on the tensors' device).
There is no fallback: if the library or a GPU is missing, calls raise.
The C contract of each function is in include/switch_moe.h.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SwitchError", "load_library", "capacity", "workspace_bytes", "route", "dispatch",
    "expert_ffn", "combine", "layer_forward", "layer_forward_profiled", "launch_names", "add_norm",
    "topk_workspace_bytes", "topk_layer_forward", "backward_workspace_bytes", "layer_backward",
    "layer_backward_profiled", "BACKWARD_KERNELS", "combine_add_norm", "SWITCH_F32", "SWITCH_BF16",
    "layer_forward_noalloc", "noalloc_scratch_bytes", "layer_forward_train", "layer_forward_add_norm",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswitchmoe.so")

SWITCH_OK, SWITCH_E_INVALID, SWITCH_E_UNSUPPORTED, SWITCH_E_WORKSPACE, SWITCH_E_HIP = 0, -1, -2, -3, -4
SWITCH_F32, SWITCH_BF16 = 0, 1
_CODES = {-1: "SWITCH_E_INVALID", -2: "SWITCH_E_UNSUPPORTED", -3: "SWITCH_E_WORKSPACE", -4: "SWITCH_E_HIP"}

EXPORTED = [
    "switch_capacity", "switch_workspace_bytes", "switch_last_error", "switch_route", "switch_dispatch",
    "switch_expert_ffn", "switch_combine", "switch_layer_forward", "switch_layer_forward_profiled",
    "switch_launch_names", "switch_add_norm", "switch_topk_workspace_bytes", "switch_topk_layer_forward",
    "switch_backward_workspace_bytes", "switch_layer_backward", "switch_layer_backward_profiled",
    "switch_combine_add_norm", "switch_route_dispatch", "switch_layer_forward_noalloc",
    "switch_noalloc_scratch_bytes", "switch_layer_forward_train", "switch_layer_forward_add_norm",
    "switch_tile_weights", "switch_untile_weights", "switch_tiled_router_bytes", "switch_tile_router",
]
BACKWARD_KERNELS = ["bwd_dz", "bwd_dw_out", "bwd_dx", "bwd_dw_in", "bwd_router", "bwd_router_dx", "bwd_router_w",
                    "bwd_router_w_sum"]


class SwitchError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODES.get(code, code)}: {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
        ("num_experts", ctypes.c_int32), ("capacity", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("weight_layout", ctypes.c_int32),
    ]


_lib = None
_P = ctypes.c_void_p


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m sparse_mixture_experts_switch_amd.build`")
    lib = ctypes.CDLL(path)
    sp = ctypes.POINTER(Shape)
    i32p, sz = ctypes.POINTER(ctypes.c_int32), ctypes.c_size_t
    lib.switch_capacity.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_double, i32p]
    lib.switch_workspace_bytes.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
    lib.switch_last_error.restype = ctypes.c_char_p
    lib.switch_route.argtypes = [sp] + [_P] * 10 + [sz, _P]
    lib.switch_dispatch.argtypes = [sp] + [_P] * 6
    lib.switch_route_dispatch.argtypes = [sp] + [_P] * 11 + [sz, _P]
    lib.switch_expert_ffn.argtypes = [sp] + [_P] * 6 + [sz, _P]
    lib.switch_combine.argtypes = [sp] + [_P] * 8
    lib.switch_layer_forward.argtypes = [sp, _P, _P, _P, _P, _P, ctypes.c_int32] + [_P] * 8 + [sz, _P]
    lib.switch_layer_forward_train.argtypes = lib.switch_layer_forward.argtypes
    lib.switch_layer_forward_add_norm.argtypes = [sp] + [_P] * 7 + [ctypes.c_float] + [_P] * 8 + [sz, _P]
    lib.switch_layer_forward_profiled.argtypes = (
        [sp, _P, _P, _P, _P, _P, ctypes.c_int32] + [_P] * 8 + [sz, _P, ctypes.c_int32, ctypes.c_int32,
                                                               ctypes.c_int32])
    lib.switch_launch_names.argtypes = [sp, _P, ctypes.c_int32, _P]
    lib.switch_add_norm.argtypes = [sp, _P, _P, _P, _P, ctypes.c_float, _P, _P]
    lib.switch_combine_add_norm.argtypes = [sp] + [_P] * 8 + [ctypes.c_float, _P, _P]
    lib.switch_topk_workspace_bytes.argtypes = [sp, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    bwd = [sp, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, sz, _P, ctypes.c_float] + [_P] * 6 + [sz, _P]
    lib.switch_backward_workspace_bytes.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
    lib.switch_layer_backward.argtypes = bwd
    lib.switch_layer_backward_profiled.argtypes = bwd + [ctypes.c_int32] * 3
    lib.switch_topk_layer_forward.argtypes = (
        [sp, ctypes.c_int32, _P, _P, _P, _P, _P, ctypes.c_int32] + [_P] * 8 + [sz, _P])
    lib.switch_layer_forward_noalloc.argtypes = [sp, _P, _P, _P, _P, _P, ctypes.c_int32] + [_P] * 7 + [_P]
    lib.switch_noalloc_scratch_bytes.argtypes = [ctypes.POINTER(ctypes.c_size_t)]
    lib.switch_tile_weights.argtypes = [ctypes.c_int32] * 3 + [_P] * 3
    lib.switch_untile_weights.argtypes = lib.switch_tile_weights.argtypes
    lib.switch_tiled_router_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.switch_tile_router.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
    for name in EXPORTED:
        if name != "switch_last_error":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != SWITCH_OK:
        raise SwitchError(rc, load_library().switch_last_error().decode())


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _expect(t, name: str, shape, dtype: torch.dtype, dev: torch.device) -> None:
    """Raise ValueError unless t is a contiguous tensor with this shape and
    dtype on the call's device (the C ABI takes raw pointers and cannot tell
    a short, mistyped or host buffer from a good one)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}; the call runs on {dev}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_acts(x, name: str = "x") -> torch.device:
    """A 2-D activation tensor of a supported dtype; returns its device (that
    it is a GPU is checked when the stream is taken, right before the call)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor [tokens][d_model]")
    _dtype_code(x.dtype)
    return x.device


def tiled_router_shape(num_experts: int, d_model: int) -> tuple:
    """Shape of W_r in the tiled layout (tile_router), bf16: 16-expert tiles x
    32-column steps x 3 planes x 64 lanes x 8 values."""
    return ((num_experts + 15) // 16, d_model // 32, 3, 64, 8)


def _check_router(x, w_router, router_bias, tiled: bool = False, num_experts: int | None = None) -> int:
    """Checks the router's weights (fp32 [N][d], or with tiled the planes of
    tile_router for num_experts experts) and bias; returns N."""
    dev = _check_acts(x)
    if tiled:
        if num_experts is None:
            raise ValueError("tiled router weights need num_experts")
        N = int(num_experts)
        _expect(w_router, "w_router (tiled)", tiled_router_shape(N, x.shape[1]), torch.bfloat16, dev)
    else:
        if not isinstance(w_router, torch.Tensor) or w_router.dim() != 2:
            raise ValueError("w_router must be a 2-D tensor [num_experts][d_model]")
        N = w_router.shape[0]
        _expect(w_router, "w_router", (N, x.shape[1]), torch.float32, dev)
    if router_bias is not None:
        _expect(router_bias, "router_bias", (N,), torch.float32, dev)
    return N


def _check_experts(w_in, w_out, N: int, d: int, dtype: torch.dtype, dev: torch.device) -> None:
    if not isinstance(w_in, torch.Tensor) or w_in.dim() != 3:
        raise ValueError("w_in must be a 3-D tensor [num_experts][d_ff][d_model]")
    f = w_in.shape[1]
    _expect(w_in, "w_in", (N, f, d), dtype, dev)
    _expect(w_out, "w_out", (N, d, f), dtype, dev)


def _check_layer_inputs(x, w_router, router_bias, w_in, w_out, tiled: bool = False) -> None:
    if not isinstance(w_in, torch.Tensor) or w_in.dim() != 3:
        raise ValueError("w_in must be a 3-D tensor [num_experts][d_ff][d_model]")
    N = _check_router(x, w_router, router_bias, tiled, w_in.shape[0])
    _check_experts(w_in, w_out, N, x.shape[1], x.dtype, x.device)


def _check_route_outputs(o: dict, T: int, N: int, dev: torch.device, k: int | None = None) -> None:
    rt = (T,) if k is None else (k, T)
    for key, dt, shp in (("expert_idx", torch.int32, rt), ("gate", torch.float32, rt), ("slot", torch.int32, rt),
                         ("dropped", torch.uint8, rt), ("expert_count", torch.int32, (N,)),
                         ("aux_loss", torch.float32, (1,))):
        if key not in o:
            raise ValueError(f"out is missing {key}")
        _expect(o[key], key, shp, dt, dev)


def _check_ws(ws, dev: torch.device) -> None:
    if not isinstance(ws, torch.Tensor) or ws.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    _expect(ws, "workspace", (ws.numel(),), torch.uint8, dev)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return SWITCH_BF16
    if dt == torch.float32:
        return SWITCH_F32
    raise ValueError(f"activation dtype {dt} is not supported (float32 or bfloat16)")


def _stream(dev: torch.device) -> int:
    if dev.type != "cuda":
        raise ValueError("the Switch layer runs on a GPU: tensors must be on a cuda device")
    return torch.cuda.current_stream(dev).cuda_stream


WEIGHTS_ROWS, WEIGHTS_TILED = 0, 1


def make_shape(tokens: int, d_model: int, d_ff: int, num_experts: int, capacity_: int, dtype: torch.dtype,
               tiled: bool = False) -> Shape:
    """The call's shape; tiled declares W_in / W_out in the tiled layout
    (tile_weights), else row-major."""
    return Shape(tokens, d_model, d_ff, num_experts, capacity_, _dtype_code(dtype),
                 WEIGHTS_TILED if tiled else WEIGHTS_ROWS)


def capacity(tokens: int, num_experts: int, capacity_factor: float) -> int:
    """ceil(tokens / num_experts * capacity_factor) (exact)."""
    out = ctypes.c_int32()
    _check(load_library().switch_capacity(tokens, num_experts, float(capacity_factor), ctypes.byref(out)))
    return out.value


def workspace_bytes(shape: Shape) -> int:
    out = ctypes.c_size_t()
    _check(load_library().switch_workspace_bytes(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def _workspace(shape: Shape, dev: torch.device, ws: torch.Tensor | None) -> torch.Tensor:
    need = workspace_bytes(shape)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check_ws(ws, dev)
    return ws


def _route_outputs(T: int, N: int, dev: torch.device, k: int | None = None) -> dict:
    rt = (T,) if k is None else (k, T)
    return {
        "expert_idx": torch.empty(rt, dtype=torch.int32, device=dev),
        "gate": torch.empty(rt, dtype=torch.float32, device=dev),
        "slot": torch.empty(rt, dtype=torch.int32, device=dev),
        "dropped": torch.empty(rt, dtype=torch.uint8, device=dev),
        "expert_count": torch.empty(N, dtype=torch.int32, device=dev),
        "aux_loss": torch.empty(1, dtype=torch.float32, device=dev),
    }


def _shape_of(x, w_in, num_experts, capacity_, d_ff=None) -> Shape:
    T, d = x.shape
    f = d_ff if d_ff is not None else w_in.shape[1]
    return make_shape(T, d, f, num_experts, capacity_, x.dtype)


def route(x: torch.Tensor, w_router: torch.Tensor, router_bias: torch.Tensor | None, capacity_: int,
          workspace: torch.Tensor | None = None, out: dict | None = None, tiled: bool = False,
          num_experts: int | None = None) -> dict:
    """Router, top-1, capacity assignment and aux loss (switch_route); tiled:
    w_router holds tile_router's planes of num_experts experts."""
    N = _check_router(x, w_router, router_bias, tiled, num_experts)
    T, d = x.shape
    shape = make_shape(T, d, 64, N, capacity_, x.dtype, tiled)
    dev = x.device
    o = out if out is not None else _route_outputs(T, N, dev)
    _check_route_outputs(o, T, N, dev)
    # routing needs the workspace of the same shape without expert buffers
    ws = _workspace(make_shape(T, d, 64, N, 0, x.dtype, tiled), dev, workspace)
    _check(load_library().switch_route(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(o["expert_idx"]), _ptr(o["gate"]),
        _ptr(o["slot"]), _ptr(o["dropped"]), _ptr(o["expert_count"]), _ptr(o["aux_loss"]), _ptr(ws),
        ws.numel(), _stream(dev)))
    return o


def route_dispatch(x: torch.Tensor, w_router: torch.Tensor, router_bias: torch.Tensor | None, capacity_: int,
                   workspace: torch.Tensor | None = None, out: dict | None = None,
                   dispatched: torch.Tensor | None = None, tiled: bool = False,
                   num_experts: int | None = None) -> dict:
    """Routing and dispatch in one pass over x (switch_route_dispatch): the
    outputs of route() plus o["dispatched"] [N][C][d]."""
    N = _check_router(x, w_router, router_bias, tiled, num_experts)
    T, d = x.shape
    shape = make_shape(T, d, 64, N, capacity_, x.dtype, tiled)
    dev = x.device
    o = out if out is not None else _route_outputs(T, N, dev)
    _check_route_outputs(o, T, N, dev)
    ws = _workspace(make_shape(T, d, 64, N, 0, x.dtype, tiled), dev, workspace)
    buf = dispatched if dispatched is not None else torch.empty(N, capacity_, d, dtype=x.dtype, device=dev)
    _expect(buf, "dispatched", (N, capacity_, d), x.dtype, dev)
    _check(load_library().switch_route_dispatch(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(o["expert_idx"]), _ptr(o["gate"]),
        _ptr(o["slot"]), _ptr(o["dropped"]), _ptr(o["expert_count"]), _ptr(o["aux_loss"]),
        _ptr(buf) if buf.numel() else None, _ptr(ws), ws.numel(), _stream(dev)))
    o["dispatched"] = buf
    return o


def dispatch(x: torch.Tensor, expert_idx: torch.Tensor, slot: torch.Tensor, dropped: torch.Tensor,
             num_experts: int, capacity_: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Gather kept token rows into [N][C][d] expert buffers (switch_dispatch)."""
    dev = _check_acts(x)
    T, d = x.shape
    _expect(expert_idx, "expert_idx", (T,), torch.int32, dev)
    _expect(slot, "slot", (T,), torch.int32, dev)
    _expect(dropped, "dropped", (T,), torch.uint8, dev)
    shape = make_shape(T, d, 64, num_experts, capacity_, x.dtype)
    buf = out if out is not None else torch.empty(num_experts, capacity_, d, dtype=x.dtype, device=x.device)
    _expect(buf, "out", (num_experts, capacity_, d), x.dtype, dev)
    _check(load_library().switch_dispatch(ctypes.byref(shape), _ptr(x), _ptr(expert_idx), _ptr(slot),
                                          _ptr(dropped), _ptr(buf), _stream(x.device)))
    return buf


def expert_ffn(dispatched: torch.Tensor, expert_count: torch.Tensor, w_in: torch.Tensor, w_out: torch.Tensor,
               workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
               tiled: bool = False) -> torch.Tensor:
    """expert_out[i][r] = W_out,i ReLU(W_in,i dispatched[i][r]) (switch_expert_ffn)."""
    if not isinstance(dispatched, torch.Tensor) or dispatched.dim() != 3:
        raise ValueError("dispatched must be a 3-D tensor [num_experts][capacity][d_model]")
    N, C, d = dispatched.shape
    dev = _check_acts(dispatched.reshape(N * C, d), "dispatched")
    _expect(expert_count, "expert_count", (N,), torch.int32, dev)
    _check_experts(w_in, w_out, N, d, dispatched.dtype, dev)
    shape = make_shape(0, d, w_in.shape[1], N, C, dispatched.dtype, tiled)
    eo = out if out is not None else torch.empty_like(dispatched)
    _expect(eo, "out", (N, C, d), dispatched.dtype, dev)
    ws = workspace
    if ws is None:  # expert_ffn alone needs only the [N][C][d_ff] hidden buffer
        ws = torch.empty(max(N * C * w_in.shape[1] * dispatched.element_size(), 256), dtype=torch.uint8,
                         device=dev)
    _check_ws(ws, dev)
    _check(load_library().switch_expert_ffn(ctypes.byref(shape), _ptr(dispatched), _ptr(expert_count), _ptr(w_in),
                                            _ptr(w_out), _ptr(eo), _ptr(ws), ws.numel(), _stream(dev)))
    return eo


def combine(expert_out: torch.Tensor, expert_idx: torch.Tensor, slot: torch.Tensor, dropped: torch.Tensor,
            gate: torch.Tensor, x_residual: torch.Tensor | None = None,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """y[t] = gate[t] expert_out[e[t]][slot[t]] (0 if dropped) (+ x) (switch_combine)."""
    if not isinstance(expert_out, torch.Tensor) or expert_out.dim() != 3:
        raise ValueError("expert_out must be a 3-D tensor [num_experts][capacity][d_model]")
    N, C, d = expert_out.shape
    dev = _check_acts(expert_out.reshape(N * C, d), "expert_out")
    T = expert_idx.shape[0]
    for t_, name, dt in ((expert_idx, "expert_idx", torch.int32), (slot, "slot", torch.int32),
                         (dropped, "dropped", torch.uint8), (gate, "gate", torch.float32)):
        _expect(t_, name, (T,), dt, dev)
    if x_residual is not None:
        _expect(x_residual, "x_residual", (T, d), expert_out.dtype, dev)
    shape = make_shape(T, d, 64, N, C, expert_out.dtype)
    y = out if out is not None else torch.empty(T, d, dtype=expert_out.dtype, device=expert_out.device)
    _expect(y, "out", (T, d), expert_out.dtype, dev)
    _check(load_library().switch_combine(ctypes.byref(shape), _ptr(expert_out), _ptr(expert_idx), _ptr(slot),
                                         _ptr(dropped), _ptr(gate), _ptr(x_residual), _ptr(y),
                                         _stream(expert_out.device)))
    return y


def _lf_args(x, w_router, router_bias, w_in, w_out, capacity_, add_residual, workspace, out, tiled=False):
    _check_layer_inputs(x, w_router, router_bias, w_in, w_out, tiled)
    T, d = x.shape
    N, f = w_in.shape[0], w_in.shape[1]
    shape = make_shape(T, d, f, N, capacity_, x.dtype, tiled)
    dev = x.device
    o = out if out is not None else _route_outputs(T, N, dev)
    if "y" not in o:
        o["y"] = torch.empty(T, d, dtype=x.dtype, device=dev)
    _check_route_outputs(o, T, N, dev)
    _expect(o["y"], "y", (T, d), x.dtype, dev)
    ws = _workspace(shape, dev, workspace)
    args = [ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_in), _ptr(w_out),
            1 if add_residual else 0, _ptr(o["y"]), _ptr(o["expert_idx"]), _ptr(o["gate"]), _ptr(o["slot"]),
            _ptr(o["dropped"]), _ptr(o["expert_count"]), _ptr(o["aux_loss"]), _ptr(ws), ws.numel(), _stream(dev)]
    return shape, o, args


def layer_forward(x: torch.Tensor, w_router: torch.Tensor, router_bias: torch.Tensor | None, w_in: torch.Tensor,
                  w_out: torch.Tensor, capacity_: int, add_residual: bool = False,
                  workspace: torch.Tensor | None = None, out: dict | None = None, tiled: bool = False) -> dict:
    """The whole Switch layer forward (switch_layer_forward); tiled: W_in and
    W_out are in the tiled layout (tile_weights) and w_router holds W_r's
    planes (tile_router)."""
    _, o, args = _lf_args(x, w_router, router_bias, w_in, w_out, capacity_, add_residual, workspace, out, tiled)
    _check(load_library().switch_layer_forward(*args))
    return o


def layer_forward_train(x: torch.Tensor, w_router: torch.Tensor, router_bias: torch.Tensor | None,
                        w_in: torch.Tensor, w_out: torch.Tensor, capacity_: int, add_residual: bool = False,
                        workspace: torch.Tensor | None = None, out: dict | None = None,
                        tiled: bool = False) -> dict:
    """The layer forward of a training step (switch_layer_forward_train): the
    results of layer_forward, and `workspace` then holds the hidden
    activations that layer_backward reads."""
    _, o, args = _lf_args(x, w_router, router_bias, w_in, w_out, capacity_, add_residual, workspace, out, tiled)
    _check(load_library().switch_layer_forward_train(*args))
    return o


def layer_forward_add_norm(x: torch.Tensor, w_router: torch.Tensor, router_bias: torch.Tensor | None,
                           w_in: torch.Tensor, w_out: torch.Tensor, capacity_: int, gamma: torch.Tensor,
                           beta: torch.Tensor, eps: float, workspace: torch.Tensor | None = None,
                           out: dict | None = None, tiled: bool = False) -> dict:
    """The layer and the block's Add + Normalize in one call
    (switch_layer_forward_add_norm): o["y"] holds LayerNorm(x + y_bare) *
    gamma + beta."""
    _, o, args = _lf_args(x, w_router, router_bias, w_in, w_out, capacity_, False, workspace, out, tiled)
    d = x.shape[1]
    _expect(gamma, "gamma", (d,), torch.float32, x.device)
    _expect(beta, "beta", (d,), torch.float32, x.device)
    shape, xp, wr, wb, wi, wo, _res, y, *rest = args
    _check(load_library().switch_layer_forward_add_norm(shape, xp, wr, wb, wi, wo, _ptr(gamma), _ptr(beta),
                                                         float(eps), y, *rest))
    return o


def layer_forward_profiled(x, w_router, router_bias, w_in, w_out, capacity_, first_kernel: int, last_kernel: int,
                           times: int = 1, add_residual=False, workspace=None, out=None, tiled=False) -> dict:
    """Kernels first_kernel..last_kernel of layer_forward only, each launched
    `times` times back to back (switch_layer_forward_profiled); asynchronous."""
    _, o, args = _lf_args(x, w_router, router_bias, w_in, w_out, capacity_, add_residual, workspace, out, tiled)
    _check(load_library().switch_layer_forward_profiled(*args, int(first_kernel), int(last_kernel), int(times)))
    return o


def noalloc_scratch_bytes() -> int:
    """Bytes of the static workspace of layer_forward_noalloc."""
    out = ctypes.c_size_t()
    _check(load_library().switch_noalloc_scratch_bytes(ctypes.byref(out)))
    return out.value


def layer_forward_noalloc(x: torch.Tensor, w_router: torch.Tensor, router_bias: torch.Tensor | None,
                          w_in: torch.Tensor, w_out: torch.Tensor, capacity_: int, add_residual: bool = False,
                          out: dict | None = None, tiled: bool = False) -> dict:
    """The layer forward on the library's static workspace
    (switch_layer_forward_noalloc): no device memory is allocated by the call.
    `out` holds the output tensors (expert_idx, gate, slot, dropped,
    expert_count, aux_loss, y); when it is None they are allocated here, by
    the caller's side, before the call."""
    T, d = x.shape
    N, f = w_in.shape[0], w_in.shape[1]
    shape = make_shape(T, d, f, N, capacity_, x.dtype, tiled)
    dev = x.device
    _check_layer_inputs(x, w_router, router_bias, w_in, w_out, tiled)
    o = out if out is not None else _route_outputs(T, N, dev)
    if "y" not in o:
        o["y"] = torch.empty(T, d, dtype=x.dtype, device=dev)
    _check_route_outputs(o, T, N, dev)
    _expect(o["y"], "y", (T, d), x.dtype, dev)
    _check(load_library().switch_layer_forward_noalloc(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_in), _ptr(w_out),
        1 if add_residual else 0, _ptr(o["y"]), _ptr(o["expert_idx"]), _ptr(o["gate"]), _ptr(o["slot"]),
        _ptr(o["dropped"]), _ptr(o["expert_count"]), _ptr(o["aux_loss"]), _stream(dev)))
    return o


def add_norm(x: torch.Tensor | None, y: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """Layer normalisation over d_model of x + y (x may be None): the block's
    Add + Normalize after the layer (switch_add_norm).  out may be y."""
    dev = _check_acts(y, "y")
    T, d = y.shape
    if x is not None:
        _expect(x, "x", (T, d), y.dtype, dev)
    _expect(gamma, "gamma", (d,), torch.float32, dev)
    _expect(beta, "beta", (d,), torch.float32, dev)
    shape = make_shape(T, d, 64, 1, 0, y.dtype)
    o = out if out is not None else torch.empty_like(y)
    _expect(o, "out", (T, d), y.dtype, dev)
    _check(load_library().switch_add_norm(ctypes.byref(shape), _ptr(x), _ptr(y), _ptr(gamma), _ptr(beta),
                                          float(eps), _ptr(o), _stream(y.device)))
    return o


def topk_workspace_bytes(shape: Shape, top_k: int) -> int:
    out = ctypes.c_size_t()
    _check(load_library().switch_topk_workspace_bytes(ctypes.byref(shape), int(top_k), ctypes.byref(out)))
    return out.value


def topk_layer_forward(x: torch.Tensor, w_router: torch.Tensor, router_bias: torch.Tensor | None,
                       w_in: torch.Tensor, w_out: torch.Tensor, capacity_: int, top_k: int,
                       add_residual: bool = False, workspace: torch.Tensor | None = None,
                       out: dict | None = None, tiled: bool = False) -> dict:
    """Classic top-k MoE layer, k = 1 or 2 (switch_topk_layer_forward); the
    routing outputs are [top_k][T]."""
    _check_layer_inputs(x, w_router, router_bias, w_in, w_out, tiled)
    T, d = x.shape
    N, f = w_in.shape[0], w_in.shape[1]
    shape = make_shape(T, d, f, N, capacity_, x.dtype, tiled)
    dev = x.device
    o = out if out is not None else _route_outputs(T, N, dev, top_k)
    if "y" not in o:
        o["y"] = torch.empty(T, d, dtype=x.dtype, device=dev)
    _check_route_outputs(o, T, N, dev, int(top_k))
    _expect(o["y"], "y", (T, d), x.dtype, dev)
    ws = workspace
    if ws is None:
        ws = torch.empty(max(topk_workspace_bytes(shape, top_k), 256), dtype=torch.uint8, device=dev)
    _check_ws(ws, dev)
    _check(load_library().switch_topk_layer_forward(
        ctypes.byref(shape), int(top_k), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_in), _ptr(w_out),
        1 if add_residual else 0, _ptr(o["y"]), _ptr(o["expert_idx"]), _ptr(o["gate"]), _ptr(o["slot"]),
        _ptr(o["dropped"]), _ptr(o["expert_count"]), _ptr(o["aux_loss"]), _ptr(ws), ws.numel(), _stream(dev)))
    return o


def _tile_call(fn, w: torch.Tensor, out: torch.Tensor | None) -> torch.Tensor:
    if not isinstance(w, torch.Tensor) or w.dim() != 3 or w.dtype != torch.bfloat16:
        raise ValueError("expert weights must be a 3-D bfloat16 tensor [count][rows][cols]")
    if not w.is_contiguous():
        raise ValueError("expert weights must be contiguous")
    dev = w.device
    o = out if out is not None else torch.empty_like(w)
    _expect(o, "out", tuple(w.shape), torch.bfloat16, dev)
    cnt, rows, cols = w.shape
    _check(fn(int(cnt), int(rows), int(cols), _ptr(w), _ptr(o), _stream(dev)))
    return o


def tile_weights(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major expert weights [count][rows][cols] (W_in [N][d_ff][d_model]
    or W_out [N][d_model][d_ff], bf16) -> the tiled layout that the layer
    calls read with tiled=True (switch_tile_weights).  Same shape and dtype;
    asynchronous on the current stream."""
    return _tile_call(load_library().switch_tile_weights, w, out)


def untile_weights(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Tiled expert weights -> row-major (switch_untile_weights)."""
    return _tile_call(load_library().switch_untile_weights, w, out)


def tiled_router_bytes(num_experts: int, d_model: int) -> int:
    out = ctypes.c_size_t()
    _check(load_library().switch_tiled_router_bytes(int(num_experts), int(d_model), ctypes.byref(out)))
    return out.value


def tile_router(w_router: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """W_r [N][d_model] fp32 -> its exact three-way bf16 split in the router's
    operand order, the form the layer calls read with tiled=True
    (switch_tile_router); bf16, shape tiled_router_shape(N, d_model);
    asynchronous on the current stream."""
    if not isinstance(w_router, torch.Tensor) or w_router.dim() != 2 or w_router.dtype != torch.float32:
        raise ValueError("w_router must be a 2-D float32 tensor [num_experts][d_model]")
    if not w_router.is_contiguous():
        raise ValueError("w_router must be contiguous")
    N, d = w_router.shape
    dev = w_router.device
    shp = tiled_router_shape(N, d)
    o = out if out is not None else torch.empty(shp, dtype=torch.bfloat16, device=dev)
    _expect(o, "out", shp, torch.bfloat16, dev)
    _check(load_library().switch_tile_router(int(N), int(d), _ptr(w_router), _ptr(o), _stream(dev)))
    return o


def backward_workspace_bytes(shape: Shape) -> int:
    out = ctypes.c_size_t()
    _check(load_library().switch_backward_workspace_bytes(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def _bwd_args(x, w_router, router_bias, w_in, w_out, capacity_, fwd: dict, fwd_workspace, dy, d_aux,
              add_residual, workspace, out):
    _check_layer_inputs(x, w_router, router_bias, w_in, w_out)
    T, d = x.shape
    N, f = w_in.shape[0], w_in.shape[1]
    shape = make_shape(T, d, f, N, capacity_, x.dtype)
    dev = x.device
    _expect(fwd["expert_idx"], "fwd expert_idx", (T,), torch.int32, dev)
    _expect(fwd["dropped"], "fwd dropped", (T,), torch.uint8, dev)
    _expect(fwd["expert_count"], "fwd expert_count", (N,), torch.int32, dev)
    _check_ws(fwd_workspace, dev)
    _expect(dy, "dy", (T, d), x.dtype, dev)
    o = out if out is not None else {}
    o.setdefault("dx", torch.empty(T, d, dtype=x.dtype, device=dev))
    o.setdefault("dw_router", torch.empty(N, d, dtype=torch.float32, device=dev))
    o.setdefault("d_router_bias", torch.empty(N, dtype=torch.float32, device=dev))
    o.setdefault("dw_in", torch.empty_like(w_in))
    o.setdefault("dw_out", torch.empty_like(w_out))
    _expect(o["dx"], "dx", (T, d), x.dtype, dev)
    _expect(o["dw_router"], "dw_router", (N, d), torch.float32, dev)
    _expect(o["d_router_bias"], "d_router_bias", (N,), torch.float32, dev)
    _expect(o["dw_in"], "dw_in", tuple(w_in.shape), x.dtype, dev)
    _expect(o["dw_out"], "dw_out", tuple(w_out.shape), x.dtype, dev)
    ws = workspace
    if ws is None:
        ws = torch.empty(max(backward_workspace_bytes(shape), 256), dtype=torch.uint8, device=dev)
    _check_ws(ws, dev)
    args = [ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_in), _ptr(w_out),
            1 if add_residual else 0, _ptr(fwd["expert_idx"]), _ptr(fwd["dropped"]), _ptr(fwd["expert_count"]),
            _ptr(fwd_workspace), fwd_workspace.numel(), _ptr(dy), float(d_aux), _ptr(o["dx"]), _ptr(o["dw_router"]),
            _ptr(o["d_router_bias"]), _ptr(o["dw_in"]), _ptr(o["dw_out"]), _ptr(ws), ws.numel(), _stream(dev)]
    return o, args


def layer_backward(x, w_router, router_bias, w_in, w_out, capacity_: int, fwd: dict, fwd_workspace: torch.Tensor,
                   dy: torch.Tensor, d_aux: float, add_residual: bool = False, workspace=None, out=None) -> dict:
    """Gradients of <dy, y> + d_aux aux_loss for the routing of the forward
    call whose outputs are `fwd` and whose workspace is `fwd_workspace`
    (switch_layer_backward); that forward must be layer_forward_train, which
    leaves the hidden activations in its workspace."""
    o, args = _bwd_args(x, w_router, router_bias, w_in, w_out, capacity_, fwd, fwd_workspace, dy, d_aux,
                        add_residual, workspace, out)
    _check(load_library().switch_layer_backward(*args))
    return o


def layer_backward_profiled(x, w_router, router_bias, w_in, w_out, capacity_, fwd, fwd_workspace, dy, d_aux,
                            first_kernel: int, last_kernel: int, times: int = 1, add_residual=False,
                            workspace=None, out=None) -> dict:
    """Kernels first_kernel..last_kernel of layer_backward only (names in
    BACKWARD_KERNELS), each `times` times (switch_layer_backward_profiled)."""
    o, args = _bwd_args(x, w_router, router_bias, w_in, w_out, capacity_, fwd, fwd_workspace, dy, d_aux,
                        add_residual, workspace, out)
    _check(load_library().switch_layer_backward_profiled(*args, int(first_kernel), int(last_kernel), int(times)))
    return o


def combine_add_norm(expert_out: torch.Tensor, expert_idx: torch.Tensor, slot: torch.Tensor,
                     dropped: torch.Tensor, gate: torch.Tensor, x: torch.Tensor, gamma: torch.Tensor,
                     beta: torch.Tensor, eps: float, out: torch.Tensor | None = None) -> torch.Tensor:
    """LayerNorm(x + combine) in one pass (switch_combine_add_norm)."""
    if not isinstance(expert_out, torch.Tensor) or expert_out.dim() != 3:
        raise ValueError("expert_out must be a 3-D tensor [num_experts][capacity][d_model]")
    N, C, d = expert_out.shape
    dev = _check_acts(expert_out.reshape(N * C, d), "expert_out")
    T = expert_idx.shape[0]
    for t_, name, dt in ((expert_idx, "expert_idx", torch.int32), (slot, "slot", torch.int32),
                         (dropped, "dropped", torch.uint8), (gate, "gate", torch.float32)):
        _expect(t_, name, (T,), dt, dev)
    _expect(x, "x", (T, d), expert_out.dtype, dev)
    _expect(gamma, "gamma", (d,), torch.float32, dev)
    _expect(beta, "beta", (d,), torch.float32, dev)
    shape = make_shape(T, d, 64, N, C, expert_out.dtype)
    o = out if out is not None else torch.empty(T, d, dtype=expert_out.dtype, device=expert_out.device)
    _expect(o, "out", (T, d), expert_out.dtype, dev)
    _check(load_library().switch_combine_add_norm(
        ctypes.byref(shape), _ptr(expert_out), _ptr(expert_idx), _ptr(slot), _ptr(dropped), _ptr(gate), _ptr(x),
        _ptr(gamma), _ptr(beta), float(eps), _ptr(o), _stream(expert_out.device)))
    return o


def launch_names(shape: Shape) -> list[str]:
    """Kernels switch_layer_forward launches for this shape, in order."""
    names = (ctypes.c_char_p * 8)()
    n = ctypes.c_int32()
    _check(load_library().switch_launch_names(ctypes.byref(shape), names, 8, ctypes.byref(n)))
    return [names[i].decode() for i in range(n.value)]
