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
    "switch_combine_add_norm", "switch_route_dispatch",
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


def make_shape(tokens: int, d_model: int, d_ff: int, num_experts: int, capacity_: int, dtype: torch.dtype) -> Shape:
    return Shape(tokens, d_model, d_ff, num_experts, capacity_, _dtype_code(dtype))


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
          workspace: torch.Tensor | None = None, out: dict | None = None) -> dict:
    """Router, top-1, capacity assignment and aux loss (switch_route)."""
    T, d = x.shape
    N = w_router.shape[0]
    shape = make_shape(T, d, 64, N, capacity_, x.dtype)
    dev = x.device
    o = out if out is not None else _route_outputs(T, N, dev)
    # routing needs the workspace of the same shape without expert buffers
    ws = _workspace(make_shape(T, d, 64, N, 0, x.dtype), dev, workspace)
    _check(load_library().switch_route(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(o["expert_idx"]), _ptr(o["gate"]),
        _ptr(o["slot"]), _ptr(o["dropped"]), _ptr(o["expert_count"]), _ptr(o["aux_loss"]), _ptr(ws),
        ws.numel(), _stream(dev)))
    return o


def route_dispatch(x: torch.Tensor, w_router: torch.Tensor, router_bias: torch.Tensor | None, capacity_: int,
                   workspace: torch.Tensor | None = None, out: dict | None = None,
                   dispatched: torch.Tensor | None = None) -> dict:
    """Routing and dispatch in one pass over x (switch_route_dispatch): the
    outputs of route() plus o["dispatched"] [N][C][d]."""
    T, d = x.shape
    N = w_router.shape[0]
    shape = make_shape(T, d, 64, N, capacity_, x.dtype)
    dev = x.device
    o = out if out is not None else _route_outputs(T, N, dev)
    ws = _workspace(make_shape(T, d, 64, N, 0, x.dtype), dev, workspace)
    buf = dispatched if dispatched is not None else torch.empty(N, capacity_, d, dtype=x.dtype, device=dev)
    _check(load_library().switch_route_dispatch(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(o["expert_idx"]), _ptr(o["gate"]),
        _ptr(o["slot"]), _ptr(o["dropped"]), _ptr(o["expert_count"]), _ptr(o["aux_loss"]),
        _ptr(buf) if buf.numel() else None, _ptr(ws), ws.numel(), _stream(dev)))
    o["dispatched"] = buf
    return o


def dispatch(x: torch.Tensor, expert_idx: torch.Tensor, slot: torch.Tensor, dropped: torch.Tensor,
             num_experts: int, capacity_: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Gather kept token rows into [N][C][d] expert buffers (switch_dispatch)."""
    T, d = x.shape
    shape = make_shape(T, d, 64, num_experts, capacity_, x.dtype)
    buf = out if out is not None else torch.empty(num_experts, capacity_, d, dtype=x.dtype, device=x.device)
    _check(load_library().switch_dispatch(ctypes.byref(shape), _ptr(x), _ptr(expert_idx), _ptr(slot),
                                          _ptr(dropped), _ptr(buf), _stream(x.device)))
    return buf


def expert_ffn(dispatched: torch.Tensor, expert_count: torch.Tensor, w_in: torch.Tensor, w_out: torch.Tensor,
               workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """expert_out[i][r] = W_out,i ReLU(W_in,i dispatched[i][r]) (switch_expert_ffn)."""
    N, C, d = dispatched.shape
    shape = make_shape(0, d, w_in.shape[1], N, C, dispatched.dtype)
    dev = dispatched.device
    eo = out if out is not None else torch.empty_like(dispatched)
    ws = workspace
    if ws is None:  # expert_ffn alone needs only the [N][C][d_ff] hidden buffer
        ws = torch.empty(max(N * C * w_in.shape[1] * dispatched.element_size(), 256), dtype=torch.uint8,
                         device=dev)
    _check(load_library().switch_expert_ffn(ctypes.byref(shape), _ptr(dispatched), _ptr(expert_count), _ptr(w_in),
                                            _ptr(w_out), _ptr(eo), _ptr(ws), ws.numel(), _stream(dev)))
    return eo


def combine(expert_out: torch.Tensor, expert_idx: torch.Tensor, slot: torch.Tensor, dropped: torch.Tensor,
            gate: torch.Tensor, x_residual: torch.Tensor | None = None,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """y[t] = gate[t] expert_out[e[t]][slot[t]] (0 if dropped) (+ x) (switch_combine)."""
    N, C, d = expert_out.shape
    T = expert_idx.shape[0]
    shape = make_shape(T, d, 64, N, C, expert_out.dtype)
    y = out if out is not None else torch.empty(T, d, dtype=expert_out.dtype, device=expert_out.device)
    _check(load_library().switch_combine(ctypes.byref(shape), _ptr(expert_out), _ptr(expert_idx), _ptr(slot),
                                         _ptr(dropped), _ptr(gate), _ptr(x_residual), _ptr(y),
                                         _stream(expert_out.device)))
    return y


def _lf_args(x, w_router, router_bias, w_in, w_out, capacity_, add_residual, workspace, out):
    T, d = x.shape
    N, f = w_in.shape[0], w_in.shape[1]
    shape = make_shape(T, d, f, N, capacity_, x.dtype)
    dev = x.device
    o = out if out is not None else _route_outputs(T, N, dev)
    if "y" not in o:
        o["y"] = torch.empty(T, d, dtype=x.dtype, device=dev)
    ws = _workspace(shape, dev, workspace)
    args = [ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_in), _ptr(w_out),
            1 if add_residual else 0, _ptr(o["y"]), _ptr(o["expert_idx"]), _ptr(o["gate"]), _ptr(o["slot"]),
            _ptr(o["dropped"]), _ptr(o["expert_count"]), _ptr(o["aux_loss"]), _ptr(ws), ws.numel(), _stream(dev)]
    return shape, o, args


def layer_forward(x: torch.Tensor, w_router: torch.Tensor, router_bias: torch.Tensor | None, w_in: torch.Tensor,
                  w_out: torch.Tensor, capacity_: int, add_residual: bool = False,
                  workspace: torch.Tensor | None = None, out: dict | None = None) -> dict:
    """The whole Switch layer forward (switch_layer_forward)."""
    _, o, args = _lf_args(x, w_router, router_bias, w_in, w_out, capacity_, add_residual, workspace, out)
    _check(load_library().switch_layer_forward(*args))
    return o


def layer_forward_profiled(x, w_router, router_bias, w_in, w_out, capacity_, first_kernel: int, last_kernel: int,
                           times: int = 1, add_residual=False, workspace=None, out=None) -> dict:
    """Kernels first_kernel..last_kernel of layer_forward only, each launched
    `times` times back to back (switch_layer_forward_profiled); asynchronous."""
    _, o, args = _lf_args(x, w_router, router_bias, w_in, w_out, capacity_, add_residual, workspace, out)
    _check(load_library().switch_layer_forward_profiled(*args, int(first_kernel), int(last_kernel), int(times)))
    return o


def add_norm(x: torch.Tensor | None, y: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """Layer normalisation over d_model of x + y (x may be None): the block's
    Add + Normalize after the layer (switch_add_norm).  out may be y."""
    T, d = y.shape
    shape = make_shape(T, d, 64, 1, 0, y.dtype)
    o = out if out is not None else torch.empty_like(y)
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
                       out: dict | None = None) -> dict:
    """Classic top-k MoE layer, k = 1 or 2 (switch_topk_layer_forward); the
    routing outputs are [top_k][T]."""
    T, d = x.shape
    N, f = w_in.shape[0], w_in.shape[1]
    shape = make_shape(T, d, f, N, capacity_, x.dtype)
    dev = x.device
    o = out if out is not None else _route_outputs(T, N, dev, top_k)
    if "y" not in o:
        o["y"] = torch.empty(T, d, dtype=x.dtype, device=dev)
    ws = workspace
    if ws is None:
        ws = torch.empty(max(topk_workspace_bytes(shape, top_k), 256), dtype=torch.uint8, device=dev)
    _check(load_library().switch_topk_layer_forward(
        ctypes.byref(shape), int(top_k), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_in), _ptr(w_out),
        1 if add_residual else 0, _ptr(o["y"]), _ptr(o["expert_idx"]), _ptr(o["gate"]), _ptr(o["slot"]),
        _ptr(o["dropped"]), _ptr(o["expert_count"]), _ptr(o["aux_loss"]), _ptr(ws), ws.numel(), _stream(dev)))
    return o


def backward_workspace_bytes(shape: Shape) -> int:
    out = ctypes.c_size_t()
    _check(load_library().switch_backward_workspace_bytes(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def _bwd_args(x, w_router, router_bias, w_in, w_out, capacity_, fwd: dict, fwd_workspace, dy, d_aux,
              add_residual, workspace, out):
    T, d = x.shape
    N, f = w_in.shape[0], w_in.shape[1]
    shape = make_shape(T, d, f, N, capacity_, x.dtype)
    dev = x.device
    o = out if out is not None else {}
    o.setdefault("dx", torch.empty(T, d, dtype=x.dtype, device=dev))
    o.setdefault("dw_router", torch.empty(N, d, dtype=torch.float32, device=dev))
    o.setdefault("d_router_bias", torch.empty(N, dtype=torch.float32, device=dev))
    o.setdefault("dw_in", torch.empty_like(w_in))
    o.setdefault("dw_out", torch.empty_like(w_out))
    ws = workspace
    if ws is None:
        ws = torch.empty(max(backward_workspace_bytes(shape), 256), dtype=torch.uint8, device=dev)
    args = [ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_in), _ptr(w_out),
            1 if add_residual else 0, _ptr(fwd["expert_idx"]), _ptr(fwd["dropped"]), _ptr(fwd["expert_count"]),
            _ptr(fwd_workspace), fwd_workspace.numel(), _ptr(dy), float(d_aux), _ptr(o["dx"]), _ptr(o["dw_router"]),
            _ptr(o["d_router_bias"]), _ptr(o["dw_in"]), _ptr(o["dw_out"]), _ptr(ws), ws.numel(), _stream(dev)]
    return o, args


def layer_backward(x, w_router, router_bias, w_in, w_out, capacity_: int, fwd: dict, fwd_workspace: torch.Tensor,
                   dy: torch.Tensor, d_aux: float, add_residual: bool = False, workspace=None, out=None) -> dict:
    """Gradients of <dy, y> + d_aux aux_loss for the routing of the forward
    call whose outputs are `fwd` and whose workspace is `fwd_workspace`
    (switch_layer_backward)."""
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
    N, C, d = expert_out.shape
    T = expert_idx.shape[0]
    shape = make_shape(T, d, 64, N, C, expert_out.dtype)
    o = out if out is not None else torch.empty(T, d, dtype=expert_out.dtype, device=expert_out.device)
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
