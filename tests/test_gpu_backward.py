"""GPU parity of the Switch layer's backward pass (switch_layer_backward)
against the CPU oracle's backward, fed the GPU forward's routing.

Tolerances (derived like the forward's): per element |err| <= tol rms(ref) +
u |ref| + c rss with tol = 2e-2 and u = 2^-8 for bf16 layers (the expert
products take bf16 operands, H and du rounded once each, and every output is
rounded once), tol = 1e-4 and u = 2^-24 for fp32 layers; rms over the whole
output.  The gradients that are sums over tokens (the router bias and weight
gradients, the expert weight gradients) add c rss, rss being the oracle's
root sum of squares of the summed terms: a sum can cancel far below its
terms, and then its error is set by the terms' errors (each term here carries
the bf16 rounding of H, du or g dy: c = 2^-6, four bf16 roundings, for bf16;
c = 2^-16 for fp32, fp32 dot products over up to a few thousand terms).
Outputs that must be exactly zero (experts with no kept token) are checked
exactly.

ReLU near-ties: the derivative of ReLU jumps at 0, and the forward computes a
pre-activation u = W_in x in fp32, so where |u| is within rounding of 0
(|u| <= 2^-18 sqrt(K) rss_k(W_in,fk x_k), 64 times the typical error of an
fp32 sum of the K exact bf16 products) either mask value is correct.  Flipping
the mask of such a (token t, unit f) moves dx_t by +-g z_f W_in,f and row f of
dW_in by +-g z_f x_t (z = W_out^T dy_t); each row holding near-ties must match
the oracle under one of the mask choices for them (all are tried), to the
same tolerance.
"""

import numpy as np
import pytest
import torch

import oracle.switch_oracle as so
import sparse_mixture_experts_switch_amd as smx
from parity_lib import f64, gpu_outputs_numpy, say, weight_source
from sparse_mixture_experts_switch_amd.inputs import CONFIGS, LayerConfig, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SMALL = LayerConfig("small", 1000, 128, 256, 16, 1.0, "bf16")
TOL = {torch.bfloat16: (2e-2, 2.0 ** -8, 2.0 ** -6), torch.float32: (1e-4, 2.0 ** -24, 2.0 ** -16)}


def _close(got: np.ndarray, ref: np.ndarray, dtype, label: str, rss: np.ndarray | None = None) -> float:
    tol, u, c = TOL[dtype]
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    diff = np.abs(got - ref)
    lim = tol * rms + u * np.abs(ref) + (c * rss if rss is not None else 0.0)
    if ref.size:
        worst = np.unravel_index(np.argmax(diff - lim), diff.shape)
        assert np.all(diff <= lim), (f"{label}: |err| {diff[worst]:.3e} > {lim[worst]:.3e} at {worst} "
                                     f"(ref {ref[worst]:.3e}, rms {rms:.3e})")
    return float(diff.max() / rms) if rms > 0 else 0.0


def _run(cfg: LayerConfig, d_aux=0.5, add_residual=False, bias=None, capacity=None, sample_experts=None, seed=5):
    say(f"backward case {cfg} d_aux={d_aux} residual={add_residual}")
    inp = make_inputs(cfg, device=DEV)
    if bias is not None:
        inp["router_bias"] = bias.to(DEV)
    C = smx.capacity(cfg.tokens, cfg.num_experts, cfg.capacity_factor) if capacity is None else capacity
    T, d = cfg.tokens, cfg.d_model
    shape = smx.binding.make_shape(T, d, cfg.d_ff, cfg.num_experts, C, cfg.torch_dtype)
    ws = torch.empty(max(smx.workspace_bytes(shape), 256), dtype=torch.uint8, device=DEV)
    fwd = smx.layer_forward_train(inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"], C,
                                  add_residual=add_residual, workspace=ws)
    g = torch.Generator().manual_seed(seed)
    dy = torch.randn(T, d, generator=g).to(cfg.torch_dtype).to(DEV)
    grads = smx.layer_backward(inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"], C, fwd, ws,
                               dy, d_aux, add_residual=add_residual)
    torch.cuda.synchronize()
    say("  gpu done")
    return inp, C, fwd, ws, dy, grads


def _relu_near_ties(inp, fed, dy):
    """Per kept token t of expert e: the units f whose pre-activation is within
    rounding of 0, with the exact mask and the flip deltas of dx_t and of row
    f of dW_in,e.  Returns {t: [(f, e, sign, dx_delta, dwin_delta)]}."""
    x = f64(inp["x"])
    dyv = f64(dy)
    K = x.shape[1]
    idx, dropped, gate = fed["expert_idx"], fed["dropped"], fed["gate"]
    out = {}
    for e in np.unique(idx[~dropped]):
        rows = np.nonzero(~dropped & (idx == e))[0]
        wi, wo = f64(inp["w_in"][int(e)]), f64(inp["w_out"][int(e)])
        u = x[rows] @ wi.T
        bound = 2.0 ** -18 * np.sqrt(K) * np.sqrt((x[rows] ** 2) @ (wi ** 2).T)
        for r, f in zip(*np.nonzero(np.abs(u) <= bound)):
            t = rows[r]
            z = dyv[t] @ wo[:, f]
            sign = 1.0 if u[r, f] <= 0 else -1.0  # the other mask value adds (sign) g z
            out.setdefault(int(t), []).append((int(f), int(e), sign, sign * gate[t] * z * wi[f],
                                               sign * gate[t] * z * x[t]))
    return out


def _best_alternative(got_row, ref_row, deltas, lim_row):
    """ref_row plus the subset of deltas that best explains got_row."""
    best, best_excess = ref_row, np.max(np.abs(got_row - ref_row) - lim_row)
    n = len(deltas)
    assert n <= 10, f"{n} near-ties in one row"
    for mask in range(1, 1 << n):
        cand = ref_row + sum(deltas[i] for i in range(n) if mask >> i & 1)
        ex = np.max(np.abs(got_row - cand) - lim_row)
        if ex < best_excess:
            best, best_excess = cand, ex
    return best


def _limit(ref, dtype, rss=None):
    tol, u, c = TOL[dtype]
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    return tol * rms + u * np.abs(ref) + (c * rss if rss is not None else 0.0)


def _check(cfg: LayerConfig, d_aux=0.5, add_residual=False, bias=None, capacity=None, sample_experts=None):
    inp, C, fwd, ws, dy, grads = _run(cfg, d_aux, add_residual, bias, capacity)
    g = gpu_outputs_numpy(fwd)
    x, wr = f64(inp["x"]), f64(inp["w_router"])
    b = None if inp["router_bias"] is None else f64(inp["router_bias"])
    ref = so.backward(x, wr, b, weight_source(inp), None, C, f64(dy), d_aux, add_residual=add_residual,
                      expert_idx=g["expert_idx"], weight_grads_for=sample_experts)
    assert np.array_equal(ref["forward"]["dropped"], g["dropped"])
    dt = cfg.torch_dtype
    ties = _relu_near_ties(inp, ref["forward"], dy) if cfg.dtype == "bf16" else {}
    dx = f64(grads["dx"])
    dx_ref = ref["dx"].copy()
    lim = _limit(ref["dx"], dt)
    for t, items in ties.items():
        dx_ref[t] = _best_alternative(dx[t], dx_ref[t], [it[3] for it in items], lim[t])
    rep = {"dx": _close(dx, dx_ref, dt, f"{cfg.name} dx"),
           "dw_router": _close(f64(grads["dw_router"]), ref["dw_router"], dt, f"{cfg.name} dw_router",
                               ref["dw_router_rss"]),
           "d_bias": _close(f64(grads["d_router_bias"]), ref["d_router_bias"], dt, f"{cfg.name} d_bias",
                            ref["d_router_bias_rss"])}
    kept = np.minimum(g["expert_count"], C)
    experts = range(cfg.num_experts) if sample_experts is None else sample_experts
    wi_ref = np.stack([ref["dw_in"][i] for i in experts])
    wo_ref = np.stack([ref["dw_out"][i] for i in experts])
    wi = np.stack([f64(grads["dw_in"][i]) for i in experts])
    wo = np.stack([f64(grads["dw_out"][i]) for i in experts])
    wi_rss = np.stack([ref["dw_in_rss"][i] for i in experts])
    wlim = _limit(wi_ref, dt, wi_rss)
    pos = {e: n for n, e in enumerate(experts)}
    by_row = {}
    for t, items in ties.items():
        for f, e, sign, _, dw in items:
            if e in pos:
                by_row.setdefault((pos[e], f), []).append(dw)
    for (n, f), deltas in by_row.items():
        wi_ref[n, f] = _best_alternative(wi[n, f], wi_ref[n, f], deltas, wlim[n, f])
    rep["dw_in"] = _close(wi, wi_ref, dt, f"{cfg.name} dw_in", wi_rss)
    rep["dw_out"] = _close(wo, wo_ref, dt, f"{cfg.name} dw_out", np.stack([ref["dw_out_rss"][i] for i in experts]))
    for n, i in enumerate(experts):
        if kept[i] == 0:
            assert np.all(wi[n] == 0.0) and np.all(wo[n] == 0.0), f"{cfg.name}: expert {i} without rows"
    say(f"  {cfg.name}: C={C} drops={int(g['dropped'].sum())} relu near-tie tokens={len(ties)} max|err|/rms " +
        " ".join(f"{k}={v:.2e}" for k, v in rep.items()))
    return inp, C, fwd, ws, dy, grads, ref


CASES = {
    "small": SMALL,
    "small_drops": SMALL.with_(capacity_factor=0.5),
    "ragged_tokens_three_experts": SMALL.with_(num_experts=3, tokens=77),
    "router_chunks_200_experts": SMALL.with_(num_experts=200, tokens=300, capacity_factor=2.0),
    "wide_d_ff": SMALL.with_(d_ff=2816 // 4 * 4, d_model=192, tokens=700),
    "capacity_above_tile": SMALL.with_(num_experts=2, tokens=512, capacity_factor=2.0),
    # the weight gradients' resident-operand kernel takes capacities up to 160
    "capacity_160": SMALL.with_(num_experts=4, tokens=640),
    "capacity_161": SMALL.with_(num_experts=4, tokens=644),
    # d_model and d_ff of 64: half a resident block, one d_ff chunk (no pair)
    "narrow_64": SMALL.with_(num_experts=5, tokens=300, d_model=64, d_ff=64),
    # 600 (expert, 128-column) units: workgroups take several, each with an odd number of d_ff chunks
    "odd_chunks_many_units": SMALL.with_(num_experts=300, tokens=3000, d_model=256, d_ff=384),
    "fp32_ragged": SMALL.with_(dtype="f32", tokens=531, num_experts=5, d_model=64, d_ff=192),
    "fp32_many_experts": SMALL.with_(dtype="f32", tokens=400, num_experts=300, d_model=128, d_ff=128,
                                     capacity_factor=3.0),
    "tiny_fp32": CONFIGS["tiny"],
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward(name):
    _check(CASES[name].with_(name=name))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_residual(dtype):
    _check(SMALL.with_(name=f"bwd_residual_{dtype}", dtype=dtype, capacity_factor=0.5), d_aux=0.01,
           add_residual=True)


def test_backward_no_aux_term():
    _check(SMALL.with_(name="bwd_no_aux"), d_aux=0.0)


def test_backward_capacity_zero():
    """Every token dropped: the experts get exact zeros and dx is the router
    part (from the loss) alone."""
    _check(SMALL.with_(name="bwd_capacity_zero", tokens=300), capacity=0)


def test_backward_base_sampled_experts():
    """The base workload (16384 tokens, d_model 768, d_ff 3072, 128 experts):
    dx and the router gradients in full, the weight gradients of 6 sampled
    experts."""
    _check(CONFIGS["base"].with_(name="base_bwd"), d_aux=0.01, sample_experts=[0, 17, 42, 63, 100, 127])


def test_backward_xxl_sampled_experts():
    """The XXL-shaped layer (8192 tokens, d_model 4096, d_ff 10240, 64
    experts, capacity 160): 32 resident column blocks and 160 d_ff chunks per
    expert in the weight-gradient kernel; dx and the router gradients in full,
    the weight gradients of 3 sampled experts."""
    _check(CONFIGS["xxl"].with_(name="xxl_bwd"), d_aux=0.01, sample_experts=[0, 31, 63])
    torch.cuda.empty_cache()


def test_backward_deterministic_and_profiled_split():
    cfg = CONFIGS["base"].with_(tokens=4096)
    inp, C, fwd, ws, dy, a = _run(cfg)
    args = (inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"], C, fwd, ws, dy, 0.5)
    b = smx.layer_backward(*args)
    n = len(smx.BACKWARD_KERNELS)
    c = {k: torch.full_like(v, 7) for k, v in a.items()}
    shape = smx.binding.make_shape(cfg.tokens, cfg.d_model, cfg.d_ff, cfg.num_experts, C, cfg.torch_dtype)
    bws = torch.empty(smx.backward_workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    for lo, hi in ((0, 2), (3, 3), (4, n - 1)):  # one workspace: later kernels read what earlier ones wrote
        smx.layer_backward_profiled(*args, first_kernel=lo, last_kernel=hi, workspace=bws, out=c)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
        assert torch.equal(a[key], c[key]), key


def test_backward_empty_batch():
    cfg = SMALL.with_(tokens=0)
    inp = make_inputs(cfg, device=DEV)
    shape = smx.binding.make_shape(0, cfg.d_model, cfg.d_ff, cfg.num_experts, 0, cfg.torch_dtype)
    ws = torch.empty(max(smx.workspace_bytes(shape), 256), dtype=torch.uint8, device=DEV)
    out = {"expert_count": torch.zeros(cfg.num_experts, dtype=torch.int32, device=DEV),
           "aux_loss": torch.zeros(1, device=DEV)}
    for key, dt in (("expert_idx", torch.int32), ("gate", torch.float32), ("slot", torch.int32),
                    ("dropped", torch.uint8)):
        out[key] = torch.empty(0, dtype=dt, device=DEV)
    out["y"] = torch.empty(0, cfg.d_model, dtype=torch.bfloat16, device=DEV)
    smx.layer_forward_train(inp["x"], inp["w_router"], None, inp["w_in"], inp["w_out"], 0, workspace=ws, out=out)
    dy = torch.empty(0, cfg.d_model, dtype=torch.bfloat16, device=DEV)
    grads = smx.layer_backward(inp["x"], inp["w_router"], None, inp["w_in"], inp["w_out"], 0, out, ws, dy, 1.0)
    torch.cuda.synchronize()
    for key in ("dw_router", "d_router_bias", "dw_in", "dw_out"):
        assert torch.count_nonzero(grads[key]).item() == 0, key
