"""Seeded synthetic inputs for the Switch FFN layer forward.

This module only draws numbers: token representations x, router weights W_r,
an optional router bias, and the expert weights W_in / W_out.  It holds none
of the layer's own arithmetic (no logits, softmax, routing, capacity or FFN),
so the HIP path's tests and benchmark and the CPU oracle's tests can both take
their inputs from it.  It imports nothing else from this package.

Recipe (Switch Transformers write-up, "Making Sparse Training Stable", smaller
initialization paragraph: weights come from a truncated normal whose scale is
10x below the default):

* x ~ N(0, 1), rounded to the activation dtype (RNE for bf16).
* W_r, W_in, W_out ~ normal with std = sqrt(0.1 / fan_in), truncated at +-2 std;
  fan_in is d_model for W_r and W_in and d_ff for W_out.  W_r stays fp32
  (selective precision: the router runs in fp32); W_in / W_out are rounded to
  the activation dtype.
* Zipf-skewed workload: a per-expert router bias b_i = a * log q_{pi(i)} with
  q_r proportional to r^-s (r = 1..N) and pi a seeded permutation of the
  experts.  a is the Gumbel scale of the largest of N logits, sigma_h / (N *
  phi(Phi^-1(1 - 1/N))), with sigma_h the logit std implied by the init.  If
  the logits were exactly Gumbel, the argmax would pick expert i with
  probability q_{pi(i)}; with Gaussian logits popularity is Zipf-shaped but
  flatter at the head.  The bias only exists to force overflow drops; the
  achieved popularity is measured, not assumed.

x, W_r and the bias are always drawn on the CPU (so routing inputs are the
same bits whatever device runs the layer) and then moved; the large expert
weights are drawn directly on the target device, expert block by expert block.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

__all__ = ["LayerConfig", "CONFIGS", "make_inputs", "zipf_router_bias"]


@dataclass(frozen=True)
class LayerConfig:
    name: str
    tokens: int
    d_model: int
    d_ff: int
    num_experts: int
    capacity_factor: float
    dtype: str  # "f32" or "bf16": x, W_in, W_out, dispatched, expert_out, y
    zipf_s: float | None = None
    seed: int = 0

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The five workloads.  Expert counts 64 and 2048 follow the Switch-XXL and
# Switch-C rows of the write-up's model table ("Scaling to a Trillion
# Parameters"); capacity factors 1.0 / 1.25 are the ones it reports as best.
CONFIGS = {
    "tiny": LayerConfig("tiny", 512, 64, 256, 8, 1.0, "f32"),
    "base": LayerConfig("base", 16384, 768, 3072, 128, 1.25, "bf16"),
    "large": LayerConfig("large", 16384, 1024, 2816, 128, 1.0, "bf16", zipf_s=1.1),
    "xxl": LayerConfig("xxl", 8192, 4096, 10240, 64, 1.25, "bf16"),
    "many": LayerConfig("many", 32768, 2048, 6144, 2048, 1.0, "bf16"),
}

_TRUNC = 2.0  # truncation at +-2 std
# Variance of a standard normal truncated to [-2, 2]:
# 1 - 2 * 2 * phi(2) / (2 * Phi(2) - 1).
_TRUNC_VAR = 1.0 - 4.0 * math.exp(-2.0) / math.sqrt(2.0 * math.pi) / math.erf(_TRUNC / math.sqrt(2.0))

# Distinct sub-seeds per drawn tensor.
_S_X, _S_WR, _S_WIN, _S_WOUT, _S_PERM = 1, 2, 3, 4, 5


def _gen(seed: int, which: int, device: str | torch.device = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + which * 7919)
    return g


def _trunc_normal_(t: torch.Tensor, std: float, g: torch.Generator) -> torch.Tensor:
    return torch.nn.init.trunc_normal_(t, 0.0, std, -_TRUNC * std, _TRUNC * std, generator=g)


def _norm_ppf(p: float) -> float:
    # Inverse of the standard normal CDF by bisection on math.erf (no scipy).
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * (1.0 + math.erf(mid / math.sqrt(2.0))) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def zipf_router_bias(num_experts: int, d_model: int, s: float, seed: int,
                     weight_scale: float = 0.1) -> torch.Tensor:
    """fp32 [N] router bias whose argmax popularity is Zipf(s)-shaped (see module doc)."""
    n = num_experts
    ranks = torch.arange(1, n + 1, dtype=torch.float64)
    q = ranks.pow(-s)
    q = q / q.sum()
    perm = torch.randperm(n, generator=_gen(seed, _S_PERM))
    sigma_h = math.sqrt(d_model * (weight_scale / d_model) * _TRUNC_VAR)  # Var(x) = 1
    if n > 1:
        b_n = _norm_ppf(1.0 - 1.0 / n)
        phi = math.exp(-0.5 * b_n * b_n) / math.sqrt(2.0 * math.pi)
        a = sigma_h / (n * phi)
    else:
        a = 0.0
    b = a * torch.log(q[perm])
    b = b - b.max()
    return b.to(torch.float32)


def make_inputs(cfg: LayerConfig, device: str | torch.device = "cpu",
                weight_scale: float = 0.1, chunk_elems: int = 1 << 26) -> dict:
    """Draw one layer's inputs.  Returns a dict of torch tensors:

    x [T][d] (cfg dtype), w_router [N][d] fp32, router_bias [N] fp32 or None,
    w_in [N][d_ff][d] (cfg dtype), w_out [N][d][d_ff] (cfg dtype).
    """
    T, d, f, n = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.num_experts
    dt = cfg.torch_dtype
    dev = torch.device(device)

    x = torch.randn(T, d, generator=_gen(cfg.seed, _S_X)).to(dt)
    w_r = torch.empty(n, d, dtype=torch.float32)
    _trunc_normal_(w_r, math.sqrt(weight_scale / d), _gen(cfg.seed, _S_WR))
    bias = None
    if cfg.zipf_s is not None:
        bias = zipf_router_bias(n, d, cfg.zipf_s, cfg.seed, weight_scale)

    def experts(shape_rows: int, shape_cols: int, fan_in: int, which: int) -> torch.Tensor:
        out = torch.empty(n, shape_rows, shape_cols, dtype=dt, device=dev)
        g = _gen(cfg.seed, which, dev)
        per = shape_rows * shape_cols
        step = max(1, chunk_elems // per)
        std = math.sqrt(weight_scale / fan_in)
        for e0 in range(0, n, step):
            e1 = min(n, e0 + step)
            tmp = torch.empty(e1 - e0, shape_rows, shape_cols, dtype=torch.float32, device=dev)
            _trunc_normal_(tmp, std, g)
            out[e0:e1].copy_(tmp)
            del tmp
        return out

    w_in = experts(f, d, d, _S_WIN)
    w_out = experts(d, f, f, _S_WOUT)
    return {
        "x": x.to(dev),
        "w_router": w_r.to(dev),
        "router_bias": None if bias is None else bias.to(dev),
        "w_in": w_in,
        "w_out": w_out,
    }
