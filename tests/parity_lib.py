"""Helpers shared by the GPU parity tests: run the HIP path through the
binding, run the CPU oracle on the same input bits, compare under the
layer's tolerances.

Tolerances (stated once here, used by every parity test):
* expert_idx equal, except tokens whose oracle top-2 logit gap is below
  NEAR_TIE (1e-4): those may go either way and are counted;
* slot, dropped, expert_count bit-exact against the oracle fed the GPU's
  expert_idx (and against the standalone oracle when nothing flipped);
* gate |gpu - oracle| <= 1e-6 + 1e-5 * oracle (fp32 router, ~1e-7 rounding
  per operation over <= 2048 terms);
* aux_loss relative error <= 1e-4;
* y (bare output): per element |err| <= 2e-2 * rms(y_oracle) + u * |y_oracle|
  in bf16 (u = 2^-8, the largest relative error of one round-to-nearest into
  bf16: the output is stored in bf16, so no implementation can beat one
  rounding of the exact value), and <= 1e-4 * rms(y_oracle) + 2^-24 |y_oracle|
  in fp32; rms over the rows the experts produced (kept tokens: dropped rows
  are checked separately and must be exactly 0 (bare) or exactly x
  (residual), so their zeros do not shrink the bound).  The report also gives
  the plain max |err| / rms.
"""

from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import torch

import oracle.switch_oracle as so
import sparse_mixture_experts_switch_amd as smx

NEAR_TIE = 1e-4
GATE_ABS, GATE_REL = 1e-6, 1e-5
AUX_REL = 1e-4
Y_TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
Y_ROUND = {torch.bfloat16: 2.0 ** -8, torch.float32: 2.0 ** -24}


def say(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def weight_source(inp: dict):
    """Oracle weight source: downloads expert i's weights on demand."""
    def get(i):
        return f64(inp["w_in"][i]), f64(inp["w_out"][i])
    return get


def oracle_run(inp: dict, capacity: int, expert_idx=None, experts=None, add_residual=False) -> dict:
    x = f64(inp["x"])
    wr = f64(inp["w_router"])
    b = None if inp["router_bias"] is None else f64(inp["router_bias"])
    return so.forward(x, wr, b, weight_source(inp), None, capacity, add_residual=add_residual,
                      expert_idx=expert_idx, experts=experts)


def gpu_outputs_numpy(o: dict) -> dict:
    out = {k: v.cpu().numpy() for k, v in o.items() if k != "y"}
    if "y" in o:
        out["y"] = f64(o["y"])
    out["dropped"] = out["dropped"].astype(bool)
    out["aux_loss"] = float(out["aux_loss"][0])
    return out


def check_routing(g: dict, own: dict, fed: dict, label: str) -> dict:
    """Routing parity; returns counts for the report."""
    e_gpu, e_orc, gap = g["expert_idx"].astype(np.int64), own["expert_idx"], own["gap"]
    flips = np.nonzero(e_gpu != e_orc)[0]
    bad = flips[gap[flips] >= NEAR_TIE]
    assert len(bad) == 0, (f"{label}: {len(bad)} routing mismatches outside near-ties, first t={bad[:5]}, "
                           f"gaps={gap[bad[:5]]}")
    near = int(np.sum(gap < NEAR_TIE))
    assert np.array_equal(g["slot"].astype(np.int64), fed["slot"]), f"{label}: slot differs from fed oracle"
    assert np.array_equal(g["dropped"], fed["dropped"]), f"{label}: dropped differs from fed oracle"
    assert np.array_equal(g["expert_count"].astype(np.int64), fed["expert_count"]), f"{label}: expert_count"
    if len(flips) == 0:
        assert np.array_equal(g["slot"].astype(np.int64), own["slot"])
        assert np.array_equal(g["dropped"], own["dropped"])
    gate_err = np.abs(g["gate"].astype(np.float64) - fed["gate"])
    lim = GATE_ABS + GATE_REL * fed["gate"]
    assert np.all(gate_err <= lim), f"{label}: gate err max {gate_err.max():.3e} (worst rel {(gate_err / lim).max():.2f})"
    aux_rel = abs(g["aux_loss"] - fed["aux_loss"]) / max(abs(fed["aux_loss"]), 1e-30)
    assert aux_rel <= AUX_REL, f"{label}: aux {g['aux_loss']} vs {fed['aux_loss']} rel {aux_rel:.2e}"
    return {"flips": int(len(flips)), "near_ties": near, "drop_rate": float(fed["dropped"].mean()) if len(
        fed["dropped"]) else 0.0, "aux_rel": float(aux_rel), "gate_err": float(gate_err.max(initial=0.0))}


def report(label: str, rec: dict) -> None:
    """Append one parity record (JSON line) to the file SMX_PARITY_REPORT
    names, if set: the per-config error statistics of a GPU test run."""
    path = os.environ.get("SMX_PARITY_REPORT")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps({"case": label, **rec}) + "\n")


def check_y(y_gpu: np.ndarray, fed: dict, dtype: torch.dtype, label: str, x: np.ndarray | None = None,
            expect_rows: int | None = None) -> dict:
    """Bare (or residual, when x is given) output parity on the rows the
    oracle computed (rows it skipped are NaN there).

    Fails when no kept row was compared, or, with expect_rows, when the number
    of kept rows compared differs from it (a sampled check must compare
    exactly the kept tokens of its sampled experts).  Returns the number of
    kept rows compared, max |err| / rms, and how many elements exceed the
    bound without the rounding term (tol * rms alone)."""
    ref = fed["y_bare"]
    rows = ~np.isnan(ref).any(axis=1)
    dropped = fed["dropped"]
    if x is None:
        assert np.all(y_gpu[dropped] == 0.0), f"{label}: dropped rows not exactly 0"
    else:
        assert np.array_equal(y_gpu[dropped], x[dropped]), f"{label}: dropped rows differ from x"
    kept = rows & ~dropped
    n_rows = int(kept.sum())
    if expect_rows is not None:
        assert expect_rows > 0, f"{label}: the sample holds no kept token"
        assert n_rows == expect_rows, f"{label}: compared {n_rows} kept rows, expected {expect_rows}"
    assert n_rows > 0, f"{label}: no kept row compared"
    got = y_gpu[kept]
    want = ref[kept] if x is None else x[kept] + ref[kept]
    rms = float(np.sqrt(np.mean(ref[kept] ** 2)))
    diff = np.abs(got - want)
    lim = Y_TOL[dtype] * rms + Y_ROUND[dtype] * np.abs(want)
    worst = np.unravel_index(np.argmax(diff - lim), diff.shape)
    assert np.all(diff <= lim), (f"{label}: |y err| {diff[worst]:.3e} > {lim[worst]:.3e} at {worst} "
                                 f"(value {want[worst]:.3e}, rms {rms:.3e})")
    return {"rows": n_rows, "elements": int(diff.size),
            "max_err_over_rms": float(diff.max() / rms) if rms > 0 else 0.0,
            "over_strict": int(np.sum(diff > Y_TOL[dtype] * rms)), "strict_tol": Y_TOL[dtype]}
