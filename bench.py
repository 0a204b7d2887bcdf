"""Benchmark of the Switch FFN layer forward on one MI355X.

One step = one switch_layer_forward call (router, capacity assignment, aux
loss, dispatch, expert FFN, combine) over the base workload: 16384 tokens
(32 sequences x 512), d_model 768, d_ff 3072, 128 experts, capacity factor
1.25, bf16 activations and expert weights, fp32 router, seeded synthetic
inputs already resident in HBM.  The headline times each step after a 1 GiB
read that evicts the caches (cold cache); back-to-back steps are reported
beside it.  The other workloads (tiny fp32, large with a Zipf-skewed router,
XXL-shaped, many experts) are measured in the `configs` section.  Prints one
JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Switch-layer fwd tokens/sec on 1 MI355X; expert-FFN % MFMA peak; route/dispatch % HBM"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, TFLOP/s (datasheet)
F32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector, TFLOP/s
PROFILES = os.path.join(ROOT, "profiles")
MIN_WARMUP_S = 0.25        # untimed warmup floor (seconds of steps)
FFN_SRC = {"ffn_up": os.path.join(ROOT, "sparse_mixture_experts_switch_amd", "csrc", "ffn.hip"),
           "ffn_down": os.path.join(ROOT, "sparse_mixture_experts_switch_amd", "csrc", "ffn.hip"),
           "ffn": os.path.join(ROOT, "sparse_mixture_experts_switch_amd", "csrc", "ffn_fused.hip")}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(name: str, T: int, d: int, f: int, N: int, C: int, counts, es: int = 2) -> float:
    """Bytes each kernel must move at minimum (every input byte read once,
    every output byte written once; no padding rows); es = bytes per
    activation / expert weight element."""
    kept = int(sum(min(int(c), C) for c in counts))
    active = int(sum(1 for c in counts if c > 0 and C > 0))
    nb = (T + 63) // 64  # router blocks of 64 tokens
    if name == "router":  # x, W_r, outputs, block partials (the W_r planes of bf16 layers are not counted)
        return T * d * es + N * d * 4 + T * 12 + nb * N * 8
    if name == "assign_scan":
        return nb * N * 12 + N * 8
    if name == "assign_apply":
        # slot/dropped/token map, plus the zero rows of dropped tokens
        return T * 13 + T * 4 + N * 8 + (T - kept) * d * es
    if name == "assign":  # scan and apply in one launch
        return sum(algorithmic_bytes(k, T, d, f, N, C, counts, es) for k in ("assign_scan", "assign_apply"))
    if name == "dispatch":
        return 2 * kept * d * es + T * 9
    if name == "ffn":  # both weight matrices of live experts, gathered x rows, y rows written; token, row, gate maps
        return 2 * active * f * d * es + 2 * kept * d * es + kept * 8
    if name == "ffn_up":    # W_in of live experts, gathered x rows, H written
        return active * f * d * es + kept * d * es + kept * f * es + kept * 4
    if name == "ffn_down":  # W_out of live experts, H read, y rows written
        return active * d * f * es + kept * f * es + kept * d * es + kept * 8
    if name == "combine":
        return kept * d * es + T * d * es + T * 13
    return float("nan")


def source_digest(path: str) -> str:
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def read_traffic(kernel: str, digest: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernel source changed since."""
    path = os.path.join(PROFILES, f"{kernel}_base_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            m = re.match(r"^(\w+)\s*=\s*(\S+)", line.strip())
            if m:
                vals[m.group(1)] = m.group(2)
    if vals.get("source_sha256") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, C: int, min_seconds: float = 10.0) -> dict:
    """The CPU oracle (numpy fp64, as it stands) timed on this host on the same
    workload: the whole layer forward (routing, slots, loss and every expert's
    FFN) for all tokens, repeated until at least min_seconds have elapsed.
    One more pass through the oracle's stage functions (routing + assignment
    + loss, dispatch to [N][C][d] buffers, the per-expert FFN loop, combine)
    gives a per-stage breakdown.  Inputs are converted to fp64 on the host
    before the clock starts."""
    import numpy as np
    import torch

    import oracle.switch_oracle as so

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    x, wr = f64(inp["x"]), f64(inp["w_router"])
    b = None if inp["router_bias"] is None else f64(inp["router_bias"])
    N = wr.shape[0]
    w = [(f64(inp["w_in"][i]), f64(inp["w_out"][i])) for i in range(N)]
    runs, t0 = 0, time.perf_counter()
    while True:
        so.forward(x, wr, b, lambda i: w[i], None, C)
        runs += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= min_seconds:
            break
    T = x.shape[0]
    per = elapsed / runs

    # stage breakdown (one pass)
    st = {}
    t = time.perf_counter()
    h = so.router_logits(x, wr, b)
    p = so.softmax(h)
    idx, _ = so.top1(h)
    gate = p[np.arange(T), idx]
    slot, dropped, count = so.assign_slots(idx, N, C)
    so.load_balancing_loss(idx, p, N)
    st["route_assign_loss"] = time.perf_counter() - t
    t = time.perf_counter()
    buf, _ = so.dispatch(x, idx, slot, dropped, N, C)
    st["dispatch"] = time.perf_counter() - t
    t = time.perf_counter()
    out = np.zeros_like(buf)
    for i in range(N):
        m = int(min(count[i], C))
        if m:
            out[i, :m] = so.expert_ffn(buf[i, :m], w[i][0], w[i][1])
    st["expert_ffn"] = time.perf_counter() - t
    t = time.perf_counter()
    so.combine(out, idx, slot, dropped, gate)
    st["combine"] = time.perf_counter() - t
    return {"value": T / per, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"numpy fp64 oracle, whole layer forward on the full workload ({T} tokens, all {N} "
                       f"experts), {runs} run(s) in {elapsed:.1f} s ({per:.2f} s each); BLAS threads "
                       f"{threads}, host cores available {len(os.sched_getaffinity(0))}, CPU {cpu_model()}"),
            "stages_s": {k: round(v, 4) for k, v in st.items()}}


def backward_alg_bytes(T: int, d: int, f: int, N: int, C: int, counts, splits: int) -> dict:
    """Algorithmic HBM bytes of each backward kernel: every input byte once and
    every output byte once, padding rows excluded.  R = kept rows, Ea = experts
    with a kept row (their weights are read), n_dg = partial dots per token."""
    R = sum(min(int(c), C) for c in counts)
    Ea = sum(1 for c in counts if min(int(c), C) > 0)
    n_dg = (f + 255) // 256
    kp = -(-6 * N // 64) * 64
    return {
        "bwd_dz": Ea * d * f * 2 + R * d * 2 + R * f * 2 + R * f * 2 + R * n_dg * 4 + R * 8,
        "bwd_dx": Ea * f * d * 2 + R * f * 2 + R * d * 4 + R * 4,
        "bwd_dw_out": R * d * 2 + R * f * 2 + R * 8 + N * d * f * 2,
        "bwd_dw_in": R * f * 2 + R * d * 2 + R * 4 + N * f * d * 2,
        # logits recomputed (x, W_r), dL/dh written fp32 and as six bf16 planes (Kp = 6 N padded to 64)
        "bwd_router": T * d * 2 + N * d * 4 + R * n_dg * 4 + T * 5 + N * 4 + T * N * 4 + T * kp * 2,
        # W_r split to planes, then dx = planes . planes + experts' part (kept rows) -> bf16
        "bwd_router_dx": N * d * 4 + kp * d * 2 + T * kp * 2 + kp * d * 2 + R * d * 4 + T + T * d * 2,
        "bwd_router_w": T * N * 4 + T * d * 2 + splits * (N * d + N) * 4,
        "bwd_router_w_sum": splits * (N * d + N) * 4 + (N * d + N) * 4,
    }


def backward_bench(smx, torch, inp, out, C, cfg, stream, steps: int) -> dict:
    T, d, f, N = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.num_experts
    dev = inp["x"].device
    shape = smx.binding.make_shape(T, d, f, N, C, cfg.torch_dtype)
    bws = torch.empty(smx.backward_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    # the training forward's own workspace: row-major weights (the layer
    # timed above may run on tiled ones, whose workspace has no W_r planes)
    ws = torch.empty(smx.workspace_bytes(shape), dtype=torch.uint8, device=dev)
    g = torch.Generator().manual_seed(5)
    dy = torch.randn(T, d, generator=g).to(cfg.torch_dtype).to(dev)
    grads = {}
    args = (inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"], C, out, ws, dy, 0.01)
    call = lambda: smx.layer_backward(*args, workspace=bws, out=grads)  # noqa: E731
    torch.cuda.synchronize()  # dy's copy (default stream) is done before the stream reads it
    with torch.cuda.stream(stream):
        # the forward of a training step, on the stream the backward runs on:
        # it leaves the token maps and hidden activations that the backward
        # reads in the workspace (allocated just above, so unwritten before)
        smx.layer_forward_train(inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"], inp["w_out"], C,
                                workspace=ws, out=out)
        call()
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < MIN_WARMUP_S:
            for _ in range(10):
                call()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        names = smx.BACKWARD_KERNELS
        part = lambda lo, hi: smx.layer_backward_profiled(*args, first_kernel=lo, last_kernel=hi,  # noqa: E731
                                                          workspace=bws, out=grads)
        kern = {}
        for i, name in enumerate(names):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            torch.cuda.synchronize()
            for e0, e1 in evs:
                if i > 0:
                    part(0, i - 1)
                e0.record(stream)
                part(i, i)
                e1.record(stream)
                if i < len(names) - 1:
                    part(i + 1, len(names) - 1)
            torch.cuda.synchronize()
            kern[name] = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
    counts = out["expert_count"].cpu().tolist()
    splits = max(1, min(64, -(-512 // ((-(-N // 64)) * (d // 64)))))
    splits = min(splits, max(1, -(-T // 256)))
    alg = backward_alg_bytes(T, d, f, N, C, counts, splits)
    kept = sum(min(int(c), C) for c in counts)
    flops = 2 * 4 * kept * d * f  # dz, dx, dW_out, dW_in: 2 kept d f each
    return {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "expert_tflop_per_s": round(flops / (sum(kern[k] for k in names[:4]) * 1e-3) / 1e12, 1),
            "kernels": {k: {"ms": round(v, 5), "alg_bytes": alg[k],
                            "GBps": round(alg[k] / (v * 1e-3) / 1e9, 1),
                            "hbm_frac": round(alg[k] / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                        for k, v in kern.items()}}


def top2_bench(smx, torch, inp, cfg, stream, steps: int, weights, tiled: bool) -> dict:
    """Classic top-2 routing on the same workload (switch_topk_layer_forward,
    capacity from 2 T so that both routes have room): whole-call time."""
    T, d, f, N = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.num_experts
    dev = inp["x"].device
    C2 = smx.capacity(2 * T, N, cfg.capacity_factor)
    shape2 = smx.binding.make_shape(T, d, f, N, C2, cfg.torch_dtype, tiled)
    ws2 = torch.empty(smx.topk_workspace_bytes(shape2, 2), dtype=torch.uint8, device=dev)
    out2 = smx.binding._route_outputs(T, N, dev, 2)
    out2["y"] = torch.empty(T, d, dtype=cfg.torch_dtype, device=dev)
    w_r, w_in, w_out = weights
    call2 = lambda: smx.topk_layer_forward(inp["x"], w_r, inp["router_bias"], w_in, w_out,  # noqa: E731
                                           C2, 2, workspace=ws2, out=out2, tiled=tiled)
    with torch.cuda.stream(stream):
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < MIN_WARMUP_S:
            for _ in range(20):
                call2()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            call2()
        b.record(stream)
        torch.cuda.synchronize()
    ms2 = a.elapsed_time(b) / steps
    kept2 = int(sum(min(int(c), C2) for c in out2["expert_count"].cpu().tolist()))
    log(f"bench: top-2 layer {ms2:.4f} ms ({T / (ms2 * 1e-3) / 1e6:.2f} Mtok/s)")
    return {"ms": round(ms2, 4), "tokens_per_s": round(T / (ms2 * 1e-3), 1), "capacity": C2,
            "route_drop_rate": round(float(out2["dropped"].float().mean().item()), 5),
            "ffn_tflop_per_s_whole_call": round(4.0 * kept2 * d * f / (ms2 * 1e-3) / 1e12, 1)}


def mfma_diag_bench(smx, torch, cfg, stream, steps: int, tiled: bool) -> dict:
    """Unranked diagnostic of the expert FFN's matrix-core use: the same
    dimensions with 4x the tokens (512 per expert, capacity 640), where each
    weight byte feeds more multiply-adds than the HBM/MFMA ridge (~315 flop/B)
    and the grouped GEMMs are bound by MFMA rather than by the weight stream.
    ffn_up / ffn_down are timed live by the event split of the layer call."""
    from sparse_mixture_experts_switch_amd.inputs import make_inputs
    dcfg = cfg.with_(name="mfma_diag", tokens=4 * cfg.tokens)
    dev = torch.device("cuda:0")
    inp = make_inputs(dcfg, device=dev)
    w_r = inp["w_router"]
    if tiled:
        w_r = smx.tile_router(w_r)
        convert_in_place(smx, torch, inp["w_in"], True)
        convert_in_place(smx, torch, inp["w_out"], True)
    T, d, f, N = dcfg.tokens, dcfg.d_model, dcfg.d_ff, dcfg.num_experts
    C = smx.capacity(T, N, dcfg.capacity_factor)
    shape = smx.binding.make_shape(T, d, f, N, C, dcfg.torch_dtype, tiled)
    ws = torch.empty(smx.workspace_bytes(shape), dtype=torch.uint8, device=dev)
    out = smx.binding._route_outputs(T, N, dev)
    out["y"] = torch.empty(T, d, dtype=dcfg.torch_dtype, device=dev)
    names = smx.launch_names(shape)
    part = lambda lo, hi: smx.layer_forward_profiled(  # noqa: E731
        inp["x"], w_r, inp["router_bias"], inp["w_in"], inp["w_out"], C, first_kernel=lo,
        last_kernel=hi, workspace=ws, out=out, tiled=tiled)
    kern = {}
    torch.cuda.synchronize()  # inputs made on the default stream are ready for the layer's stream
    with torch.cuda.stream(stream):
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < MIN_WARMUP_S:
            part(0, len(names) - 1)
            torch.cuda.synchronize()
        for i, name in enumerate(names):
            if name not in ("ffn_up", "ffn_down"):
                continue
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            for e0, e1 in evs:
                part(0, i - 1)
                e0.record(stream)
                part(i, i)
                e1.record(stream)
                if i < len(names) - 1:
                    part(i + 1, len(names) - 1)
            torch.cuda.synchronize()
            kern[name] = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
    kept = sum(min(int(c), C) for c in out["expert_count"].cpu().tolist())
    ffn_ms = kern["ffn_up"] + kern["ffn_down"]
    tflops = 4.0 * kept * d * f / (ffn_ms * 1e-3) / 1e12
    log(f"bench: MFMA diagnostic ({T} tokens, capacity {C}): ffn {ffn_ms:.4f} ms, {tflops:.1f} TFLOP/s")
    return {"tokens": T, "capacity": C, "ffn_up_ms": round(kern["ffn_up"], 5),
            "ffn_down_ms": round(kern["ffn_down"], 5), "ffn_tflop_per_s": round(tflops, 1),
            "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
            "note": "unranked: 512 tokens per expert puts the expert FFN above the HBM/MFMA ridge"}


def convert_in_place(smx, torch, w, to_tiled: bool, chunk: int = 8) -> None:
    """Expert weights [N][rows][cols] between the row-major and the tiled
    layout in their own memory, `chunk` experts at a time through a small
    buffer (the many-expert workload's weights take 103 GB: no second copy)."""
    tmp = torch.empty_like(w[:chunk])
    fn = smx.tile_weights if to_tiled else smx.untile_weights
    for i in range(0, w.shape[0], chunk):
        j = min(i + chunk, w.shape[0])
        fn(w[i:j], out=tmp[:j - i])
        w[i:j].copy_(tmp[:j - i])
    torch.cuda.synchronize()
    del tmp


def measure_layer(smx, torch, cfg, inp, stream, steps: int, warmup: int, kernels: bool = True,
                  weights=None, tiled: bool = False) -> dict:
    """Times switch_layer_forward on one workload: `steps` back-to-back steps
    after the warmup, then `steps` cold-cache steps, then (kernels=True) each
    kernel of the step bracketed by HIP events on the layer's stream.
    weights: (W_r, W_in, W_out) in the layout `tiled` declares (default:
    inp's, row-major)."""
    dev = inp["x"].device
    T, d, f, N = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.num_experts
    C = smx.capacity(T, N, cfg.capacity_factor)
    w_r, w_in, w_out = weights if weights is not None else (inp["w_router"], inp["w_in"], inp["w_out"])
    shape = smx.binding.make_shape(T, d, f, N, C, cfg.torch_dtype, tiled)
    ws = torch.empty(smx.workspace_bytes(shape), dtype=torch.uint8, device=dev)
    out = smx.binding._route_outputs(T, N, dev)
    out["y"] = torch.empty(T, d, dtype=cfg.torch_dtype, device=dev)
    call = lambda: smx.layer_forward(inp["x"], w_r, inp["router_bias"], w_in,  # noqa: E731
                                     w_out, C, workspace=ws, out=out, tiled=tiled)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        # untimed warmup: at least W steps and at least MIN_WARMUP_S seconds
        # of steps (the GPU needs a fraction of a second of load to reach its
        # steady clock; timing before that reads ~10% slow)
        warm_run, t_warm = 0, time.perf_counter()
        while warm_run < warmup or time.perf_counter() - t_warm < MIN_WARMUP_S:
            call()
            warm_run += 1
            if warm_run % 50 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        log(f"bench: {cfg.name}: warmup {warm_run} steps done; timing {steps} steps")
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        start.record(stream)
        for _ in range(steps):
            call()
        stop.record(stream)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(stop) / steps
    counts = out["expert_count"].cpu().tolist()
    drop_rate = float(out["dropped"].float().mean().item()) if T else 0.0

    # cold-cache steps: before each, a 1 GiB read evicts L2 and the 256 MB
    # MALL (a read leaves clean lines; a fill would leave ~290 MB of dirty
    # lines whose write-back the next step would pay); events bracket the
    # layer call only
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()  # filled (default stream) before the layer's stream reads it
    cold = []
    with torch.cuda.stream(stream):
        for _ in range(steps):
            scratch.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            cold.append((e0, e1))
        torch.cuda.synchronize()
    ms_cold = sum(a.elapsed_time(b) for a, b in cold) / steps
    del scratch
    log(f"bench: {cfg.name}: cold-cache step {ms_cold:.4f} ms (back-to-back {ms:.4f} ms)")

    # per-kernel durations, live: K more ordinary steps in which HIP events
    # (on the layer's stream) bracket kernel i alone -- kernels 0..i-1, event,
    # kernel i, event, kernels i+1..n-1; no kernel of the layer modifies its
    # inputs, so the split calls reproduce the ordinary step
    kern = {}
    if kernels:
        names = smx.launch_names(shape)
        n_k = len(names)
        part = lambda lo, hi: smx.layer_forward_profiled(  # noqa: E731
            inp["x"], w_r, inp["router_bias"], w_in, w_out, C, first_kernel=lo,
            last_kernel=hi, workspace=ws, out=out, tiled=tiled)
        with torch.cuda.stream(stream):
            for i, name in enumerate(names):
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(steps)]
                torch.cuda.synchronize()
                for a, b in evs:
                    if i > 0:
                        part(0, i - 1)
                    a.record(stream)
                    part(i, i)
                    b.record(stream)
                    if i < n_k - 1:
                        part(i + 1, n_k - 1)
                torch.cuda.synchronize()
                kern[name] = sum(a.elapsed_time(b) for a, b in evs) / steps
        log(f"bench: {cfg.name}: per-kernel ms " + ", ".join(f"{k}={v:.4f}" for k, v in kern.items()))
    return {"C": C, "shape": shape, "ws": ws, "out": out, "kern": kern, "ms_warm": ms, "ms_cold": ms_cold,
            "counts": counts, "drop_rate": drop_rate, "warm_run": warm_run, "t_wall": t_wall}


def near_ties_fp64(torch, inp, tol: float = 1e-4) -> dict:
    """Top-1 choice and top-2 logit gap of every token, computed on the GPU in
    fp64 with torch's own matmul (x, W_r and the bias are exact in fp64, so
    this is the router's exact logits up to fp64 rounding): the number of
    tokens whose two largest logits lie within tol of each other, where the
    fp32 router may pick either."""
    x = inp["x"].to(torch.float64)
    h = x @ inp["w_router"].to(torch.float64).t()
    if inp["router_bias"] is not None:
        h += inp["router_bias"].to(torch.float64)
    if h.shape[1] < 2:
        return {"near_ties": 0, "tol": tol}
    top = torch.topk(h, 2, dim=1).values
    n = int(((top[:, 0] - top[:, 1]) < tol).sum().item())
    del x, h
    return {"near_ties": n, "tol": tol}


def cpu_sampled(inp, C: int, n_experts: int, min_seconds: float) -> dict:
    """The CPU oracle on a workload too large to run whole: the oracle's full
    forward with its FFN restricted to a sample of experts (the routing,
    capacity assignment and loss run on every token), repeated for at least
    min_seconds; the time of the sampled experts' FFN is then scaled to all
    kept rows (the FFN costs the same per kept row) and the rest counted once:
    an extrapolation, labelled as one.  Only the sampled experts' weights are
    converted to fp64 on the host, before the clock starts."""
    import numpy as np
    import torch

    import oracle.switch_oracle as so

    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    x, wr = f64(inp["x"]), f64(inp["w_router"])
    b = None if inp["router_bias"] is None else f64(inp["router_bias"])
    T, N = x.shape[0], wr.shape[0]
    # the sample: evenly spaced experts
    sample = sorted({int(i * N / n_experts) for i in range(n_experts)})
    w = {i: (f64(inp["w_in"][i]), f64(inp["w_out"][i])) for i in sample}
    runs, t0 = 0, time.perf_counter()
    while True:
        res = so.forward(x, wr, b, lambda i: w[i], None, C, experts=sample)
        runs += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= min_seconds:
            break
    per = elapsed / runs
    idx, dropped, count = res["expert_idx"], res["dropped"], res["expert_count"]
    # the sampled experts' FFN alone, timed the same way
    rows = {i: np.nonzero((idx == i) & ~dropped)[0] for i in sample}
    t = time.perf_counter()
    for _ in range(runs):
        for i in sample:
            if len(rows[i]):
                so.expert_ffn(x[rows[i]], *w[i])
    t_ffn = (time.perf_counter() - t) / runs
    kept_s = sum(len(r) for r in rows.values())
    kept = int(np.minimum(count, C).sum())
    est = per - t_ffn + (t_ffn * kept / kept_s if kept_s else 0.0)
    threads = _blas_threads()
    return {"value": T / est, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"numpy fp64 oracle, extrapolated: routing, assignment and loss on all {T} tokens, the "
                       f"FFN of {len(sample)} of {N} experts ({kept_s} of {kept} kept rows, {t_ffn:.3f} s) "
                       f"scaled to every kept row; {runs} run(s) in {elapsed:.1f} s; BLAS threads {threads}")}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] + [1]))
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def cpu_whole(inp, C: int, min_seconds: float) -> dict:
    """The CPU oracle's whole layer forward on the full workload, repeated for
    at least min_seconds (inputs converted to fp64 before the clock)."""
    import torch

    import oracle.switch_oracle as so

    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    x, wr = f64(inp["x"]), f64(inp["w_router"])
    b = None if inp["router_bias"] is None else f64(inp["router_bias"])
    N = wr.shape[0]
    w = [(f64(inp["w_in"][i]), f64(inp["w_out"][i])) for i in range(N)]
    runs, t0 = 0, time.perf_counter()
    while True:
        so.forward(x, wr, b, lambda i: w[i], None, C)
        runs += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= min_seconds:
            break
    threads = _blas_threads()
    return {"value": x.shape[0] * runs / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"numpy fp64 oracle, whole layer forward on the full workload, {runs} run(s) in "
                       f"{elapsed:.1f} s; BLAS threads {threads}")}


# Expert sample of the CPU oracle on the workloads it cannot run whole.
CPU_SAMPLED = {"xxl": 4, "many": 16}


def configs_bench(smx, torch, stream, steps: int, warmup: int, cpu: bool, names) -> dict:
    """The layer forward on the other workloads: back-to-back and cold-cache
    step, each kernel's time and fraction of the HBM roofline on its
    algorithmic bytes, the expert FFN's useful TFLOP/s and fraction of the
    dense MFMA peak for its dtype, the drop rate, the near-tie count and the
    CPU oracle's rate (whole, or sampled and extrapolated)."""
    from sparse_mixture_experts_switch_amd.inputs import CONFIGS, make_inputs

    res = {}
    for name in names:
        cfg = CONFIGS[name]
        T, d, f, N = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.num_experts
        es = 2 if cfg.dtype == "bf16" else 4
        log(f"bench: configs: generating {cfg}")
        inp = make_inputs(cfg, device=stream.device)
        tiled = cfg.dtype == "bf16"  # bf16 layers run on tiled weights, converted before timing
        w_r = inp["w_router"]
        if tiled:
            w_r = smx.tile_router(w_r)
            convert_in_place(smx, torch, inp["w_in"], True)
            convert_in_place(smx, torch, inp["w_out"], True)
        m = measure_layer(smx, torch, cfg, inp, stream, steps, warmup, weights=(w_r, inp["w_in"], inp["w_out"]),
                          tiled=tiled)
        del w_r
        if tiled:  # back to row-major for the oracle
            convert_in_place(smx, torch, inp["w_in"], False)
            convert_in_place(smx, torch, inp["w_out"], False)
        C, kern, counts = m["C"], m["kern"], m["counts"]
        kept = int(sum(min(int(c), C) for c in counts))
        per_kernel = {}
        for k, v in kern.items():
            b = algorithmic_bytes(k, T, d, f, N, C, counts, es)
            per_kernel[k] = {"ms": round(v, 5), "GBps": round(b / (v * 1e-3) / 1e9, 1),
                             "hbm_frac": round(b / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        ffn_ms = kern.get("ffn", 0.0) + kern.get("ffn_up", 0.0) + kern.get("ffn_down", 0.0)
        ffn_tflops = 4.0 * kept * d * f / (ffn_ms * 1e-3) / 1e12 if ffn_ms else 0.0
        peak = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else F32_PEAK_TFLOPS
        rec = {"workload": (f"{T} tokens, d_model {d}, d_ff {f}, {N} experts, capacity factor "
                            f"{cfg.capacity_factor} (capacity {C}), {cfg.dtype} activations and expert weights"
                            + (" (tiled layout, router planes)" if tiled else "") + ", fp32 router"
                            + (f", Zipf({cfg.zipf_s}) router bias" if cfg.zipf_s else "")),
               "ms_per_step": round(m["ms_cold"], 4), "tokens_per_s": round(T / (m["ms_cold"] * 1e-3), 1),
               "ms_per_step_back_to_back": round(m["ms_warm"], 4),
               "tokens_per_s_back_to_back": round(T / (m["ms_warm"] * 1e-3), 1),
               "kernels": per_kernel,
               "ffn": {"ms": round(ffn_ms, 4), "tflops": round(ffn_tflops, 2),
                       "mfma_frac": round(ffn_tflops / peak, 4), "peak_tflops": peak},
               "drop_rate": round(m["drop_rate"], 5), "kept_rows": kept, **near_ties_fp64(torch, inp)}
        del m
        if cpu:
            log(f"bench: configs: {name}: timing the CPU oracle")
            rec["cpu_oracle"] = (cpu_sampled(inp, C, CPU_SAMPLED[name], 3.0) if name in CPU_SAMPLED
                                 else cpu_whole(inp, C, 3.0))
        res[name] = rec
        del inp
        torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config", default="base", help="workload (the metric is quoted on 'base')")
    ap.add_argument("--sections", default="stages,top2,mfma_diag,backward,configs",
                    help="extra measurements after the layer forward: any of stages, top2, mfma_diag, backward, "
                         "configs")
    ap.add_argument("--configs", default="tiny,large,xxl,many",
                    help="workloads of the configs section")
    ap.add_argument("--weights", choices=("tiled", "rows"), default="tiled",
                    help="expert weight layout of the timed forward calls (bf16): tiled (converted once before "
                         "timing) or row-major")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device-to-device copy (HBM counter calibration)")
    args = ap.parse_args()
    sections = set(filter(None, args.sections.split(",")))
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import torch

    import sparse_mixture_experts_switch_amd as smx
    from sparse_mixture_experts_switch_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: generating {cfg}")
    inp = make_inputs(cfg, device=dev)
    T, d, f, N = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.num_experts
    # the layer runs on a stream of its own (the legacy default stream
    # synchronises with every other stream at each launch)
    stream = torch.cuda.Stream(device=dev)
    # the weights in the layout the forward calls read: tiled (W_r's planes
    # and the expert matrices in operand order, a copy converted once, before
    # any timing: the parameters' storage format) or row-major; the backward
    # reads row-major weights
    tiled = args.weights == "tiled" and cfg.dtype == "bf16"
    wts = ((smx.tile_router(inp["w_router"]), smx.tile_weights(inp["w_in"]), smx.tile_weights(inp["w_out"]))
           if tiled else (inp["w_router"], inp["w_in"], inp["w_out"]))
    torch.cuda.synchronize()
    m = measure_layer(smx, torch, cfg, inp, stream, args.steps, args.warmup, weights=wts, tiled=tiled)
    C, shape, ws, out, kern = m["C"], m["shape"], m["ws"], m["out"], m["kern"]
    ms, ms_cold, counts, drop_rate = m["ms_warm"], m["ms_cold"], m["counts"], m["drop_rate"]
    rows_rec = None
    if tiled:  # the same step on row-major weights
        mr = measure_layer(smx, torch, cfg, inp, stream, args.steps, 0, kernels=False)
        rows_rec = {"ms_per_step": round(mr["ms_cold"], 4), "tokens_per_s": round(T / (mr["ms_cold"] * 1e-3), 1),
                    "ms_per_step_back_to_back": round(mr["ms_warm"], 4),
                    "note": "switch_layer_forward with row-major expert weights, cold-cache step as the headline"}
        del mr

    # the stage entry points' data-movement kernels on the same routing (not
    # on the layer path, which gathers and scatters inside the expert FFN):
    # switch_dispatch (x rows -> [N][C][d]) and switch_combine ([N][C][d] ->
    # y, here fed the dispatched buffer as expert output), and the block's
    # Add + Normalize after the layer (switch_add_norm), K launches each
    kept = int(sum(min(int(c), C) for c in counts))
    disp = torch.empty(N, C, d, dtype=cfg.torch_dtype, device=dev)
    gamma = torch.ones(d, device=dev)
    beta = torch.zeros(d, device=dev)
    ystage = torch.empty(T, d, dtype=cfg.torch_dtype, device=dev)
    rstage = {k: torch.empty_like(v) for k, v in out.items() if k != "y"}
    stage_ms = {}
    torch.cuda.synchronize()  # gamma and beta (filled on the default stream) are ready
    stage_fns = () if "stages" not in sections else (
        ("dispatch", lambda: smx.dispatch(inp["x"], out["expert_idx"], out["slot"], out["dropped"], N, C,
                                          out=disp)),
        ("combine", lambda: smx.combine(disp, out["expert_idx"], out["slot"], out["dropped"], out["gate"],
                                        out=ystage)),
        ("add_norm", lambda: smx.add_norm(inp["x"], out["y"], gamma, beta, 1e-6, out=ystage)),
        ("combine_add_norm", lambda: smx.combine_add_norm(disp, out["expert_idx"], out["slot"], out["dropped"],
                                                          out["gate"], inp["x"], gamma, beta, 1e-6, out=ystage)),
        # routing alone (router + assignment), and routing with the dispatch
        # copy in one pass over x (its workspace's ordering state is cleared
        # by a small kernel inside each call)
        ("route", lambda: smx.route(inp["x"], wts[0], inp["router_bias"], C, workspace=ws, out=rstage,
                                    tiled=tiled, num_experts=N)),
        ("route_dispatch", lambda: smx.route_dispatch(inp["x"], wts[0], inp["router_bias"], C, workspace=ws,
                                                      out=rstage, dispatched=disp, tiled=tiled, num_experts=N)))
    with torch.cuda.stream(stream):
        for name, fn in stage_fns:
            fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(args.steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            stage_ms[name] = a.elapsed_time(b) / args.steps
    stage_bytes = {"dispatch": 2 * kept * d * 2 + T * 9,          # read kept x rows, write them; idx/slot/drop
                   "combine": kept * d * 2 + T * d * 2 + T * 13,  # read kept rows, write every y row; + gate
                   "add_norm": 3 * T * d * 2 + 2 * d * 4,         # read x and y, write the block output
                   # read kept expert rows and x, write the block output; + gate and routing
                   "combine_add_norm": kept * d * 2 + 2 * T * d * 2 + 2 * d * 4 + T * 13,
                   # read x and W_r, write expert_idx, gate, slot, dropped (+ the kept rows)
                   "route": T * d * 2 + N * d * 4 + T * 13 + N * 8,
                   "route_dispatch": T * d * 2 + N * d * 4 + T * 13 + N * 8 + kept * d * 2}
    stage_kernels = {k: {"ms": round(v, 5), "alg_bytes": stage_bytes[k],
                         "GBps": round(stage_bytes[k] / (v * 1e-3) / 1e9, 1),
                         "hbm_frac": round(stage_bytes[k] / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                     for k, v in stage_ms.items()}
    log("bench: stage kernels " + ", ".join(f"{k}={v['GBps']} GB/s" for k, v in stage_kernels.items()))
    # the forward of a training step (switch_layer_forward_train: the expert
    # FFN as two products, the hidden activations saved for the backward)
    train_ms = None
    if "stages" in sections:
        # row-major weights: the workspace also holds W_r's split planes
        tws = torch.empty(smx.workspace_bytes(smx.binding.make_shape(T, d, f, N, C, cfg.torch_dtype)),
                          dtype=torch.uint8, device=dev)
        tout = {k: torch.empty_like(v) for k, v in out.items()}
        tcall = lambda: smx.layer_forward_train(inp["x"], inp["w_router"], inp["router_bias"], inp["w_in"],  # noqa: E731
                                                inp["w_out"], C, workspace=tws, out=tout)
        with torch.cuda.stream(stream):
            for _ in range(3):
                tcall()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(args.steps):
                tcall()
            b.record(stream)
            torch.cuda.synchronize()
        train_ms = a.elapsed_time(b) / args.steps
        log(f"bench: training-step forward (hidden activations saved) {train_ms:.4f} ms")
        del tws, tout
    # the layer with the block's Add + Normalize in the same call, back to back
    # against the bare layer timed the same way
    norm_rec = None
    if "stages" in sections:
        nout = {k: torch.empty_like(v) for k, v in out.items()}
        ncall = lambda: smx.layer_forward_add_norm(inp["x"], wts[0], inp["router_bias"],  # noqa: E731
                                                   wts[1], wts[2], C, gamma, beta, 1e-6, workspace=ws, out=nout,
                                                   tiled=tiled)
        bcall = lambda: smx.layer_forward(inp["x"], wts[0], inp["router_bias"], wts[1], wts[2],  # noqa: E731
                                          C, workspace=ws, out=nout, tiled=tiled)
        times = {}
        with torch.cuda.stream(stream):
            for name, fn in (("bare", bcall), ("add_norm", ncall), ("bare2", bcall), ("add_norm2", ncall)):
                for _ in range(3):
                    fn()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                a.record(stream)
                for _ in range(args.steps):
                    fn()
                b.record(stream)
                torch.cuda.synchronize()
                times[name] = a.elapsed_time(b) / args.steps
        bare_ms = min(times["bare"], times["bare2"])
        norm_ms = min(times["add_norm"], times["add_norm2"])
        norm_rec = {"ms_per_step": round(norm_ms, 4), "bare_ms_per_step": round(bare_ms, 4),
                    "extra_us": round((norm_ms - bare_ms) * 1e3, 2),
                    "note": "switch_layer_forward_add_norm vs switch_layer_forward, back to back, best of two runs"}
        log(f"bench: layer + Add & Normalize {norm_ms:.4f} ms, bare layer {bare_ms:.4f} ms")
        del nout
    top2 = top2_bench(smx, torch, inp, cfg, stream, args.steps, wts, tiled) if "top2" in sections else None
    # backward pass of the same step (switch_layer_backward on the forward's
    # routing and saved workspace; dy ~ N(0, 1), d_aux = 0.01): whole-call
    # time, then each kernel bracketed by events as for the forward
    diag = mfma_diag_bench(smx, torch, cfg, stream, args.steps, tiled) if "mfma_diag" in sections else None
    bwd = None
    if "backward" in sections:
        bwd = backward_bench(smx, torch, inp, out, C, cfg, stream, args.steps)
        log("bench: backward " + f"{bwd['ms']:.4f} ms; per-kernel ms " +
            ", ".join(f"{k}={v['ms']:.4f}" for k, v in bwd["kernels"].items()))
    per_kernel = {}
    for k, v in kern.items():
        b = algorithmic_bytes(k, T, d, f, N, C, counts)
        per_kernel[k] = {"ms": round(v, 5), "alg_bytes": b, "GBps": round(b / (v * 1e-3) / 1e9, 1),
                         "hbm_frac": round(b / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # the dominant kernel: the fused expert FFN, or the larger of its two products
    dom = "ffn" if "ffn" in kern else max(("ffn_up", "ffn_down"), key=lambda k: kern.get(k, 0.0))
    dom_b = algorithmic_bytes(dom, T, d, f, N, C, counts)
    achieved = dom_b / (kern[dom] * 1e-3) / 1e9
    kept = sum(min(c, C) for c in counts)
    ffn_ms = sum(kern.get(k, 0.0) for k in ("ffn", "ffn_up", "ffn_down"))
    ffn_tflops = 4.0 * kept * d * f / (ffn_ms * 1e-3) / 1e12
    rdc = [k for k in ("router", "assign", "assign_scan", "assign_apply") if k in kern]
    rdc_b = sum(algorithmic_bytes(k, T, d, f, N, C, counts) for k in rdc)
    rdc_ms = sum(kern[k] for k in rdc)
    res = {
        "metric": METRIC,
        "value": T / (ms_cold * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": m["warm_run"],
        "ms_per_step": ms_cold,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens, truncated-normal 0.1-scale weights; no dataset)",
        "config": {"workload": f"{cfg.name}: {T} tokens (32 seqs x 512), d_model {d}, d_ff {f}, {N} experts, "
                               f"capacity factor {cfg.capacity_factor} (capacity {C}), bf16 activations and "
                               f"expert weights" + (" (tiled layout, router planes)" if tiled else "") + ", fp32 router",
                   "tokens": T, "d_model": d, "d_ff": f, "num_experts": N, "capacity": C,
                   "drop_rate": round(drop_rate, 5),
                   "weight_layout": "tiled" if tiled else "row-major"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(dom, source_digest(FFN_SRC[dom]))},
        "ffn": {"ms": round(ffn_ms, 4), "tflops": round(ffn_tflops, 1),
                "mfma_frac": round(ffn_tflops / BF16_PEAK_TFLOPS, 4)},
        "route": {"ms": round(rdc_ms, 4), "alg_bytes": rdc_b,
                                   "hbm_frac": round(rdc_b / (rdc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "kernels": per_kernel,
        "stage_kernels": stage_kernels,
        "top2": top2,
        "mfma_diagnostic": diag,
        "backward": bwd,
        "timing": ("value and ms_per_step: each of the K steps after a 1 GiB read that evicts L2 and the MALL, "
                   "HIP events around the layer call; back_to_back: K steps in a row (x and W_r may stay in "
                   "the MALL; the 1.2 GB of expert weights cannot)"),
        "back_to_back": {"ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
                         "wall_s_timed": round(m["t_wall"], 4)},
        "row_major_weights": rows_rec,
        "train_forward": None if train_ms is None else {
            "ms_per_step": round(train_ms, 4), "tokens_per_s": round(T / (train_ms * 1e-3), 1),
            "note": ("switch_layer_forward_train, back to back, row-major expert weights (those the backward "
                     "reads): the expert FFN as two products with H saved")},
        "layer_add_norm": norm_rec,
        "configs": None,
    }
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(inp, C)
    else:
        res["cpu_baseline"] = None
    if "configs" in sections:
        del inp, m, ws, out, wts
        torch.cuda.empty_cache()
        res["configs"] = configs_bench(smx, torch, stream, args.steps, args.warmup, not args.no_cpu_baseline,
                                       [c for c in args.configs.split(",") if c and c != args.config])
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
