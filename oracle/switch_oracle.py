"""CPU oracle of the Switch FFN layer forward -- TEST INFRASTRUCTURE ONLY.

This is a plain, slow, fp64 statement of what the layer computes, written from
the Switch Transformers engineering write-up ("Switch Transformers: Scaling to
Trillion Parameter Models", sections "Switch Routing: From Top-k to k = 1",
"Expert Capacity and the Capacity Factor", "The Load-Balancing Loss" and "The
Architecture in Place").  It exists so that tests, the package's smoke check
and the benchmark's CPU-baseline leg can check and time the HIP path.  Nothing
else may import it: the product path never routes through it, and it never
imports the HIP path, its binding or its library.

Inputs are numpy arrays holding the exact values of the layer's inputs
(bf16 / fp32 values widened to float64 without rounding).  Every step is in
float64; numpy's matmul, exp, argmax and (top-k) stable argsort are the only
library primitives used.

Readings taken where the write-up leaves a step open (each is repeated at the
function that takes it):

* capacity = ceil(T * cf / N) on the exact binary64 value of cf;
* overflow is decided in token order: the lower token index wins a slot;
* argmax ties go to the lowest expert index, decided on the logits;
* f_i counts argmax choices before capacity (dropped tokens included); P_i
  averages the full softmax over all T tokens; the loss returned is
  N * sum_i f_i P_i with no alpha; T == 0 gives 0;
* expert FFN E(x) = W_out . ReLU(W_in . x), no biases;
* a dropped token's bare output is 0; with the residual flag the output is
  x + bare output;
* the block's "Add + Normalize" after the layer is layer normalisation over
  d_model of x + y (population variance, eps inside the square root, a
  per-feature scale and shift);
* the backward pass differentiates L = <dy, y> + d_aux * aux with the routing
  (expert choice, f_i, capacity drops) held fixed: f_i is a hard count with no
  gradient, so the loss reaches the router only through P_i, and the output
  reaches it only through the gate of each kept token;
* classic top-k routing (the variant the Switch layer simplifies): a token's
  k routes go to its k largest logits, in decreasing order (ties to the lower
  index); each route's gate is the full softmax p_i(x), not renormalised over
  the k chosen experts; routes claim capacity route-major (every token's
  first choice, in token order, before any second choice); the capacity is
  the caller's (k T / N x cf when each expert receives k routes' worth of
  tokens); f_i is the fraction of the k T routes that choose expert i.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py (hand-worked fixtures under tests/golden/, closed
forms, brute force and textbook special cases).
"""

from __future__ import annotations

from fractions import Fraction
from typing import Callable, Sequence

import numpy as np


# ---------------------------------------------------------------------------
# Capacity ("Expert Capacity and the Capacity Factor", the capacity equation)
# ---------------------------------------------------------------------------
def expert_capacity(tokens: int, num_experts: int, capacity_factor: float) -> int:
    """Tokens per batch / number of experts x capacity factor, rounded up.

    The write-up gives the real-valued formula only.  Reading: the buffer holds
    ceil(T * cf / N) tokens, with cf taken as its exact binary64 value (so a
    token is kept iff its 0-based position within its expert is < T*cf/N).
    """
    if tokens < 0 or num_experts < 1 or not capacity_factor > 0:
        raise ValueError("need tokens >= 0, num_experts >= 1, capacity_factor > 0")
    v = Fraction(tokens) * Fraction(capacity_factor) / num_experts
    c = v.numerator // v.denominator
    if c * v.denominator != v.numerator:
        c += 1
    return int(c)


# ---------------------------------------------------------------------------
# Router ("Switch Routing": logits h(x) = W_r . x and the softmax equation)
# ---------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """h[t, i] = sum_k W_r[i, k] x[t, k] (+ b_i) for x [T][d], W_r [N][d]."""
    h = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        h = h + np.asarray(bias, np.float64)[None, :]
    return h


def softmax(h: np.ndarray) -> np.ndarray:
    """p_i = e^{h_i} / sum_j e^{h_j}, evaluated as e^{h_i - m} / sum_j e^{h_j - m}."""
    m = h.max(axis=1, keepdims=True)
    e = np.exp(h - m)
    return e / e.sum(axis=1, keepdims=True)


def top1(h: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Switch routing picks one expert per token: the argmax of p(x).

    softmax is strictly increasing in each logit, so the argmax of p equals
    the argmax of h; ties (silent in the write-up) go to the lowest index.
    Also returns each token's gap between its largest and second-largest
    logit (0 when N == 1 would be meaningless, so +inf there), which decides
    whether a routing decision is a near-tie.
    """
    e = np.argmax(h, axis=1).astype(np.int64)  # numpy returns the first maximum
    if h.shape[1] == 1:
        gap = np.full(h.shape[0], np.inf)
    else:
        top2 = np.partition(h, h.shape[1] - 2, axis=1)[:, -2:]
        gap = top2[:, 1] - top2[:, 0]
    return e, gap


# ---------------------------------------------------------------------------
# Capacity assignment ("Expert Capacity": overflow tokens are dropped)
# ---------------------------------------------------------------------------
def assign_slots(expert_idx: np.ndarray, num_experts: int, capacity: int):
    """Position of each token inside its expert's buffer, in token order.

    slot[t] = number of earlier tokens t' < t routed to the same expert;
    dropped[t] = slot[t] >= capacity.  Also returns count[i], the number of
    tokens routed to expert i before capacity is applied.
    """
    T = len(expert_idx)
    seen = [0] * num_experts
    slot = np.empty(T, np.int64)
    for t in range(T):
        i = int(expert_idx[t])
        slot[t] = seen[i]
        seen[i] += 1
    dropped = slot >= capacity
    return slot, dropped, np.asarray(seen, np.int64)


# ---------------------------------------------------------------------------
# Load-balancing loss ("The Load-Balancing Loss", loss and f/P equations)
# ---------------------------------------------------------------------------
def load_balancing_loss(expert_idx: np.ndarray, probs: np.ndarray, num_experts: int) -> float:
    """N * sum_i f_i * P_i (the coefficient alpha is left to the caller).

    f_i = (1/T) #{t : argmax p(x_t) = i}  -- before capacity, drops included;
    P_i = (1/T) sum_t p_i(x_t)            -- full softmax over every token.
    """
    T = len(expert_idx)
    if T == 0:
        return 0.0
    f = np.zeros(num_experts)
    for i in range(num_experts):
        f[i] = np.count_nonzero(expert_idx == i) / T
    P = probs.sum(axis=0) / T
    return float(num_experts * np.sum(f * P))


# ---------------------------------------------------------------------------
# Experts and combine ("The Core Idea": N independent FFNs; combine equation)
# ---------------------------------------------------------------------------
def expert_ffn(x_e: np.ndarray, w_in_e: np.ndarray, w_out_e: np.ndarray) -> np.ndarray:
    """E(x) = W_out . ReLU(W_in . x) for rows x of x_e [M][d].

    W_in_e is [d_ff][d] and W_out_e is [d][d_ff] (each output feature's
    weights contiguous).
    """
    hid = np.maximum(np.asarray(x_e, np.float64) @ np.asarray(w_in_e, np.float64).T, 0.0)
    return hid @ np.asarray(w_out_e, np.float64).T


WeightSource = Callable[[int], tuple]


def _weights(w_in, w_out) -> WeightSource:
    if callable(w_in):
        return w_in
    return lambda i: (w_in[i], w_out[i])


def forward(x: np.ndarray, w_router: np.ndarray, router_bias, w_in, w_out,
            capacity: int, add_residual: bool = False,
            expert_idx: np.ndarray | None = None,
            experts: Sequence[int] | None = None) -> dict:
    """The whole Switch layer forward for a batch of T tokens.

    w_in / w_out are indexable by expert ([N][d_ff][d] and [N][d][d_ff]
    arrays), or w_in is a callable i -> (W_in_i, W_out_i) and w_out is None.
    expert_idx, when given, replaces the oracle's own top-1 choice ("fed"
    mode): gates, slots, drops, the loss and y then follow that routing.
    experts, when given, restricts the FFN to those experts; rows of tokens
    routed elsewhere are NaN in y.

    The combine equation y = sum_{i in T} p_i(x) E_i(x) with k = 1 is
    y = p_e(x) E_e(x); a dropped token's computation is skipped, so its bare
    output is 0 and it continues only through the residual.
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    N = w_router.shape[0]
    h = router_logits(x, w_router, router_bias)
    p = softmax(h) if T else np.zeros((0, N))
    own_idx, gap = top1(h) if T else (np.zeros(0, np.int64), np.zeros(0))
    idx = own_idx if expert_idx is None else np.asarray(expert_idx, np.int64)
    gate = p[np.arange(T), idx]
    slot, dropped, count = assign_slots(idx, N, capacity)
    aux = load_balancing_loss(idx, p, N)

    get = _weights(w_in, w_out)
    y_bare = np.zeros((T, d))
    todo = range(N) if experts is None else experts
    if experts is not None:
        y_bare[:] = np.nan
        y_bare[dropped] = 0.0
    for i in todo:
        rows = np.nonzero((idx == i) & ~dropped)[0]
        if experts is not None:
            y_bare[rows] = 0.0
        if len(rows) == 0:
            continue
        wi, wo = get(i)
        y_bare[rows] = gate[rows, None] * expert_ffn(x[rows], wi, wo)
    y = x + y_bare if add_residual else y_bare
    return {
        "logits": h, "probs": p, "expert_idx": idx, "own_expert_idx": own_idx,
        "gap": gap, "gate": gate, "slot": slot, "dropped": dropped,
        "expert_count": count, "aux_loss": aux, "y_bare": y_bare, "y": y,
    }


def dispatch(x: np.ndarray, expert_idx: np.ndarray, slot: np.ndarray, dropped: np.ndarray,
             num_experts: int, capacity: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-expert buffers [N][C][d]: row slot[t] of expert e[t] holds x[t] for
    every kept token.  Returns the buffers and a [N][C] mask of filled rows
    (rows past an expert's kept count are padding and hold no value)."""
    T, d = x.shape
    buf = np.zeros((num_experts, capacity, d))
    filled = np.zeros((num_experts, capacity), bool)
    for t in range(T):
        if not dropped[t]:
            buf[expert_idx[t], slot[t]] = x[t]
            filled[expert_idx[t], slot[t]] = True
    return buf, filled


def combine(expert_out: np.ndarray, expert_idx: np.ndarray, slot: np.ndarray,
            dropped: np.ndarray, gate: np.ndarray, x_residual: np.ndarray | None = None) -> np.ndarray:
    """y[t] = gate[t] * expert_out[e[t]][slot[t]] for kept tokens, 0 for dropped
    ones; plus x[t] for every token when a residual is given."""
    T = len(expert_idx)
    d = expert_out.shape[2]
    y = np.zeros((T, d))
    for t in range(T):
        if not dropped[t]:
            y[t] = gate[t] * np.asarray(expert_out[expert_idx[t], slot[t]], np.float64)
    if x_residual is not None:
        y = y + np.asarray(x_residual, np.float64)
    return y


# ---------------------------------------------------------------------------
# Block epilogue ("The Architecture in Place": the Add + Normalize box after
# the Switch FFN layer)
# ---------------------------------------------------------------------------
def add_normalize(x: np.ndarray, y: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    """out[t] = (v[t] - mean v[t]) / sqrt(var v[t] + eps) * gamma + beta with
    v = x + y (the residual add) and the mean and population variance taken
    over d_model.  Reading: the write-up names the box only; it is taken to be
    layer normalisation with a per-feature scale gamma and shift beta."""
    v = np.asarray(x, np.float64) + np.asarray(y, np.float64)
    mu = v.mean(axis=1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=1, keepdims=True)
    return (v - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


# ---------------------------------------------------------------------------
# Classic top-k routing ("Switch Routing: From Top-k to k = 1": the router
# sends each token to its top-k experts and the output is the gate-weighted
# sum over that set)
# ---------------------------------------------------------------------------
def topk_choice(h: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """The k experts with the largest logits, best first: idx [k][T].

    Order: larger logit first, the lower expert index first among equal
    logits (a stable sort of -h).  Also returns, per token, the smallest gap
    between consecutive logits among the min(k + 1, N) largest (+inf for
    N == 1): below it a rounding difference can change the chosen set or its
    order.
    """
    T, N = h.shape
    if not 1 <= k <= N:
        raise ValueError("need 1 <= k <= N")
    order = np.argsort(-h, axis=1, kind="stable")
    idx = order[:, :k].T.astype(np.int64).copy()
    m = min(k + 1, N)
    top = np.take_along_axis(h, order[:, :m], axis=1)
    gap = np.min(top[:, :-1] - top[:, 1:], axis=1) if m > 1 else np.full(T, np.inf)
    return idx, gap


def assign_slots_topk(expert_idx: np.ndarray, num_experts: int, capacity: int):
    """Slots of the k routes of every token, route-major.

    The routes are ranked (route 0 of tokens 0..T-1, then route 1 of tokens
    0..T-1, ...); a route's slot is the number of earlier-ranked routes to
    the same expert and it is dropped when that reaches the capacity.  With
    the routes laid out [k][T] that order is the flattened order, so this is
    the token-order assignment applied to the k T routes.  Returns slot and
    dropped [k][T] and count [N] (routes per expert before capacity).
    """
    k, T = expert_idx.shape
    slot, dropped, count = assign_slots(expert_idx.reshape(-1), num_experts, capacity)
    return slot.reshape(k, T), dropped.reshape(k, T), count


def load_balancing_loss_topk(expert_idx: np.ndarray, probs: np.ndarray, num_experts: int) -> float:
    """N * sum_i f_i P_i with f_i = (routes choosing i) / (k T) and P_i the
    batch mean of p_i(x); k = 1 gives the Switch loss."""
    k, T = expert_idx.shape
    if T == 0:
        return 0.0
    f = np.zeros(num_experts)
    for i in range(num_experts):
        f[i] = np.count_nonzero(expert_idx == i) / (k * T)
    P = probs.sum(axis=0) / T
    return float(num_experts * np.sum(f * P))


def forward_topk(x: np.ndarray, w_router: np.ndarray, router_bias, w_in, w_out, capacity: int, k: int,
                 add_residual: bool = False, expert_idx: np.ndarray | None = None) -> dict:
    """Top-k MoE layer: y[t] = sum over the token's kept routes r of
    p_{e_r}(x) E_{e_r}(x) (+ x with the residual flag).

    expert_idx [k][T], when given, replaces the oracle's own choice ("fed"
    mode).  Outputs as forward(), with the routing arrays [k][T].
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    N = w_router.shape[0]
    h = router_logits(x, w_router, router_bias)
    p = softmax(h) if T else np.zeros((0, N))
    own_idx, gap = topk_choice(h, k) if T else (np.zeros((k, 0), np.int64), np.zeros(0))
    idx = own_idx if expert_idx is None else np.asarray(expert_idx, np.int64).reshape(k, T)
    gate = np.empty((k, T))
    for r in range(k):
        gate[r] = p[np.arange(T), idx[r]]
    slot, dropped, count = assign_slots_topk(idx, N, capacity)
    aux = load_balancing_loss_topk(idx, p, N)

    get = _weights(w_in, w_out)
    y_bare = np.zeros((T, d))
    for i in range(N):
        for r in range(k):
            rows = np.nonzero((idx[r] == i) & ~dropped[r])[0]
            if len(rows) == 0:
                continue
            wi, wo = get(i)
            y_bare[rows] += gate[r, rows, None] * expert_ffn(x[rows], wi, wo)
    y = x + y_bare if add_residual else y_bare
    return {
        "logits": h, "probs": p, "expert_idx": idx, "own_expert_idx": own_idx,
        "gap": gap, "gate": gate, "slot": slot, "dropped": dropped,
        "expert_count": count, "aux_loss": aux, "y_bare": y_bare, "y": y,
    }


# ---------------------------------------------------------------------------
# Backward pass ("Switch Routing": the gate multiplies the expert output, so
# the router stays differentiable with one expert; "The Load-Balancing Loss":
# f_i is a hard count with no gradient, P_i is differentiable)
# ---------------------------------------------------------------------------
def softmax_backward(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dL/dh from dL/dp through p = softmax(h): p * (dp - <dp, p>) per row
    (the softmax Jacobian diag(p) - p p^T applied to dp)."""
    return p * (dp - np.sum(dp * p, axis=1, keepdims=True))


def expert_backward(x_e: np.ndarray, w_in_e: np.ndarray, w_out_e: np.ndarray, dy_e: np.ndarray,
                    gate_e: np.ndarray):
    """Backward of y = g W_out ReLU(W_in x) for the rows of one expert.

    Returns (dL/dg per row, dW_in, dW_out, dL/dx rows): with u = W_in x,
    h = ReLU(u), o = W_out h: dL/dg = <dy, o>, dL/do = g dy, dW_out =
    sum (g dy) h^T, dL/du = (W_out^T g dy) * [u > 0], dW_in = sum dL/du x^T,
    dL/dx = W_in^T dL/du.
    """
    u = x_e @ w_in_e.T
    h = np.maximum(u, 0.0)
    o = h @ w_out_e.T
    dgate = np.sum(dy_e * o, axis=1)
    do = gate_e[:, None] * dy_e
    du = (do @ w_out_e) * (u > 0)
    return dgate, du.T @ x_e, do.T @ h, du @ w_in_e


def backward(x: np.ndarray, w_router: np.ndarray, router_bias, w_in, w_out, capacity: int,
             dy: np.ndarray, d_aux: float, add_residual: bool = False,
             expert_idx: np.ndarray | None = None, weight_grads_for: Sequence[int] | None = None) -> dict:
    """Gradients of L = sum_t <dy_t, y_t> + d_aux * aux with respect to x,
    W_r, the router bias, W_in and W_out, for the Switch layer (k = 1).

    The routing (expert choice, capacity drops, the counts f_i) is held fixed
    at the forward's values; expert_idx, when given, replaces the oracle's own
    choice as in forward().  Kept tokens go through expert_backward with their
    expert's weights.  Router: dL/dp_i(x_t) = d_aux N f_i / T (from P_i)
    + [i = e, kept] dL/dg; dL/dh_t = softmax_backward(p, dL/dp); dW_r = sum_t
    dL/dh_t x_t^T, dbias = sum_t dL/dh_t, dx_t += W_r^T dL/dh_t.  A dropped
    token's bare output is 0, so only the loss term reaches its router.  With
    the residual, dx_t += dy_t.  weight_grads_for, when given, keeps the
    weight gradients of those experts only (the others are None); every
    expert's rows still feed dx and the router.

    Also returned, for the gradients that are sums over tokens, the root sum
    of squares of their terms (d_router_bias_rss, dw_router_rss, dw_in_rss,
    dw_out_rss): the scale of the rounding error such a sum can carry when its
    terms carry independent relative errors, whatever cancellation the sum
    itself has.
    """
    fwd = forward(x, w_router, router_bias, w_in, w_out, capacity, add_residual=add_residual,
                  expert_idx=expert_idx)
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    T, d = x.shape
    N = w_router.shape[0]
    get = _weights(w_in, w_out)
    idx, dropped, gate, p = fwd["expert_idx"], fwd["dropped"], fwd["gate"], fwd["probs"]
    dx = dy.copy() if add_residual else np.zeros((T, d))
    dgate = np.zeros(T)
    dw_in, dw_out, dw_in_rss, dw_out_rss = [], [], [], []
    for i in range(N):
        wi, wo = get(i)
        wi = np.asarray(wi, np.float64)
        wo = np.asarray(wo, np.float64)
        rows = np.nonzero((idx == i) & ~dropped)[0]
        keep = weight_grads_for is None or i in weight_grads_for
        if len(rows):
            dg, gi, go, dxr = expert_backward(x[rows], wi, wo, dy[rows], gate[rows])
            dgate[rows] = dg
            dx[rows] += dxr
            if keep:  # term scales: du_t x_t^T and (g dy_t) h_t^T
                u = x[rows] @ wi.T
                du = ((gate[rows, None] * dy[rows]) @ wo) * (u > 0)
                ri = np.sqrt((du ** 2).T @ (x[rows] ** 2))
                ro = np.sqrt(((gate[rows, None] * dy[rows]) ** 2).T @ (np.maximum(u, 0.0) ** 2))
        else:
            gi, go = np.zeros_like(wi), np.zeros_like(wo)
            ri, ro = np.zeros_like(wi), np.zeros_like(wo)
        dw_in.append(gi if keep else None)
        dw_out.append(go if keep else None)
        dw_in_rss.append(ri if keep else None)
        dw_out_rss.append(ro if keep else None)
    if T:
        f = np.bincount(idx, minlength=N) / T
        dp = np.tile(d_aux * N * f / T, (T, 1))
        kept = np.nonzero(~dropped)[0]
        dp[kept, idx[kept]] += dgate[kept]
        dh = softmax_backward(p, dp)
    else:
        dh = np.zeros((0, N))
    dw_r = dh.T @ x
    db = dh.sum(axis=0)
    dx += dh @ np.asarray(w_router, np.float64)
    return {"dx": dx, "dw_router": dw_r, "d_router_bias": db, "dw_in": dw_in, "dw_out": dw_out,
            "dgate": dgate, "dlogits": dh, "forward": fwd,
            "d_router_bias_rss": np.sqrt((dh ** 2).sum(axis=0)), "dw_router_rss": np.sqrt((dh ** 2).T @ (x ** 2)),
            "dw_in_rss": dw_in_rss, "dw_out_rss": dw_out_rss}
