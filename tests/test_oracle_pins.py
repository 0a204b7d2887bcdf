"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each check cites the passage of the Switch Transformers write-up it follows.
Sources of truth: hand-worked fixtures (tests/golden/), closed forms the
write-up states (the uniform-routing value of the loss), textbook routines
that compute the same thing another way (stable sort ranks, scipy's softmax,
explicit-loop matrix products), brute force over every routing of tiny
batches, and invariants (conservation of tokens, monotonicity in the capacity
factor).  The mutation tests at the end plant plausible mistakes in the oracle
and check that some pin catches each one.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle.switch_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _hand_inputs():
    g = _load("hand_layer_example.json")
    inp = g["inputs"]
    ln3 = math.log(3.0)
    x = np.array(inp["x"], np.float64)
    w_r = np.array(inp["w_router_over_ln3"], np.float64) * ln3
    w_in = np.array(inp["w_in"], np.float64)
    w_out = np.array(inp["w_out"], np.float64)
    return g, x, w_r, w_in, w_out


def _rand_layer(rng, T, d, f, N, scale=1.0):
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((N, d)) * scale
    w_in = rng.standard_normal((N, f, d)) * 0.3
    w_out = rng.standard_normal((N, d, f)) * 0.3
    return x, w_r, w_in, w_out


# ---------------------------------------------------------------- pins -----
def pin_capacity_table():
    """Capacity equation ('Expert Capacity and the Capacity Factor'), by hand."""
    for c in _load("capacity_table.json")["cases"]:
        got = so.expert_capacity(c["tokens"], c["experts"], c["cf"])
        assert got == c["capacity"], (c, got)


def pin_hand_example():
    """The whole hand-worked layer (tests/golden/hand_layer_example.json)."""
    g, x, w_r, w_in, w_out = _hand_inputs()
    exp = g["expected"]
    C = so.expert_capacity(4, 2, g["inputs"]["capacity_factor"])
    assert C == exp["capacity"]
    out = so.forward(x, w_r, None, w_in, w_out, C)
    np.testing.assert_allclose(out["probs"], exp["probs"], rtol=0, atol=1e-14)
    assert out["expert_idx"].tolist() == exp["expert_idx"]
    np.testing.assert_allclose(out["gate"], exp["gate"], rtol=0, atol=1e-14)
    assert out["slot"].tolist() == exp["slot"]
    assert out["dropped"].tolist() == exp["dropped"]
    assert out["expert_count"].tolist() == exp["expert_count"]
    assert abs(out["aux_loss"] - exp["aux_loss"]) < 1e-14
    np.testing.assert_allclose(out["y_bare"], exp["y_bare"], rtol=0, atol=1e-14)
    res = so.forward(x, w_r, None, w_in, w_out, C, add_residual=True)
    np.testing.assert_allclose(res["y"], exp["y_residual"], rtol=0, atol=1e-14)
    # the stage functions reproduce the same answer
    buf, filled = so.dispatch(x, out["expert_idx"], out["slot"], out["dropped"], 2, C)
    assert filled.tolist() == [[True, True], [True, False]]
    eo = np.zeros_like(buf)
    for i in range(2):
        eo[i] = so.expert_ffn(buf[i], w_in[i], w_out[i])
    y = so.combine(eo, out["expert_idx"], out["slot"], out["dropped"], out["gate"])
    np.testing.assert_allclose(y, exp["y_bare"], rtol=0, atol=1e-14)


def pin_softmax_library(rng):
    """Softmax equation ('Switch Routing'): scipy's softmax, sum 1, gate bounds."""
    h = rng.standard_normal((64, 9)) * 3
    p = so.softmax(h)
    np.testing.assert_allclose(p, scipy.special.softmax(h, axis=1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    e, _ = so.top1(h)
    gate = p[np.arange(64), e]
    assert np.all(gate >= 1.0 / 9 - 1e-15) and np.all(gate <= 1.0)
    # gate = 1 / sum_j e^{h_j - max h}, computed by an explicit loop
    for t in range(64):
        s = 0.0
        for j in range(9):
            s += math.exp(h[t, j] - max(h[t]))
        assert abs(gate[t] - 1.0 / s) < 1e-14


def pin_top1_bruteforce(rng):
    """Top-1 selection ('Switch Routing: From Top-k to k = 1'), brute force."""
    h = np.round(rng.standard_normal((200, 5)), 1)  # coarse values => many ties
    e, gap = so.top1(h)
    for t in range(200):
        best = 0
        for j in range(1, 5):
            if h[t, j] > h[t, best]:
                best = j
        assert e[t] == best
        srt = sorted(h[t])
        assert abs(gap[t] - (srt[-1] - srt[-2])) < 1e-15
    # equal router rows: every token is an exact tie -> expert 0
    x = rng.standard_normal((10, 4))
    w = np.tile(rng.standard_normal((1, 4)), (3, 1))
    e, gap = so.top1(so.router_logits(x, w))
    assert e.tolist() == [0] * 10 and np.all(gap == 0)


def pin_router_logits_loops(rng):
    """h(x) = W_r . x (+ b), against explicit loops with d != N."""
    x = rng.standard_normal((5, 7))
    w = rng.standard_normal((3, 7))
    b = rng.standard_normal(3)
    h = so.router_logits(x, w, b)
    for t in range(5):
        for i in range(3):
            s = b[i]
            for k in range(7):
                s += w[i, k] * x[t, k]
            assert abs(h[t, i] - s) < 1e-12


def pin_slots_stable_sort(rng):
    """Token-order slots equal ranks from a stable sort (textbook routine)."""
    for N in (1, 2, 7, 128):
        e = rng.integers(0, N, size=3000)
        slot, dropped, count = so.assign_slots(e, N, 20)
        order = np.argsort(e, kind="stable")
        starts = np.concatenate([[0], np.cumsum(np.bincount(e, minlength=N))[:-1]])
        rank = np.empty(len(e), np.int64)
        rank[order] = np.arange(len(e)) - starts[e[order]]
        assert np.array_equal(slot, rank)
        assert np.array_equal(count, np.bincount(e, minlength=N))
        assert np.array_equal(dropped, rank >= 20)


def pin_slots_bruteforce():
    """Every routing of T <= 6 tokens over N <= 3 experts: slots are a
    bijection onto 0..count-1 per expert that preserves token order, and
    conservation sum_i min(count_i, C) + #dropped = T holds."""
    for N in (1, 2, 3):
        for T in range(0, 7):
            for e in itertools.product(range(N), repeat=T):
                e = np.array(e, np.int64)
                for C in (0, 1, 2, T):
                    slot, dropped, count = so.assign_slots(e, N, C)
                    for i in range(N):
                        toks = [t for t in range(T) if e[t] == i]
                        assert [slot[t] for t in toks] == list(range(len(toks)))
                        assert count[i] == len(toks)
                    assert sum(min(c, C) for c in count) + int(dropped.sum()) == T


def pin_aux_uniform_closed_form():
    """'The Load-Balancing Loss': under uniform routing sum_i f_i P_i = 1/N, so
    N * sum f_i P_i = 1.  (a) f uniform: one-hot tokens x_t = e_{t mod N}
    with W_r = [I 0]; (b) P uniform: W_r = 0 (all logits equal)."""
    for N in (1, 2, 5, 16):
        T, d = 3 * N, N + 3
        x = np.zeros((T, d))
        x[np.arange(T), np.arange(T) % N] = 1.0
        w = np.zeros((N, d))
        w[:, :N] = np.eye(N)
        out = so.forward(x, w, None, np.zeros((N, 2, d)), np.zeros((N, d, 2)), 3)
        assert abs(out["aux_loss"] - 1.0) < 1e-13
        rng = np.random.default_rng(N)
        x = rng.standard_normal((T, d))
        out = so.forward(x, np.zeros((N, d)), None, np.zeros((N, 2, d)), np.zeros((N, d, 2)), 3)
        assert abs(out["aux_loss"] - 1.0) < 1e-13
        assert np.all(out["expert_idx"] == 0)  # all-tie routing -> expert 0


def pin_ffn_loops(rng):
    """E(x) = W_out . ReLU(W_in . x), against explicit loops; square dims so a
    transposed operand would not fail on shape alone."""
    for d, f in ((3, 3), (4, 6)):
        x = rng.standard_normal((4, d))
        wi = rng.standard_normal((f, d))
        wo = rng.standard_normal((d, f))
        y = so.expert_ffn(x, wi, wo)
        for m in range(4):
            hid = [max(0.0, sum(wi[j, k] * x[m, k] for k in range(d))) for j in range(f)]
            for n in range(d):
                assert abs(y[m, n] - sum(wo[n, j] * hid[j] for j in range(f))) < 1e-12


def pin_single_expert_dense(rng):
    """N = 1: softmax of one logit is 1 and cf >= 1 drops nothing, so the layer
    is the dense ReLU FFN (explicit loops) on every token."""
    T, d, f = 6, 3, 5
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, 1)
    out = so.forward(x, w_r, None, w_in, w_out, so.expert_capacity(T, 1, 1.0))
    assert np.all(out["gate"] == 1.0) and not out["dropped"].any()
    for t in range(T):
        hid = [max(0.0, sum(w_in[0, j, k] * x[t, k] for k in range(d))) for j in range(f)]
        for n in range(d):
            assert abs(out["y_bare"][t, n] - sum(w_out[0, n, j] * hid[j] for j in range(f))) < 1e-12


def pin_layer_properties(rng):
    """Invariants of the layer: capacity >= T drops nothing; kept sets grow with
    cf; dropped rows are exactly 0 (bare) or exactly x (residual); doubling
    W_out doubles y; y / gate = E_e(x); with no drops, permuting tokens
    permutes every per-token output."""
    T, d, f, N = 40, 6, 10, 4
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, N, scale=2.0)
    b = np.array([1.5, 0.0, -0.5, 0.2])  # skew popularity to force drops
    prev_kept = None
    for cf in (0.25, 0.5, 1.0, 2.0, float(N)):
        C = so.expert_capacity(T, N, cf)
        out = so.forward(x, w_r, b, w_in, w_out, C)
        kept = ~out["dropped"]
        if prev_kept is not None:
            assert np.all(kept[prev_kept])
        prev_kept = kept
        assert np.sum(np.minimum(out["expert_count"], C)) + out["dropped"].sum() == T
        assert np.all(out["y_bare"][out["dropped"]] == 0.0)
        res = so.forward(x, w_r, b, w_in, w_out, C, add_residual=True)
        assert np.array_equal(res["y"][out["dropped"]], x[out["dropped"]])
        dbl = so.forward(x, w_r, b, w_in, 2 * w_out, C)
        assert np.array_equal(dbl["y_bare"], 2 * out["y_bare"])
        for t in np.nonzero(kept)[0][:5]:
            e = out["expert_idx"][t]
            ref = so.expert_ffn(x[t:t + 1], w_in[e], w_out[e])[0]
            np.testing.assert_allclose(out["y_bare"][t] / out["gate"][t], ref, rtol=1e-12, atol=1e-12)
    assert prev_kept is not None and prev_kept.all()  # cf = N keeps all
    perm = rng.permutation(T)
    a = so.forward(x, w_r, b, w_in, w_out, T)
    p = so.forward(x[perm], w_r, b, w_in, w_out, T)
    for k in ("expert_idx", "gate", "y_bare"):
        np.testing.assert_array_equal(p[k], a[k][perm])


def pin_aux_counts_before_capacity():
    """f_i follows the f equation (argmax indicator, before capacity): the
    hand example's dropped token still counts (17/16, not 25/32)."""
    g, x, w_r, w_in, w_out = _hand_inputs()
    out = so.forward(x, w_r, None, w_in, w_out, 1)  # capacity 1 drops more
    assert abs(out["aux_loss"] - 17 / 16) < 1e-14


def pin_fed_mode():
    """Fed routing: the oracle follows the given expert_idx for gates, slots,
    drops, the loss and y."""
    g, x, w_r, w_in, w_out = _hand_inputs()
    out = so.forward(x, w_r, None, w_in, w_out, 2, expert_idx=np.array([1, 1, 1, 0]))
    assert out["slot"].tolist() == [0, 1, 2, 0] and out["dropped"].tolist() == [False, False, True, False]
    np.testing.assert_allclose(out["gate"], [0.25, 0.75, 0.25, 0.5], atol=1e-14)
    # f = [1/4, 3/4], P = [9/16, 7/16] -> 2 * (9/64 + 21/64) = 15/16
    assert abs(out["aux_loss"] - 15 / 16) < 1e-14
    # token 3 -> expert 0 with input [1,1]: W_in0.[1,1] = [3,0,-3] -> ReLU [3,0,0] -> [3,9]; x 1/2
    np.testing.assert_allclose(out["y_bare"][3], [1.5, 4.5], atol=1e-14)


def pin_add_norm_zscore(rng):
    """Add + Normalize ('The Architecture in Place'): with eps = 0, unit scale
    and zero shift it is scipy's z-score of x + y over d_model (population
    standard deviation)."""
    import scipy.stats
    x, y = rng.standard_normal((7, 12)), rng.standard_normal((7, 12)) * 0.1
    got = so.add_normalize(x, y, np.ones(12), np.zeros(12), 0.0)
    np.testing.assert_allclose(got, scipy.stats.zscore(x + y, axis=1, ddof=0), rtol=0, atol=1e-12)


def pin_add_norm_hand():
    """A hand-worked row: x + y = [2, 2, 2, 4], mean 5/2, variance 3/4; with
    eps = 1/4 the denominator is exactly 1, so out = (v - 5/2) * gamma + beta."""
    out = so.add_normalize(np.array([[1.0, 2.0, 3.0, 4.0]]), np.array([[1.0, 0.0, -1.0, 0.0]]),
                           np.array([1.0, 2.0, 1.0, 1.0]), np.array([0.0, 0.0, 1.0, 0.0]), 0.25)
    assert out.tolist() == [[-0.5, -1.0, 0.5, 1.5]]


def pin_add_norm_invariants(rng):
    """Normalisation removes a per-row shift of x + y; scale and shift act per
    feature after it."""
    x, y = rng.standard_normal((5, 16)), rng.standard_normal((5, 16))
    g, b = rng.standard_normal(16), rng.standard_normal(16)
    base = so.add_normalize(x, y, np.ones(16), np.zeros(16), 1e-6)
    shifted = so.add_normalize(x + rng.standard_normal((5, 1)) * 3.0, y, np.ones(16), np.zeros(16), 1e-6)
    np.testing.assert_allclose(shifted, base, atol=1e-10)
    np.testing.assert_allclose(so.add_normalize(x, y, g, b, 1e-6), base * g + b, atol=1e-12)


def _top2_hand_inputs():
    g = _load("top2_hand_example.json")
    inp = g["inputs"]
    x = np.array(inp["x_over_ln2"], np.float64) * math.log(2.0)
    w_r = np.array(inp["w_router"], np.float64)
    w_in = np.stack([np.eye(3)] * 3)
    w_out = np.stack([s * np.eye(3) for s in inp["w_out_scale"]])
    return g, x, w_r, w_in, w_out


def pin_topk_hand_example():
    """The hand-worked top-2 layer (tests/golden/top2_hand_example.json):
    choice order, un-renormalised gates, route-major capacity, the loss."""
    g, x, w_r, w_in, w_out = _top2_hand_inputs()
    exp = g["expected"]
    for cap in (2, 3):
        e = exp[f"capacity_{cap}"]
        out = so.forward_topk(x, w_r, None, w_in, w_out, cap, 2)
        np.testing.assert_allclose(out["probs"] * 7, exp["probs_times_7"], rtol=0, atol=1e-13)
        assert out["expert_idx"].tolist() == exp["expert_idx"]
        np.testing.assert_allclose(out["gate"] * 7, exp["gate_times_7"], rtol=0, atol=1e-13)
        assert out["dropped"].tolist() == e["dropped"]
        coef = np.array([n / d for n, d in e["y_over_x_num_den"]])
        np.testing.assert_allclose(out["y_bare"], coef[:, None] * x, rtol=0, atol=1e-13)
        if "slot" in e:
            assert out["slot"].tolist() == e["slot"]
            assert out["expert_count"].tolist() == e["expert_count"]
            n, d = e["aux_loss_num_den"]
            assert abs(out["aux_loss"] - n / d) < 1e-14


def pin_topk_choice_loops(rng):
    """Top-k selection ('Switch Routing: From Top-k to k = 1'): repeated
    explicit-loop argmax with the chosen entries removed, on coarse values
    with many ties; the near-tie gap by brute force over sorted values."""
    for N, k in ((5, 2), (4, 4), (6, 3), (2, 1)):
        h = np.round(rng.standard_normal((150, N)), 1)
        idx, gap = so.topk_choice(h, k)
        for t in range(150):
            left = list(range(N))
            for r in range(k):
                best = left[0]
                for j in left[1:]:
                    if h[t, j] > h[t, best]:
                        best = j
                assert idx[r, t] == best
                left.remove(best)
            srt = sorted(h[t], reverse=True)[:min(k + 1, N)]
            want = min(a - b for a, b in zip(srt, srt[1:])) if len(srt) > 1 else math.inf
            assert gap[t] == want


def pin_topk_k1_is_switch(rng):
    """k = 1 is the Switch layer: every output equals the top-1 oracle's,
    with drops (skewed bias) and with the residual."""
    T, d, f, N = 30, 5, 7, 4
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, N, scale=2.0)
    b = np.array([1.0, 0.0, -0.5, 0.3])
    for cap in (3, 8, 30):
        for res in (False, True):
            a = so.forward(x, w_r, b, w_in, w_out, cap, add_residual=res)
            t = so.forward_topk(x, w_r, b, w_in, w_out, cap, 1, add_residual=res)
            for key in ("expert_idx", "gate", "slot", "dropped"):
                np.testing.assert_array_equal(t[key][0], a[key])
            np.testing.assert_array_equal(t["expert_count"], a["expert_count"])
            assert t["aux_loss"] == a["aux_loss"]
            np.testing.assert_allclose(t["y"], a["y"], rtol=0, atol=1e-13)


def pin_topk_dense_mixture(rng):
    """k = N with room for every route is the dense softmax mixture
    sum_i p_i(x) E_i(x) over all experts (scipy's softmax, einsum experts)."""
    T, d, f, N = 12, 4, 6, 3
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, N)
    out = so.forward_topk(x, w_r, None, w_in, w_out, N * T, N)
    p = scipy.special.softmax(x @ w_r.T, axis=1)
    hid = np.maximum(np.einsum("td,nfd->ntf", x, w_in), 0.0)
    e = np.einsum("ntf,ndf->ntd", hid, w_out)
    np.testing.assert_allclose(out["y_bare"], np.einsum("tn,ntd->td", p, e), rtol=0, atol=1e-12)
    assert not out["dropped"].any()
    np.testing.assert_allclose(out["gate"].sum(axis=0), 1.0, rtol=0, atol=1e-14)


def pin_topk_route_major_bruteforce():
    """Route-major capacity over every top-2 routing of T <= 4 tokens over
    N = 3 experts: route 0's slots are the top-1 slots of route 0 alone (a
    second choice never displaces a first choice); each expert's slots run
    0..count-1 in route-major order; conservation over the 2T routes."""
    pairs = [(a, b) for a in range(3) for b in range(3) if a != b]
    for T in range(0, 5):
        for choice in itertools.product(pairs, repeat=T):
            idx = np.array(choice, np.int64).reshape(T, 2).T if T else np.zeros((2, 0), np.int64)
            for C in (0, 1, 2, 2 * T):
                slot, dropped, count = so.assign_slots_topk(idx, 3, C)
                s0, d0, _ = so.assign_slots(idx[0], 3, C)
                assert np.array_equal(slot[0], s0) and np.array_equal(dropped[0], d0)
                for i in range(3):
                    seq = [slot[r, t] for r in range(2) for t in range(T) if idx[r, t] == i]
                    assert seq == list(range(len(seq))) and count[i] == len(seq)
                assert sum(min(c, C) for c in count) + int(dropped.sum()) == 2 * T


def pin_topk_aux_uniform():
    """'The Load-Balancing Loss' closed form carried to k routes: with every
    p_i = 1/N (W_r = 0) the loss is sum_i f_i = 1 whatever the routing."""
    rng = np.random.default_rng(7)
    for N, k in ((2, 2), (5, 2), (8, 3)):
        T, d = 4 * N, 6
        x = rng.standard_normal((T, d))
        out = so.forward_topk(x, np.zeros((N, d)), None, np.zeros((N, 2, d)), np.zeros((N, d, 2)), T, k)
        assert abs(out["aux_loss"] - 1.0) < 1e-13
        assert out["expert_idx"].tolist() == [[r] * T for r in range(k)]  # all-tie -> lowest indices


def _bwd_loss(x, w_r, b, w_in, w_out, C, dy, d_aux, res):
    out = so.forward(x, w_r, b, w_in, w_out, C, add_residual=res)
    return float(np.sum(dy * out["y"]) + d_aux * out["aux_loss"]), out


def pin_backward_finite_differences(rng):
    """Backward pass against central finite differences of the forward
    oracle's L = <dy, y> + d_aux aux, for every scalar of x, W_r, b, W_in and
    W_out, with drops and with and without the residual.  The routing must not
    change under the perturbation (checked), so f_i stays fixed as the
    write-up's hard count."""
    T, d, f, N = 9, 4, 5, 3
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, N, scale=1.5)
    b = np.array([0.7, 0.0, -0.4])
    dy = rng.standard_normal((T, d))
    eps = 1e-6
    for res, C in ((False, 2), (True, 3)):
        g = so.backward(x, w_r, b, w_in, w_out, C, dy, 0.37, add_residual=res)
        base = g["forward"]
        assert base["dropped"].any()
        params = [("x", x, g["dx"]), ("w_r", w_r, g["dw_router"]), ("b", b, g["d_router_bias"]),
                  ("w_in", w_in, np.stack(g["dw_in"])), ("w_out", w_out, np.stack(g["dw_out"]))]
        for name, arr, grad in params:
            for i in np.ndindex(arr.shape):
                old = arr[i]
                arr[i] = old + eps
                lp, op = _bwd_loss(x, w_r, b, w_in, w_out, C, dy, 0.37, res)
                arr[i] = old - eps
                lm, om = _bwd_loss(x, w_r, b, w_in, w_out, C, dy, 0.37, res)
                arr[i] = old
                for o in (op, om):
                    assert np.array_equal(o["expert_idx"], base["expert_idx"])
                    assert np.array_equal(o["dropped"], base["dropped"])
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - grad[i]) <= 2e-6 * (1 + abs(fd)), (name, i, fd, grad[i], res)


def pin_backward_aux_closed_form():
    """'The Load-Balancing Loss': with W_r = 0 every p_i = 1/N and every token
    ties to expert 0, so f = e_0; with dy = 0 and d_aux = 1 the logit gradient
    is (e_0 - 1/N) / T for every token, dW_r = (e_0 - 1/N) (sum_t x_t)^T / T,
    dbias = e_0 - 1/N, and nothing reaches the experts or x."""
    rng = np.random.default_rng(3)
    for N in (2, 5):
        T, d, f = 6, 3, 4
        x = rng.standard_normal((T, d))
        w_in, w_out = rng.standard_normal((N, f, d)), rng.standard_normal((N, d, f))
        g = so.backward(x, np.zeros((N, d)), None, w_in, w_out, T, np.zeros((T, d)), 1.0)
        v = -np.full(N, 1.0 / N)
        v[0] += 1.0
        np.testing.assert_allclose(g["dlogits"], np.tile(v / T, (T, 1)), rtol=0, atol=1e-15)
        np.testing.assert_allclose(g["dw_router"], np.outer(v, x.sum(axis=0)) / T, rtol=0, atol=1e-14)
        np.testing.assert_allclose(g["d_router_bias"], v, rtol=0, atol=1e-14)
        assert np.all(g["dx"] == 0.0)
        assert all(np.all(a == 0.0) for a in g["dw_in"] + g["dw_out"])


def pin_backward_single_expert_dense(rng):
    """N = 1: the gate is 1 and the softmax of one logit has no gradient, so
    the router gets nothing and the experts' gradients are the dense ReLU
    FFN's, written out with explicit loops."""
    T, d, f = 5, 3, 4
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, 1)
    dy = rng.standard_normal((T, d))
    g = so.backward(x, w_r, None, w_in, w_out, T, dy, 0.5)
    assert np.all(g["dw_router"] == 0.0) and np.all(g["d_router_bias"] == 0.0)
    wi, wo = w_in[0], w_out[0]
    dwi, dwo, dx = np.zeros_like(wi), np.zeros_like(wo), np.zeros_like(x)
    for t in range(T):
        u = [sum(wi[j, k] * x[t, k] for k in range(d)) for j in range(f)]
        h = [max(0.0, v) for v in u]
        dh = [sum(wo[n, j] * dy[t, n] for n in range(d)) for j in range(f)]
        du = [dh[j] if u[j] > 0 else 0.0 for j in range(f)]
        for n in range(d):
            for j in range(f):
                dwo[n, j] += dy[t, n] * h[j]
        for j in range(f):
            for k in range(d):
                dwi[j, k] += du[j] * x[t, k]
                dx[t, k] += wi[j, k] * du[j]
    np.testing.assert_allclose(g["dw_out"][0], dwo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dw_in"][0], dwi, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dx"], dx, rtol=0, atol=1e-12)


def pin_backward_dropped_tokens(rng):
    """A dropped token's bare output is 0: with no loss term its gradient is
    exactly 0 (bare) or exactly dy (residual), and its logits get nothing."""
    T, d, f, N = 12, 4, 5, 3
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, N, scale=2.0)
    dy = rng.standard_normal((T, d))
    for res in (False, True):
        g = so.backward(x, w_r, np.array([2.0, 0.0, 0.0]), w_in, w_out, 2, dy, 0.0, add_residual=res)
        drop = g["forward"]["dropped"]
        assert drop.sum() >= 3
        assert np.all(g["dlogits"][drop] == 0.0)
        assert np.array_equal(g["dx"][drop], dy[drop] if res else np.zeros_like(dy[drop]))


def pin_forward_sampled_experts(rng):
    """forward(experts=S) restricts the expert FFN to the experts in S (what
    the parity tests of the largest layers use): the routing outputs do not
    change; the rows of kept tokens routed to S are the full forward's rows
    bit for bit; every other kept row is NaN (so a comparison skips it);
    dropped rows are exactly 0 ('Expert Capacity': a dropped token's
    computation is skipped); weights of experts outside S are never asked
    for; S = every expert is the full forward."""
    T, d, f, N = 48, 5, 7, 6
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, N, scale=2.0)
    b = np.array([1.0, 0.5, 0.0, 0.0, -0.5, 0.0])  # skewed: forces drops
    C = so.expert_capacity(T, N, 1.0)
    full = so.forward(x, w_r, b, w_in, w_out, C)
    kept = ~full["dropped"]
    assert full["dropped"].any() and kept.any()
    for S in ([], [2], [0, 3, 5], list(range(N))):
        asked = []

        def source(i, asked=asked):
            asked.append(i)
            return w_in[i], w_out[i]

        part = so.forward(x, w_r, b, source, None, C, experts=S)
        assert set(asked) <= set(S)
        for k in ("expert_idx", "gate", "slot", "dropped", "expert_count"):
            assert np.array_equal(part[k], full[k]), k
        assert part["aux_loss"] == full["aux_loss"]
        in_s = np.isin(full["expert_idx"], S)
        assert np.array_equal(part["y_bare"][kept & in_s], full["y_bare"][kept & in_s])
        assert np.all(np.isnan(part["y_bare"][kept & ~in_s]))
        assert np.all(part["y_bare"][~kept] == 0.0)
        if S == [0, 3, 5]:
            assert (kept & in_s).sum() >= 10  # the sample is not empty
    np.testing.assert_array_equal(so.forward(x, w_r, b, w_in, w_out, C, experts=list(range(N)))["y_bare"],
                                  full["y_bare"])


def pin_combine_residual():
    """combine with x_residual: every row is x + the bare combined row and a
    dropped row is exactly x ('Expert Capacity': a dropped token continues
    through the residual; 'Switch Routing': y = p_e(x) E_e(x) for k = 1), on
    the hand-worked layer with the expert outputs worked by hand there
    (expert 0 maps [1, 0] to [1, 3]; expert 1 maps [0, 1] to [2, 1])."""
    g, x, w_r, w_in, w_out = _hand_inputs()
    exp = g["expected"]
    e = np.array(exp["expert_idx"])
    slot = np.array(exp["slot"])
    dropped = np.array(exp["dropped"])
    gate = np.array(exp["gate"])
    eo = np.zeros((2, 2, 2))
    eo[0, 0] = eo[0, 1] = [1.0, 3.0]  # tokens 0 and 2 (slots 0 and 1 of expert 0)
    eo[1, 0] = [2.0, 1.0]             # token 1
    np.testing.assert_allclose(so.combine(eo, e, slot, dropped, gate), exp["y_bare"], rtol=0, atol=1e-14)
    y = so.combine(eo, e, slot, dropped, gate, x_residual=x)
    np.testing.assert_allclose(y, exp["y_residual"], rtol=0, atol=1e-14)
    assert np.array_equal(y[dropped], x[dropped])


def pin_combine_residual_matches_layer(rng):
    """Stage path with the residual: dispatch, the expert FFN of each buffer
    and combine(x_residual=x) give the layer's y with add_residual, rows of
    dropped tokens exactly x."""
    T, d, f, N = 30, 4, 6, 3
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, N, scale=2.0)
    b = np.array([1.0, 0.0, -1.0])
    C = so.expert_capacity(T, N, 0.75)
    lay = so.forward(x, w_r, b, w_in, w_out, C, add_residual=True)
    assert lay["dropped"].any()
    buf, filled = so.dispatch(x, lay["expert_idx"], lay["slot"], lay["dropped"], N, C)
    eo = np.stack([so.expert_ffn(buf[i], w_in[i], w_out[i]) for i in range(N)])
    y = so.combine(eo, lay["expert_idx"], lay["slot"], lay["dropped"], lay["gate"], x_residual=x)
    np.testing.assert_allclose(y, lay["y"], rtol=1e-13, atol=1e-13)
    assert np.array_equal(y[lay["dropped"]], x[lay["dropped"]])


def pin_backward_rss_loops(rng):
    """The root-sum-square scales backward reports beside each gradient that
    sums over tokens are sqrt(sum_t term_t^2) over that sum's terms, written
    here as explicit loops from quantities recomputed by loops: dbias_i sums
    dh[t, i]; dW_r[i, k] sums dh[t, i] x[t, k]; dW_in[e][j, k] sums du[t, j]
    x[t, k] and dW_out[e][n, j] sums g_t dy[t, n] h[t, j] over e's kept
    tokens, with u = W_in x, h = ReLU(u), du = [u > 0] W_out^T (g dy).  dh
    is the oracle's dL/dh (pinned to finite differences above).  Also: the
    magnitude of a sum of n terms is at most sqrt(n) times the scale
    (Cauchy-Schwarz), and equals the scale when one token contributes."""
    T, d, f, N = 9, 3, 4, 3
    x, w_r, w_in, w_out = _rand_layer(rng, T, d, f, N, scale=1.5)
    dy = rng.standard_normal((T, d))
    C = so.expert_capacity(T, N, 1.0)
    g = so.backward(x, w_r, np.array([0.3, 0.0, -0.2]), w_in, w_out, C, dy, 0.7)
    fw = g["forward"]
    dh = g["dlogits"]
    for i in range(N):
        assert abs(g["d_router_bias_rss"][i] - math.sqrt(sum(dh[t, i] ** 2 for t in range(T)))) < 1e-12
        for k in range(d):
            ref = math.sqrt(sum((dh[t, i] * x[t, k]) ** 2 for t in range(T)))
            assert abs(g["dw_router_rss"][i, k] - ref) < 1e-12
    for e in range(N):
        rows = [t for t in range(T) if fw["expert_idx"][t] == e and not fw["dropped"][t]]
        u = {t: [sum(w_in[e, j, k] * x[t, k] for k in range(d)) for j in range(f)] for t in rows}
        gd = {t: [fw["gate"][t] * dy[t, n] for n in range(d)] for t in rows}
        du = {t: [(u[t][j] > 0) * sum(w_out[e, n, j] * gd[t][n] for n in range(d)) for j in range(f)] for t in rows}
        for j in range(f):
            for k in range(d):
                ref = math.sqrt(sum((du[t][j] * x[t, k]) ** 2 for t in rows))
                assert abs(g["dw_in_rss"][e][j, k] - ref) < 1e-12
        for n in range(d):
            for j in range(f):
                ref = math.sqrt(sum((gd[t][n] * max(u[t][j], 0.0)) ** 2 for t in rows))
                assert abs(g["dw_out_rss"][e][n, j] - ref) < 1e-12
        if len(rows) == 1:
            np.testing.assert_allclose(g["dw_in_rss"][e], np.abs(g["dw_in"][e]), rtol=1e-12, atol=1e-15)
    # Cauchy-Schwarz: |sum of n terms| <= sqrt(n) * their root sum of squares
    assert np.all(math.sqrt(T) * g["d_router_bias_rss"] >= np.abs(g["d_router_bias"]) - 1e-15)
    assert np.all(math.sqrt(T) * g["dw_router_rss"] >= np.abs(g["dw_router"]) - 1e-15)
    for e in range(N):
        n = max(1, int(np.sum((fw["expert_idx"] == e) & ~fw["dropped"])))
        assert np.all(math.sqrt(n) * g["dw_in_rss"][e] >= np.abs(g["dw_in"][e]) - 1e-15)
        assert np.all(math.sqrt(n) * g["dw_out_rss"][e] >= np.abs(g["dw_out"][e]) - 1e-15)


ALL_PINS = [
    pin_capacity_table, pin_hand_example, pin_softmax_library, pin_top1_bruteforce,
    pin_router_logits_loops, pin_slots_stable_sort, pin_slots_bruteforce,
    pin_aux_uniform_closed_form, pin_ffn_loops, pin_single_expert_dense,
    pin_layer_properties, pin_aux_counts_before_capacity, pin_fed_mode,
    pin_add_norm_zscore, pin_add_norm_hand, pin_add_norm_invariants,
    pin_topk_hand_example, pin_topk_choice_loops, pin_topk_k1_is_switch, pin_topk_dense_mixture,
    pin_topk_route_major_bruteforce, pin_topk_aux_uniform,
    pin_backward_finite_differences, pin_backward_aux_closed_form, pin_backward_single_expert_dense,
    pin_backward_dropped_tokens, pin_forward_sampled_experts, pin_combine_residual,
    pin_combine_residual_matches_layer, pin_backward_rss_loops,
]


def _run(pin):
    import inspect
    if "rng" in inspect.signature(pin).parameters:
        pin(np.random.default_rng(1234))
    else:
        pin()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    _run(pin)


# ------------------------------------------------------------ mutations -----
def _mut_top1_last_tie(h):
    e = (h.shape[1] - 1 - np.argmax(h[:, ::-1], axis=1)).astype(np.int64)
    srt = np.sort(h, axis=1)
    gap = srt[:, -1] - srt[:, -2] if h.shape[1] > 1 else np.full(h.shape[0], np.inf)
    return e, gap


def _mut_slots_reversed(expert_idx, num_experts, capacity):
    T = len(expert_idx)
    seen = [0] * num_experts
    slot = np.empty(T, np.int64)
    for t in reversed(range(T)):
        i = int(expert_idx[t])
        slot[t] = seen[i]
        seen[i] += 1
    return slot, slot >= capacity, np.asarray(seen, np.int64)


def _mut_slots_off_by_one(expert_idx, num_experts, capacity):
    slot, _, count = _ORIG["assign_slots"](expert_idx, num_experts, capacity)
    return slot, slot > capacity, count


def _mut_aux_after_capacity(expert_idx, probs, num_experts):
    T = len(expert_idx)
    if T == 0:
        return 0.0
    C = so.expert_capacity(T, num_experts, 1.0)
    slot, dropped, _ = _ORIG["assign_slots"](expert_idx, num_experts, C)
    f = np.array([np.count_nonzero((expert_idx == i) & ~dropped) / T for i in range(num_experts)])
    return float(num_experts * np.sum(f * probs.sum(axis=0) / T))


def _mut_aux_no_n(expert_idx, probs, num_experts):
    return _ORIG["load_balancing_loss"](expert_idx, probs, num_experts) / num_experts


def _mut_ffn_no_relu(x_e, w_in_e, w_out_e):
    return (np.asarray(x_e) @ np.asarray(w_in_e).T) @ np.asarray(w_out_e).T


def _mut_ffn_transposed(x_e, w_in_e, w_out_e):
    hid = np.maximum(np.asarray(x_e) @ np.asarray(w_in_e).T, 0.0)
    wo = np.asarray(w_out_e)
    return hid @ (wo if wo.shape[0] == wo.shape[1] else wo.T)


def _mut_softmax_wrong_axis(h):
    m = h.max(axis=1, keepdims=True)
    e = np.exp(h - m)
    return e / e.sum(axis=0, keepdims=True)


def _mut_logits_no_bias(x, w_router, bias=None):
    return np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T


def _mut_norm_sample_variance(x, y, gamma, beta, eps):
    v = np.asarray(x, np.float64) + np.asarray(y, np.float64)
    mu = v.mean(axis=1, keepdims=True)
    var = ((v - mu) ** 2).sum(axis=1, keepdims=True) / (v.shape[1] - 1)
    return (v - mu) / np.sqrt(var + eps) * gamma + beta


def _mut_norm_eps_outside(x, y, gamma, beta, eps):
    v = np.asarray(x, np.float64) + np.asarray(y, np.float64)
    mu = v.mean(axis=1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=1, keepdims=True)
    return (v - mu) / (np.sqrt(var) + eps) * gamma + beta


def _mut_norm_no_residual(x, y, gamma, beta, eps):
    return _ORIG["add_normalize"](np.zeros_like(np.asarray(x, np.float64)), y, gamma, beta, eps)


def _mut_topk_token_major(expert_idx, num_experts, capacity):
    k, T = expert_idx.shape
    slot, dropped, count = _ORIG["assign_slots"](expert_idx.T.reshape(-1), num_experts, capacity)
    return slot.reshape(T, k).T, dropped.reshape(T, k).T, count


def _mut_topk_last_tie(h, k):
    N = h.shape[1]
    order = (N - 1 - np.argsort(-h[:, ::-1], axis=1, kind="stable"))
    idx = order[:, :k].T.astype(np.int64).copy()
    return idx, _ORIG["topk_choice"](h, k)[1]


def _mut_topk_f_over_T(expert_idx, probs, num_experts):
    return _ORIG["load_balancing_loss_topk"](expert_idx, probs, num_experts) * expert_idx.shape[0]


def _mut_topk_renormalised(*args, **kw):
    out = _ORIG["forward_topk"](*args, **kw)
    s = out["gate"].sum(axis=0)
    out["y_bare"] = out["y_bare"] / s[:, None]
    return out


def _mut_topk_skips_second(*args, **kw):
    out = _ORIG["forward_topk"](*args, **kw)
    k = out["expert_idx"].shape[0]
    if k > 1:
        args = list(args)
        x, w_r, b, w_in, w_out, cap = args[:6]
        first = so.forward(x, w_r, b, w_in, w_out, cap, expert_idx=out["expert_idx"][0])
        out["y_bare"] = first["y_bare"]
    return out


def _mut_softmax_bwd_no_mean(p, dp):
    return p * dp


def _mut_expert_bwd_no_relu_mask(x_e, w_in_e, w_out_e, dy_e, gate_e):
    o = np.maximum(x_e @ w_in_e.T, 0.0) @ w_out_e.T
    do = gate_e[:, None] * dy_e
    du = do @ w_out_e
    return np.sum(dy_e * o, axis=1), du.T @ x_e, do.T @ np.maximum(x_e @ w_in_e.T, 0.0), du @ w_in_e


def _mut_expert_bwd_no_gate(x_e, w_in_e, w_out_e, dy_e, gate_e):
    return _ORIG["expert_backward"](x_e, w_in_e, w_out_e, dy_e, np.ones_like(gate_e))


def _mut_expert_bwd_pre_relu(x_e, w_in_e, w_out_e, dy_e, gate_e):
    dg, gi, go, dx = _ORIG["expert_backward"](x_e, w_in_e, w_out_e, dy_e, gate_e)
    return dg, gi, (gate_e[:, None] * dy_e).T @ (x_e @ w_in_e.T), dx


def _mut_bwd_aux_ignored(*args, **kw):
    args = list(args)
    if len(args) > 7:
        args[7] = 0.0
    else:
        kw["d_aux"] = 0.0
    return _ORIG["backward"](*args, **kw)


def _mut_bwd_residual_ignored(*args, **kw):
    out = _ORIG["backward"](*args, **kw)
    res = kw.get("add_residual", args[8] if len(args) > 8 else False)
    if res:
        dy = args[6] if len(args) > 6 else kw["dy"]
        out["dx"] = out["dx"] - dy
    return out


def _mut_forward_sample_all_nan(*args, **kw):
    out = _ORIG["forward"](*args, **kw)
    if kw.get("experts") is not None:
        out["y_bare"][~out["dropped"]] = np.nan
        out["y"] = out["y_bare"]
    return out


def _mut_forward_sample_zero_rows(*args, **kw):
    out = _ORIG["forward"](*args, **kw)
    if kw.get("experts") is not None:
        out["y_bare"] = np.nan_to_num(out["y_bare"], nan=0.0)
        out["y"] = out["y_bare"]
    return out


def _mut_forward_sample_shifted(*args, **kw):
    # computes the sampled rows with the next expert's weights
    S = kw.get("experts")
    if S is None:
        return _ORIG["forward"](*args, **kw)
    x, w_r, b, w_in, w_out, cap = args[:6]
    n = np.asarray(w_r).shape[0]
    get = _ORIG["_weights"](w_in, w_out)
    kw = dict(kw)
    return _ORIG["forward"](x, w_r, b, lambda i: get((i + 1) % n), None, cap, *args[6:], **kw)


def _mut_combine_residual_kept_only(expert_out, expert_idx, slot, dropped, gate, x_residual=None):
    y = _ORIG["combine"](expert_out, expert_idx, slot, dropped, gate)
    if x_residual is not None:
        y[~dropped] += np.asarray(x_residual, np.float64)[~dropped]
    return y


def _mut_combine_residual_ignored(expert_out, expert_idx, slot, dropped, gate, x_residual=None):
    return _ORIG["combine"](expert_out, expert_idx, slot, dropped, gate)


def _mut_bwd_rss_squared(*args, **kw):
    out = _ORIG["backward"](*args, **kw)
    out["d_router_bias_rss"] = out["d_router_bias_rss"] ** 2
    out["dw_router_rss"] = out["dw_router_rss"] ** 2
    out["dw_in_rss"] = [None if r is None else r ** 2 for r in out["dw_in_rss"]]
    out["dw_out_rss"] = [None if r is None else r ** 2 for r in out["dw_out_rss"]]
    return out


def _mut_bwd_rss_router_without_x(*args, **kw):
    out = _ORIG["backward"](*args, **kw)
    out["dw_router_rss"] = np.broadcast_to(out["d_router_bias_rss"][:, None], out["dw_router_rss"].shape).copy()
    return out


def _mut_bwd_rss_out_pre_relu(*args, **kw):
    out = _ORIG["backward"](*args, **kw)
    x, w_r, b, w_in, w_out, cap, dy = args[:7]
    fw = out["forward"]
    for e in range(len(out["dw_out_rss"])):
        rows = np.nonzero((fw["expert_idx"] == e) & ~fw["dropped"])[0]
        if len(rows) and out["dw_out_rss"][e] is not None:
            u = np.asarray(x)[rows] @ np.asarray(w_in[e]).T
            gd = fw["gate"][rows, None] * np.asarray(dy)[rows]
            out["dw_out_rss"][e] = np.sqrt((gd ** 2).T @ (u ** 2))
    return out


_ORIG = {k: getattr(so, k) for k in ("softmax_backward", "expert_backward", "backward","assign_slots", "load_balancing_loss", "top1", "expert_ffn",
                                     "softmax", "router_logits", "add_normalize", "topk_choice",
                                     "load_balancing_loss_topk", "forward_topk", "forward", "combine",
                                     "_weights")}

MUTANTS = {
    "top1_last_index_on_tie": ("top1", _mut_top1_last_tie),
    "slots_later_token_wins": ("assign_slots", _mut_slots_reversed),
    "drop_off_by_one": ("assign_slots", _mut_slots_off_by_one),
    "f_after_capacity": ("load_balancing_loss", _mut_aux_after_capacity),
    "loss_missing_N": ("load_balancing_loss", _mut_aux_no_n),
    "ffn_without_relu": ("expert_ffn", _mut_ffn_no_relu),
    "ffn_transposed_w_out": ("expert_ffn", _mut_ffn_transposed),
    "softmax_wrong_axis": ("softmax", _mut_softmax_wrong_axis),
    "router_bias_dropped": ("router_logits", _mut_logits_no_bias),
    "norm_sample_variance": ("add_normalize", _mut_norm_sample_variance),
    "norm_eps_outside_sqrt": ("add_normalize", _mut_norm_eps_outside),
    "norm_without_residual": ("add_normalize", _mut_norm_no_residual),
    "topk_token_major_capacity": ("assign_slots_topk", _mut_topk_token_major),
    "topk_last_index_on_tie": ("topk_choice", _mut_topk_last_tie),
    "topk_f_over_T": ("load_balancing_loss_topk", _mut_topk_f_over_T),
    "topk_renormalised_gates": ("forward_topk", _mut_topk_renormalised),
    "topk_second_route_ignored": ("forward_topk", _mut_topk_skips_second),
    "bwd_softmax_without_mean": ("softmax_backward", _mut_softmax_bwd_no_mean),
    "bwd_no_relu_mask": ("expert_backward", _mut_expert_bwd_no_relu_mask),
    "bwd_gate_ignored": ("expert_backward", _mut_expert_bwd_no_gate),
    "bwd_w_out_grad_pre_relu": ("expert_backward", _mut_expert_bwd_pre_relu),
    "bwd_aux_ignored": ("backward", _mut_bwd_aux_ignored),
    "bwd_residual_ignored": ("backward", _mut_bwd_residual_ignored),
    "sampled_experts_all_nan": ("forward", _mut_forward_sample_all_nan),
    "sampled_experts_zero_rows": ("forward", _mut_forward_sample_zero_rows),
    "sampled_experts_wrong_weights": ("forward", _mut_forward_sample_shifted),
    "combine_residual_on_kept_rows_only": ("combine", _mut_combine_residual_kept_only),
    "combine_residual_ignored": ("combine", _mut_combine_residual_ignored),
    "bwd_rss_without_sqrt": ("backward", _mut_bwd_rss_squared),
    "bwd_rss_router_without_x": ("backward", _mut_bwd_rss_router_without_x),
    "bwd_rss_w_out_pre_relu": ("backward", _mut_bwd_rss_out_pre_relu),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(so, attr, fn)
    failures = 0
    for pin in ALL_PINS:
        try:
            _run(pin)
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failures += 1
    assert failures > 0, f"no pin catches the planted mistake {name}"
