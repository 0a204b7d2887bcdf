"""Property tests of the oracle (CPU, hypothesis): invariants that the
Switch layer's definitions fix for every input, swept over random token
counts and widths, expert counts N in {1, 2, 3, 8, 128, 2048}, capacity
factors in {0.5, 1, 1.25, N} and router biases that are absent, Zipf-skewed
or pinned to one expert.

Each property follows from the write-up (Switch Transformers: Scaling to
Trillion Parameter Models):
* "Switch Routing: From Top-k to k = 1": one expert per token, the argmax of
  the softmax (so of the logits), gate = that probability;
* "Expert Capacity and the Capacity Factor": capacity = T / N x cf rounded
  up, tokens fill each expert's buffer in token order and the overflow is
  dropped (a dropped token's layer output is 0);
* "The Load-Balancing Loss": N sum_i f_i P_i with f the routed fraction and P
  the mean probability, so it lies in (0, N] and is unchanged when the
  experts are relabelled.
"""

from __future__ import annotations

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle.switch_oracle as so

N_CHOICES = [1, 2, 3, 8, 128, 2048]
PROP = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                suppress_health_check=[HealthCheck.too_slow])


@st.composite
def routing_case(draw):
    T = draw(st.integers(0, 300))
    N = draw(st.sampled_from(N_CHOICES))
    d = draw(st.sampled_from([8, 64, 96]))
    cf = draw(st.sampled_from([0.5, 1.0, 1.25, float(N)]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    bias_kind = draw(st.sampled_from(["none", "zipf", "hot"]))
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((N, d)) * np.sqrt(0.1 / d)
    if bias_kind == "none":
        b = None
    elif bias_kind == "zipf":
        b = np.log(np.arange(1, N + 1, dtype=np.float64) ** -1.1)[rng.permutation(N)] * 0.3
    else:
        b = np.zeros(N)
        b[int(rng.integers(N))] = 30.0
    return x, w, b, cf


def _route(x, w, b, cf):
    T, N = x.shape[0], w.shape[0]
    C = so.expert_capacity(T, N, cf)
    h = so.router_logits(x, w, b)
    p = so.softmax(h) if T else np.zeros((0, N))
    idx, gap = so.top1(h) if T else (np.zeros(0, np.int64), np.zeros(0))
    slot, dropped, count = so.assign_slots(idx, N, C)
    aux = so.load_balancing_loss(idx, p, N)
    return C, h, p, idx, slot, dropped, count, aux


@PROP
@given(routing_case())
def test_capacity_is_the_rounded_up_share(case):
    x, w, _, cf = case
    T, N = x.shape[0], w.shape[0]
    C = so.expert_capacity(T, N, cf)
    # C is the least integer >= T cf / N (exact rational arithmetic on cf)
    from fractions import Fraction
    share = Fraction(T) * Fraction(cf) / N
    assert C >= share and C - 1 < share


@PROP
@given(routing_case())
def test_choice_is_the_first_largest_logit(case):
    C, h, p, idx, *_ = _route(*case)
    for t in range(h.shape[0]):
        e = idx[t]
        assert np.all(h[t] <= h[t, e])
        assert np.all(h[t, :e] < h[t, e])  # ties go to the lowest index
        assert p[t, e] == p[t].max()


@PROP
@given(routing_case())
def test_probabilities_and_gate(case):
    C, h, p, idx, *_ = _route(*case)
    N = h.shape[1]
    if h.shape[0] == 0:
        return
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)
    gate = p[np.arange(len(idx)), idx]
    # the largest of N probabilities that sum to 1 is at least 1/N
    assert np.all(gate >= 1.0 / N - 1e-15) and np.all(gate <= 1.0)


@PROP
@given(routing_case())
def test_buffers_fill_in_token_order_and_overflow_drops(case):
    C, h, p, idx, slot, dropped, count, _ = _route(*case)
    N = h.shape[1]
    assert count.sum() == len(idx)
    for i in range(N):
        toks = np.nonzero(idx == i)[0]  # increasing token order
        assert count[i] == len(toks)
        assert np.array_equal(slot[toks], np.arange(len(toks)))
        assert np.array_equal(dropped[toks], np.arange(len(toks)) >= C)
        assert np.count_nonzero(~dropped[toks]) == min(len(toks), C)
    if C >= len(idx):  # every buffer can hold the whole batch (e.g. cf = N)
        assert not dropped.any()


@PROP
@given(routing_case(), st.integers(0, 40))
def test_more_capacity_never_drops_more(case, extra):
    C, h, p, idx, slot, dropped, count, _ = _route(*case)
    _, dropped2, _ = so.assign_slots(idx, h.shape[1], C + extra)
    assert np.all(dropped2 <= dropped)  # kept at C stays kept at C + extra


@PROP
@given(routing_case())
def test_loss_bounds_and_relabelling(case):
    x, w, b, cf = case
    C, h, p, idx, slot, dropped, count, aux = _route(x, w, b, cf)
    T, N = h.shape
    if T == 0:
        assert aux == 0.0
        return
    assert 0.0 < aux <= N * (1 + 1e-12)
    # relabel the experts: every count and the loss follow the permutation
    perm = np.random.default_rng(N + T).permutation(N)
    _, h2, p2, idx2, _, _, count2, aux2 = _route(x, w[perm], None if b is None else b[perm], cf)
    gap = so.top1(h)[1]
    clear = gap > 1e-9  # relabelling may reorder exact ties only
    assert np.array_equal(perm[idx2[clear]], idx[clear])
    if clear.all():
        assert np.array_equal(count2, count[perm])
        assert aux2 == pytest.approx(aux, rel=1e-12)


@settings(max_examples=25, deadline=None, derandomize=True, database=None)
@given(routing_case(), st.sampled_from([8, 16]))
def test_layer_output_rows(case, f):
    x, w, b, cf = case
    T, d = x.shape
    N = w.shape[0]
    rng = np.random.default_rng(T * 7 + N)
    w_in = rng.standard_normal((N, f, d)) * np.sqrt(0.1 / d) if N <= 128 else None
    if w_in is None:  # 2048 experts: draw weights only for the experts in use
        def get(i, _r={}):
            if i not in _r:
                g = np.random.default_rng(i)
                _r[i] = (g.standard_normal((f, d)) * np.sqrt(0.1 / d), g.standard_normal((d, f)) * np.sqrt(0.1 / f))
            return _r[i]
        src = (get, None)
    else:
        w_out = rng.standard_normal((N, d, f)) * np.sqrt(0.1 / f)
        src = (w_in, w_out)
    C = so.expert_capacity(T, N, cf)
    out = so.forward(x, w, b, *src, C)
    assert np.all(out["y_bare"][out["dropped"]] == 0.0)
    # doubling every W_out doubles every output row exactly (power-of-two
    # scaling is exact in binary floating point; routing does not see W_out)
    if w_in is not None:
        out2 = so.forward(x, w, b, w_in, 2.0 * src[1], C)
        assert np.array_equal(out2["y_bare"], 2.0 * out["y_bare"])
        assert np.array_equal(out2["expert_idx"], out["expert_idx"])
    # residual mode adds x to every row, dropped rows included
    res = so.forward(x, w, b, *src, C, add_residual=True)
    assert np.array_equal(res["y"], x + out["y_bare"])
