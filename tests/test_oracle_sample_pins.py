"""Pins of the oracle's sampler (no GPU): closed forms, exact arithmetic and invariants.

The readings under test (the pages name greedy and stochastic sampling with an fp64 CPU oracle,
Leone "What ships", and give no formula): order by logit descending, ties by index ascending;
weights W = floor(2^31 e^d), d = (l - l_max) / T; top-k keeps the first k of the order; top-p keeps
the shortest prefix whose weight reaches ceil(p Wk); the draw U = floor(u Wp) picks the first element
whose running weight exceeds U.  Expected values here come from exact rational / decimal arithmetic or
from reasoning about special inputs, never from the oracle's own formulas.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle

getcontext().prec = 60
TWO31 = 1 << 31


def _exact_exp(d: float) -> Decimal:
    return Decimal(d).exp()


def _ulp(x: float) -> float:
    return math.ulp(x)


def test_exp_within_one_ulp_of_exact():
    ds = np.concatenate([np.linspace(-22.0, 0.0, 4001), -np.arange(0, 33) * math.log(2.0) / 2.0,
                         -np.arange(0, 32) * math.log(2.0), [-1e-300, -5e-324, -21.999999999999996]])
    for d in ds:
        d = float(d)
        if d < -22.0:
            continue
        got = oracle.exp_neg(d)
        ex = _exact_exp(d)
        assert abs(Decimal(got) - ex) <= Decimal(_ulp(float(ex))), d
    assert oracle.exp_neg(0.0) == 1.0
    assert oracle.exp_neg(-0.0) == 1.0


def test_weight_is_the_floor_of_exact_value():
    rng = np.random.default_rng(7)
    ds = np.concatenate([rng.uniform(-22.0, 0.0, 3000), rng.uniform(-1e-6, 0.0, 200), [0.0, -22.0]])
    for d in ds:
        d = float(d)
        ex = _exact_exp(d) * TWO31
        fl = int(ex)  # floor of a positive value
        if ex - fl < Decimal("1e-6") or (fl + 1) - ex < Decimal("1e-6"):
            continue  # a last-place difference may move the floor here
        assert oracle.sample_weight(d) == fl, d
    assert oracle.sample_weight(0.0) == TWO31
    assert oracle.sample_weight(-22.0000001) == 0
    assert oracle.sample_weight(float("nan")) == 0
    assert oracle.sample_weight(float("-inf")) == 0
    # e^-22 sits below 2^-31, so nothing is cut that the floor would keep
    assert _exact_exp(-22.0) * TWO31 < 1


def test_greedy_is_first_argmax():
    rng = np.random.default_rng(11)
    lg = rng.normal(0, 3, (6, 4099)).astype(np.float32)
    lg[1, 17] = lg[1, 4000] = lg[1].max() + 1  # tie at the max: the lower index wins
    lg[2, :] = 0.0
    lg[3, 5] = np.float32(-0.0)
    lg[3, :] = np.float32(-1.0)
    lg[3, 9] = np.float32(-0.0)
    lg[3, 2] = np.float32(0.0)  # -0 equals +0: index 2 comes first
    lg[4, ::3] = np.nan  # NaN sorts last
    expect = []
    for r in lg:
        finite = np.where(np.isnan(r), -np.inf, r)
        expect.append(int(np.flatnonzero(finite == finite.max())[0]))
    for t, k in [(0.0, 0), (-1.0, 50), (float("nan"), 0), (1.0, 1), (5e-324, 0)]:
        tok = oracle.sample(lg, t, 0.9, k, 0.77)
        assert list(tok) == expect, (t, k)


def test_uniform_row_closed_form():
    """All-equal logits: every weight is 2^31, so the token is floor(u n) over the kept n."""
    v = 8
    lg = np.full((1, v), 2.5, np.float32)
    for u in [0.0, 0.1, 0.125, 0.375, 0.5, 0.874, 0.875, 0.999999]:
        assert oracle.sample(lg, 1.0, 1.0, 0, u)[0] == math.floor(u * v)
        assert oracle.sample(lg, 0.3, 1.0, 3, u)[0] == math.floor(u * 3)
        # p = 3/8 exactly: the prefix is the first 3 (a strict comparison would keep 4)
        assert oracle.sample(lg, 2.0, 0.375, 0, u)[0] == math.floor(u * 3)
        # p just above 3/8 needs a fourth element
        assert oracle.sample(lg, 2.0, 0.375 + 2 ** -40, 0, u)[0] == math.floor(u * 4)
    tok, wk, wp = oracle.sample(lg, 1.0, 0.375, 5, 0.5, diag=True)
    assert wk[0] == 5 * TWO31 and wp[0] == 2 * TWO31  # ceil(0.375 * 5) = 2 elements
    # u outside [0, 1) clamps to the ends
    assert oracle.sample(lg, 1.0, 1.0, 0, 1.0)[0] == v - 1
    assert oracle.sample(lg, 1.0, 1.0, 0, -3.0)[0] == 0
    assert oracle.sample(lg, 1.0, 1.0, 0, float("nan"))[0] == 0


def test_two_level_row_closed_form():
    """Two logit values a > b: group A in index order, then group B; weights 2^31 and floor(2^31 e^((b-a)/T))."""
    rng = np.random.default_rng(3)
    v = 97
    a, b, T = 1.75, -0.5, 0.8
    lg = np.full(v, b, np.float32)
    ia = np.sort(rng.choice(v, 11, replace=False))
    lg[ia] = a
    ib = np.array([i for i in range(v) if i not in set(ia.tolist())])
    d = (float(np.float32(b)) - float(np.float32(a))) * (1.0 / T)
    wb = int(_exact_exp(d) * TWO31)
    total = len(ia) * TWO31 + len(ib) * wb
    for u in np.linspace(0, 1, 301, endpoint=False):
        U = math.floor(Fraction(float(u)) * total)
        if U < len(ia) * TWO31:
            expect = ia[U // TWO31]
        else:
            expect = ib[(U - len(ia) * TWO31) // wb]
        assert oracle.sample(lg[None], T, 1.0, 0, float(u))[0] == expect


def test_top_k_splits_a_tie_by_index():
    lg = np.array([[1.0, 5.0, 5.0, 5.0, 5.0, -2.0]], np.float32)
    for u, e in [(0.0, 1), (0.49, 1), (0.5, 2), (0.99, 2)]:
        assert oracle.sample(lg, 1.0, 1.0, 2, u)[0] == e
    tok, wk, wp = oracle.sample(lg, 1.0, 1.0, 2, 0.3, diag=True)
    assert wk[0] == 2 * TWO31 == wp[0]


def test_masked_and_degenerate_rows():
    lg = np.full((4, 64), -np.inf, np.float32)
    lg[1, 40] = 3.0  # one finite logit among masked ones
    lg[2, :] = np.nan
    lg[2, 7] = -1.0
    lg[3, :5] = np.inf  # non-finite maximum: greedy
    for u in [0.0, 0.3, 0.999]:
        tok = oracle.sample(lg, 1.0, 0.9, 0, u)
        assert list(tok) == [0, 40, 7, 0]


def _numpy_kept(l, T, k, p):
    """Kept set and renormalised probabilities from a float64 softmax (independent of the weights)."""
    order = np.lexsort((np.arange(len(l)), -l.astype(np.float64)))
    kk = len(l) if k <= 0 or k >= len(l) else k
    top = order[:kk]
    z = (l[top].astype(np.float64) - float(l[order[0]])) / T
    pr = np.exp(z)
    pr /= pr.sum()
    c = np.cumsum(pr)
    m = kk if p >= 1 else int(np.searchsorted(c, p - 1e-12)) + 1
    return order, top[:m], pr[:m] / pr[:m].sum(), c


@pytest.mark.parametrize("T,k,p", [(0.7, 50, 0.9), (1.0, 0, 0.8), (1.3, 0, 1.0), (0.5, 7, 1.0)])
def test_draw_frequencies_match_softmax(T, k, p):
    rng = np.random.default_rng(int(T * 100) + k)
    v = 1000
    l = rng.normal(0, 2.0, v).astype(np.float32)
    order, kept, prob, c = _numpy_kept(l, T, k, p)
    n = 40000
    us = (np.arange(n) + 0.5) / n
    toks = oracle.sample(np.repeat(l[None], n, 0), np.full(n, T), np.full(n, p), np.full(n, k, np.int32), us)
    assert set(np.unique(toks).tolist()) <= set(kept.tolist())
    freq = np.bincount(toks, minlength=v)[kept] / n
    assert np.abs(freq - prob).max() <= 2.0 / n + 1e-6
    # the token's rank in the order never decreases as u grows
    rank = np.empty(v, np.int64)
    rank[order] = np.arange(v)
    assert np.all(np.diff(rank[toks]) >= 0)


def test_rows_are_independent():
    rng = np.random.default_rng(5)
    lg = rng.normal(0, 1.5, (5, 777)).astype(np.float32)
    T = np.array([0.0, 0.6, 1.0, 2.0, 0.9])
    P = np.array([1.0, 0.95, 0.5, 1.0, 0.7])
    K = np.array([0, 40, 0, 3, 1], np.int32)
    U = rng.random(5)
    both = oracle.sample(lg, T, P, K, U)
    alone = [int(oracle.sample(lg[i:i + 1], T[i], P[i], K[i], U[i])[0]) for i in range(5)]
    assert list(both) == alone
