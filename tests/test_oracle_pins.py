"""Pins for the fp64 oracle, against facts fixed independently of its code.

Each test checks the oracle against something it does not share code with:
hand-derived fixtures (tests/golden/), closed forms, library routines
(numpy.cumsum, math.fsum, scipy.signal.lfilter, numpy.matmul, complex
arithmetic), exact rational arithmetic over random association trees, O(T^2)
brute force, and adjoint identities (tangent-linear dot products and central
finite differences). A plausible slip anywhere in the oracle -- a dropped term,
a wrong sign, an off-by-one shift, a transposed operand, a segment leak --
makes at least one of these fail.
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import scipy.signal
import scipy.special

import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _arr(v):
    return None if v is None else np.array(v, dtype=np.float64)


# ---------------------------------------------------------------------------
# hand-derived fixtures
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", _load("scalar_hand.json")["cases"], ids=lambda c: c["name"])
def test_scalar_hand_fixture(oracle_lib, case):
    o = oracle_lib
    g, x, dy = _arr(case["g"]), _arr(case["x"]), _arr(case["dy"])
    h0, cu = _arr(case["h0"]), case["cu_seqlens"]
    h = o.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=case["reverse"])
    assert np.array_equal(h, _arr(case["h"]))
    dx, dg, dh0 = o.scan_bwd(g, h, dy, h0=h0, cu_seqlens=cu, reverse=case["reverse"])
    assert np.array_equal(dx, _arr(case["dx"]))
    assert np.array_equal(dg, _arr(case["dg"]))
    assert np.array_equal(dh0, _arr(case["dh0"]))


@pytest.mark.parametrize("case", _load("log_hand.json")["cases"], ids=lambda c: c["name"])
def test_log_hand_fixture(oracle_lib, case):
    with np.errstate(divide="ignore"):
        la, lb = np.log(_arr(case["a"])), np.log(_arr(case["b"]))
        lh0 = None if case["h0"] is None else np.log(_arr(case["h0"]))
    h = oracle_lib.scan_log_fwd(la, lb, log_h0=lh0, reverse=case["reverse"])
    np.testing.assert_allclose(h, _arr(case["h"]), rtol=1e-14, atol=0)


@pytest.mark.parametrize("case", _load("matrix_hand.json")["cases"], ids=lambda c: c["name"])
def test_matrix_hand_fixture(oracle_lib, case):
    o = oracle_lib
    A, B, dy = _arr(case["A"]), _arr(case["B"]), _arr(case["dy"])
    h = o.matrix_affine_scan_fwd(A, B, h0=_arr(case["h0"]), reverse=case["reverse"])
    assert np.array_equal(h, _arr(case["h"]))
    dA, dB, dh0 = o.matrix_affine_scan_bwd(A, h, dy, h0=_arr(case["h0"]), reverse=case["reverse"])
    assert np.array_equal(dB, _arr(case["dB"]))
    assert np.array_equal(dA, _arr(case["dA"]))
    assert np.array_equal(dh0, _arr(case["dh0"]))


# ---------------------------------------------------------------------------
# special cases and closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("reverse", [False, True])
def test_zero_gate_gives_x(oracle_lib, reverse):
    """a_t = 0 erases the prefix (RG-LRU audit, 'Exact real chunk algebra'): h = x exactly."""
    r = _rng(1)
    x = r.standard_normal((5, 77))
    h0 = r.standard_normal((3, 5))
    cu = np.array([0, 10, 10, 77], dtype=np.int32)
    h = oracle_lib.scan_fwd(np.zeros_like(x), x, h0=h0, cu_seqlens=cu, reverse=reverse)
    assert np.array_equal(h, x)
    dy = r.standard_normal(x.shape)
    dx, dg, _ = oracle_lib.scan_bwd(np.zeros_like(x), h, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    assert np.array_equal(dx, dy)


def test_unit_gate_is_cumsum(oracle_lib):
    """a_t = 1 turns the scan into h0 + a running sum; compare with exact fsum prefixes."""
    r = _rng(2)
    x = r.standard_normal((4, 300))
    h0 = r.standard_normal(4)
    h = oracle_lib.scan_fwd(np.ones_like(x), x, h0=h0)
    for i in range(4):
        exact = np.array([math.fsum([h0[i], *x[i, : t + 1]]) for t in range(300)])
        np.testing.assert_allclose(h[i], exact, rtol=0, atol=1e-12)
        np.testing.assert_allclose(h[i], h0[i] + np.cumsum(x[i]), rtol=0, atol=1e-12)
    dy = r.standard_normal(x.shape)
    dx, _, _ = oracle_lib.scan_bwd(np.ones_like(x), h, dy, h0=h0)
    np.testing.assert_allclose(dx, np.cumsum(dy[:, ::-1], axis=1)[:, ::-1], rtol=0, atol=1e-12)


@pytest.mark.parametrize("a", [0.3, 0.9, -0.7, 1.05])
def test_constant_gate_geometric(oracle_lib, a):
    """Constant a with x = 1: h_n = a^n h0 + (1 - a^n)/(1 - a); random x: scipy lfilter."""
    T = 200
    h0 = 0.75
    h = oracle_lib.scan_fwd(np.full((1, T), a), np.ones((1, T)), h0=np.array([h0]))[0]
    n = np.arange(1, T + 1)
    closed = a ** n * h0 + (1 - a ** n) / (1 - a)
    np.testing.assert_allclose(h, closed, rtol=1e-12, atol=1e-12)
    x = _rng(3).standard_normal(T)
    h = oracle_lib.scan_fwd(np.full((1, T), a), x[None], h0=np.array([h0]))[0]
    ref, _ = scipy.signal.lfilter([1.0], [1.0, -a], x, zi=[a * h0])
    np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-11)


def test_brute_force_sum_of_products(oracle_lib):
    """h_t = (prod_{r=s..t} g_r) h0 + sum_u (prod_{r=u+1..t} g_r) x_u, O(T^2), every segment."""
    r = _rng(4)
    T = 48
    g = r.uniform(-1.2, 1.2, (3, T))
    x = r.standard_normal((3, T))
    cu = np.array([0, 5, 5, 20, 48], dtype=np.int32)
    h0 = r.standard_normal((4, 3))
    for reverse in (False, True):
        h = oracle_lib.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=reverse)
        ref = np.zeros_like(h)
        for row in range(3):
            for s in range(4):
                idx = list(range(cu[s], cu[s + 1]))
                if reverse:
                    idx = idx[::-1]
                for j, t in enumerate(idx):
                    tot = np.prod([g[row, idx[q]] for q in range(0, j + 1)]) * h0[s, row]
                    for i in range(j + 1):
                        tot += np.prod([g[row, idx[q]] for q in range(i + 1, j + 1)]) * x[row, idx[i]]
                    ref[row, t] = tot
        np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-12)


def _compose(e, l):
    """(P, Q) of 'apply e then l' for maps h -> P h + Q."""
    return (l[0] * e[0], l[0] * e[1] + l[1])


def _tree_reduce(items, rnd):
    """Combine a list of maps in order with a random binary bracketing."""
    if len(items) == 1:
        return items[0]
    cut = rnd.randint(1, len(items) - 1)
    return _compose(_tree_reduce(items[:cut], rnd), _tree_reduce(items[cut:], rnd))


def test_regrouping_exact_rationals(oracle_lib):
    """The affine monoid (minGRU page, 'One associative-scan family') is associative: any
    bracketing of the steps, in exact rationals, gives the same prefix, and the fp64
    oracle must agree with it."""
    rnd = random.Random(5)
    for trial in range(40):
        T = rnd.randint(1, 16)
        g = [Fraction(rnd.randint(-9, 9), rnd.randint(1, 8)) for _ in range(T)]
        x = [Fraction(rnd.randint(-9, 9), rnd.randint(1, 8)) for _ in range(T)]
        h0 = Fraction(rnd.randint(-5, 5), 3)
        ref = []
        for t in range(T):
            P, Q = _tree_reduce(list(zip(g[: t + 1], x[: t + 1])), rnd)
            P2, Q2 = _tree_reduce(list(zip(g[: t + 1], x[: t + 1])), rnd)
            assert (P, Q) == (P2, Q2)
            ref.append(P * h0 + Q)
        h = oracle_lib.scan_fwd(np.array([[float(v) for v in g]]), np.array([[float(v) for v in x]]),
                                h0=np.array([float(h0)]))[0]
        refd = np.array([float(v) for v in ref])
        np.testing.assert_allclose(h, refd, rtol=1e-13, atol=1e-13)


def test_reverse_is_flip_scan_flip(oracle_lib):
    r = _rng(6)
    T = 101
    g, x = r.uniform(0, 1, (4, T)), r.standard_normal((4, T))
    cu = np.array([0, 1, 40, 40, 101], dtype=np.int32)
    h0 = r.standard_normal((4, 4))
    hr = oracle_lib.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=True)
    for s in range(4):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        hf = oracle_lib.scan_fwd(g[:, a:b][:, ::-1], x[:, a:b][:, ::-1], h0=h0[s])
        assert np.array_equal(hr[:, a:b], hf[:, ::-1])


def test_varlen_equals_separate_sequences(oracle_lib):
    """cu_seqlens packing: each sequence is scanned on its own, no cross-document leakage."""
    r = _rng(7)
    T = 300
    g, x, dy = r.uniform(0, 1, (3, T)), r.standard_normal((3, T)), r.standard_normal((3, T))
    cu = gen.segments_random(r, T, 9)
    h0 = r.standard_normal((9, 3))
    # poison one segment: nothing else may change
    s_bad = int(np.argmax(np.diff(cu)))
    g[:, cu[s_bad]:cu[s_bad + 1]] = np.nan
    for reverse in (False, True):
        h = oracle_lib.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=reverse)
        dx, dg, dh0 = oracle_lib.scan_bwd(g, h, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
        for s in range(9):
            a, b = cu[s], cu[s + 1]
            if b == a:
                assert np.all(dh0[s] == 0)
                continue
            hs = oracle_lib.scan_fwd(g[:, a:b], x[:, a:b], h0=h0[s], reverse=reverse)
            assert np.array_equal(h[:, a:b], hs, equal_nan=True)
            dxs, dgs, dh0s = oracle_lib.scan_bwd(g[:, a:b], hs, dy[:, a:b], h0=h0[s], reverse=reverse)
            assert np.array_equal(dx[:, a:b], dxs, equal_nan=True)
            assert np.array_equal(dg[:, a:b], dgs, equal_nan=True)
            if s != s_bad:
                assert np.all(np.isfinite(h[:, a:b])) and np.all(np.isfinite(dg[:, a:b]))


def test_exact_integer_mode(oracle_lib):
    """g in {0,1}, x in {-1,0,1}: the scan is exact integer arithmetic."""
    r = _rng(8)
    g, x, dy = gen.exact_mode(r, (3, 500), max_run=64)
    h0 = r.integers(-1, 2, size=3).astype(np.float64)
    h = oracle_lib.scan_fwd(g, x, h0=h0)
    for i in range(3):
        st = int(h0[i])
        for t in range(500):
            st = int(g[i, t]) * st + int(x[i, t])
            assert h[i, t] == st


# ---------------------------------------------------------------------------
# backward: adjoint identities
# ---------------------------------------------------------------------------
def _tangent_scalar(g, x, h0, gd, xd, h0d, cu, reverse):
    """Forward-mode derivative of the scalar scan: hd_t = gd_t h_{t-1} + g_t hd_{t-1} + xd_t."""
    rows, T = g.shape
    h = np.zeros_like(g)
    hd = np.zeros_like(g)
    for s in range(len(cu) - 1):
        idx = list(range(cu[s], cu[s + 1]))
        if reverse:
            idx = idx[::-1]
        st = h0[s].copy()
        std = h0d[s].copy()
        for t in idx:
            std = gd[:, t] * st + g[:, t] * std + xd[:, t]
            st = g[:, t] * st + x[:, t]
            h[:, t], hd[:, t] = st, std
    return h, hd


@pytest.mark.parametrize("reverse", [False, True])
def test_scalar_adjoint_dot_product(oracle_lib, reverse):
    """<dy, J v> = <J^T dy, v> with J v from the tangent-linear recurrence."""
    r = _rng(9)
    T = 257
    g, x = r.uniform(-1, 1, (4, T)), r.standard_normal((4, T))
    cu = gen.segments_random(r, T, 6)
    h0 = r.standard_normal((6, 4))
    gd, xd, h0d = r.standard_normal(g.shape), r.standard_normal(g.shape), r.standard_normal(h0.shape)
    dy = r.standard_normal(g.shape)
    href, hd = _tangent_scalar(g, x, h0, gd, xd, h0d, cu, reverse)
    h = oracle_lib.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=reverse)
    np.testing.assert_allclose(h, href, rtol=1e-13, atol=1e-13)
    dx, dg, dh0 = oracle_lib.scan_bwd(g, h, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    lhs = np.sum(dy * hd)
    rhs = np.sum(dg * gd) + np.sum(dx * xd) + np.sum(dh0 * h0d)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_scalar_finite_differences(oracle_lib):
    r = _rng(10)
    T = 24
    g, x = r.uniform(-1, 1, (2, T)), r.standard_normal((2, T))
    cu = np.array([0, 9, 24], dtype=np.int32)
    h0 = r.standard_normal((2, 2))
    dy = r.standard_normal(g.shape)
    for reverse in (False, True):
        L = lambda g_, x_, h0_: np.sum(dy * oracle_lib.scan_fwd(g_, x_, h0=h0_, cu_seqlens=cu, reverse=reverse))
        h = oracle_lib.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=reverse)
        dx, dg, dh0 = oracle_lib.scan_bwd(g, h, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
        eps = 1e-6
        for (i, t) in [(0, 0), (0, 8), (1, 9), (1, 23), (0, 15)]:
            for arr, grad in ((g, dg), (x, dx)):
                p, m = arr.copy(), arr.copy()
                p[i, t] += eps
                m[i, t] -= eps
                args_p = (p, x, h0) if arr is g else (g, p, h0)
                args_m = (m, x, h0) if arr is g else (g, m, h0)
                fd = (L(*args_p) - L(*args_m)) / (2 * eps)
                assert abs(fd - grad[i, t]) < 1e-6 * max(1, abs(fd))
        for s in range(2):
            for i in range(2):
                p, m = h0.copy(), h0.copy()
                p[s, i] += eps
                m[s, i] -= eps
                fd = (L(g, x, p) - L(g, x, m)) / (2 * eps)
                assert abs(fd - dh0[s, i]) < 1e-6 * max(1, abs(fd))


# ---------------------------------------------------------------------------
# log space
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("reverse", [False, True])
def test_log_equals_linear(oracle_lib, reverse):
    """The log-space form is the same recurrence: compare with the linear scan on
    a = exp(log_a), b = exp(log_b), using the log-space workload's distributions."""
    d = gen.logspace(B=2, D=8, T=2048)
    la, lb = d["log_a"].astype(np.float64), d["log_b"].astype(np.float64)
    cu = np.array([0, 700, 700, 2048], dtype=np.int32)
    lh0 = _rng(11).standard_normal((3, 16))
    h = oracle_lib.scan_log_fwd(la, lb, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
    hl = oracle_lib.scan_fwd(np.exp(la), np.exp(lb), h0=np.exp(lh0), cu_seqlens=cu, reverse=reverse)
    np.testing.assert_allclose(h, hl, rtol=1e-11, atol=0)


def test_log_wide_dynamic_range(oracle_lib):
    """Shifting every log_b by c scales h by e^c (the recurrence is linear in b);
    with c = -600 the values sit near fp64's lower range and stay accurate."""
    r = _rng(12)
    la = -np.log1p(np.exp(r.standard_normal((2, 500))))
    lb = r.standard_normal((2, 500))
    h1 = oracle_lib.scan_log_fwd(la, lb)
    h2 = oracle_lib.scan_log_fwd(la, lb - 600.0)
    np.testing.assert_allclose(h2, h1 * np.exp(-600.0), rtol=1e-12)
    assert np.all(h2 > 0)


def test_log_zero_gate_restarts(oracle_lib):
    r = _rng(13)
    la = -np.log1p(np.exp(r.standard_normal((3, 64))))
    lb = r.standard_normal((3, 64))
    la[:, 20] = -np.inf
    h = oracle_lib.scan_log_fwd(la, lb, log_h0=r.standard_normal(3))
    np.testing.assert_allclose(h[:, 20], np.exp(lb[:, 20]), rtol=1e-15)
    h_tail = oracle_lib.scan_log_fwd(la[:, 21:], lb[:, 21:], log_h0=np.log(h[:, 20]))
    np.testing.assert_allclose(h[:, 21:], h_tail, rtol=1e-13)


def _tangent_log(la, lb, lh0, lad, lbd, lh0d, cu, reverse):
    """Forward-mode derivative of h_t = a_t h_{t-1} + b_t with a = e^{log_a},
    b = e^{log_b}, h0 = e^{log_h0}, for perturbations of the log inputs:
    hd_t = a_t lad_t h_{t-1} + a_t hd_{t-1} + b_t lbd_t, hd before a segment = h0 lh0d."""
    a, b = np.exp(la), np.exp(lb)
    h, hd = np.zeros_like(la), np.zeros_like(la)
    for s in range(len(cu) - 1):
        idx = list(range(cu[s], cu[s + 1]))
        if reverse:
            idx = idx[::-1]
        st = np.exp(lh0[s])
        std = st * lh0d[s]
        for t in idx:
            std = a[:, t] * lad[:, t] * st + a[:, t] * std + b[:, t] * lbd[:, t]
            st = a[:, t] * st + b[:, t]
            h[:, t], hd[:, t] = st, std
    return h, hd


@pytest.mark.parametrize("reverse", [False, True])
def test_log_bwd_adjoint_dot_product(oracle_lib, reverse):
    """<dy, J v> = <J^T dy, v> for the log-space adjoint, J v from the tangent-linear
    recurrence written in linear space."""
    r = _rng(14)
    T = 301
    la = -np.log1p(np.exp(r.standard_normal((4, T))))
    lb = r.standard_normal((4, T))
    cu = gen.segments_random(r, T, 5)
    lh0 = r.standard_normal((5, 4))
    lad, lbd, lh0d = r.standard_normal(la.shape), r.standard_normal(la.shape), r.standard_normal(lh0.shape)
    dy = r.standard_normal(la.shape)
    href, hd = _tangent_log(la, lb, lh0, lad, lbd, lh0d, cu, reverse)
    h = oracle_lib.scan_log_fwd(la, lb, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
    np.testing.assert_allclose(h, href, rtol=1e-12)
    dla, dlb, dlh0 = oracle_lib.scan_log_bwd(la, lb, h, dy, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
    lhs = np.sum(dy * hd)
    rhs = np.sum(dla * lad) + np.sum(dlb * lbd) + np.sum(dlh0 * lh0d)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_log_bwd_finite_differences(oracle_lib):
    """Central differences of <dy, scan_log_fwd(.)> in every kind of log input."""
    r = _rng(15)
    T = 30
    la = -np.log1p(np.exp(r.standard_normal((2, T))))
    lb = r.standard_normal((2, T))
    cu = np.array([0, 11, 11, 30], dtype=np.int32)
    lh0 = r.standard_normal((3, 2))
    dy = r.standard_normal(la.shape)
    eps = 1e-6
    for reverse in (False, True):
        L = lambda a_, b_, h0_: np.sum(dy * oracle_lib.scan_log_fwd(a_, b_, log_h0=h0_, cu_seqlens=cu, reverse=reverse))
        h = oracle_lib.scan_log_fwd(la, lb, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
        dla, dlb, dlh0 = oracle_lib.scan_log_bwd(la, lb, h, dy, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
        for (i, t) in [(0, 0), (0, 10), (1, 11), (1, 29), (0, 17), (1, 5)]:
            for which in ("a", "b"):
                arr, grad = (la, dla) if which == "a" else (lb, dlb)
                p, m = arr.copy(), arr.copy()
                p[i, t] += eps
                m[i, t] -= eps
                fd = (L(p, lb, lh0) - L(m, lb, lh0)) / (2 * eps) if which == "a" else \
                     (L(la, p, lh0) - L(la, m, lh0)) / (2 * eps)
                assert abs(fd - grad[i, t]) < 1e-6 * max(1, abs(fd)), (reverse, which, i, t, fd, grad[i, t])
        for s in (0, 2):  # segment 1 is empty: its h0 touches nothing
            for i in range(2):
                p, m = lh0.copy(), lh0.copy()
                p[s, i] += eps
                m[s, i] -= eps
                fd = (L(la, lb, p) - L(la, lb, m)) / (2 * eps)
                assert abs(fd - dlh0[s, i]) < 1e-6 * max(1, abs(fd))
        assert np.all(dlh0[1] == 0.0)


def test_log_bwd_shift_scales_gradients(oracle_lib):
    """log_b + c and log_h0 + c scale h by e^c and leave the adjoint state alone,
    so every log-input gradient of <dy, h> scales by e^c."""
    r = _rng(16)
    la = -np.log1p(np.exp(r.standard_normal((3, 400))))
    lb = r.standard_normal((3, 400))
    lh0 = r.standard_normal(3)
    dy = r.standard_normal(la.shape)
    c = -3.25
    h1 = oracle_lib.scan_log_fwd(la, lb, log_h0=lh0)
    h2 = oracle_lib.scan_log_fwd(la, lb + c, log_h0=lh0 + c)
    g1 = oracle_lib.scan_log_bwd(la, lb, h1, dy, log_h0=lh0)
    g2 = oracle_lib.scan_log_bwd(la, lb + c, h2, dy, log_h0=lh0 + c)
    for x1, x2 in zip(g1, g2):
        np.testing.assert_allclose(x2, x1 * np.exp(c), rtol=1e-12, atol=1e-300)


def test_log_bwd_zero_gate(oracle_lib):
    """log_a = -inf (a = 0) at t: no gradient reaches log_a_t, and nothing after t
    reaches the log inputs before t."""
    r = _rng(17)
    la = -np.log1p(np.exp(r.standard_normal((2, 80))))
    lb = r.standard_normal((2, 80))
    la[:, 30] = -np.inf
    dy = r.standard_normal(la.shape)
    h = oracle_lib.scan_log_fwd(la, lb)
    dla, dlb, _ = oracle_lib.scan_log_bwd(la, lb, h, dy)
    assert np.all(dla[:, 30] == 0.0)
    dy2 = dy.copy()
    dy2[:, 30:] = r.standard_normal((2, 50))
    dla2, dlb2, _ = oracle_lib.scan_log_bwd(la, lb, h, dy2)
    assert np.array_equal(dla[:, :30], dla2[:, :30]) and np.array_equal(dlb[:, :30], dlb2[:, :30])


def test_log_bwd_is_linear_adjoint_through_exp(oracle_lib):
    """Chain rule through exp against the independently pinned linear adjoint:
    dlog_b = dx * b, dlog_a = dg * a, dlog_h0 = dh0 * h0 (to rounding: the two sides
    take exp in different libraries)."""
    d = gen.logspace(B=2, D=4, T=1500)
    la, lb = d["log_a"].astype(np.float64), d["log_b"].astype(np.float64)
    r = _rng(18)
    cu = np.array([0, 600, 1500], dtype=np.int32)
    lh0 = r.standard_normal((2, 8))
    dy = r.standard_normal(la.shape)
    for reverse in (False, True):
        h = oracle_lib.scan_log_fwd(la, lb, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
        dla, dlb, dlh0 = oracle_lib.scan_log_bwd(la, lb, h, dy, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
        dx, dg, dh0 = oracle_lib.scan_bwd(np.exp(la), h, dy, h0=np.exp(lh0), cu_seqlens=cu, reverse=reverse)
        np.testing.assert_allclose(dlb, dx * np.exp(lb), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(dla, dg * np.exp(la), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(dlh0, dh0 * np.exp(lh0), rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# gate activations (scans that take gate logits)
# ---------------------------------------------------------------------------
def test_gate_sigmoid_against_library(oracle_lib):
    z = np.concatenate([np.linspace(-40, 40, 2001), [-750.0, 750.0, 0.0]])
    g = oracle_lib.gate(1, z)
    np.testing.assert_allclose(g, scipy.special.expit(z), rtol=1e-15, atol=0)
    assert g[-1] == 0.5 and g[-3] == 0.0 and g[-2] == 1.0
    # sigmoid(-z) = 1 - sigmoid(z) (absolute: the right side cancels for large z)
    np.testing.assert_allclose(oracle_lib.gate(1, -z), 1.0 - g, rtol=0, atol=3e-16)


def test_gate_neg_softplus_against_library(oracle_lib):
    z = np.concatenate([np.linspace(-40, 40, 2001), [-700.0, 700.0]])
    la = oracle_lib.gate(2, z)
    np.testing.assert_allclose(la, -np.logaddexp(0.0, z), rtol=1e-15, atol=0)
    # log a = -softplus(z) is log sigmoid(-z): a = sigmoid(-z)
    np.testing.assert_allclose(np.exp(la), scipy.special.expit(-z), rtol=1e-13, atol=0)


@pytest.mark.parametrize("kind", [1, 2])
def test_gate_grad_finite_differences(oracle_lib, kind):
    r = _rng(19)
    z = np.concatenate([r.standard_normal(50) * 4, [0.0, -30.0, 30.0]])
    dact = r.standard_normal(z.shape)
    dz = oracle_lib.gate_grad(kind, z, dact)
    eps = 1e-6
    fd = (oracle_lib.gate(kind, z + eps) - oracle_lib.gate(kind, z - eps)) / (2 * eps) * dact
    np.testing.assert_allclose(dz, fd, rtol=1e-7, atol=1e-10)


@pytest.mark.parametrize("reverse", [False, True])
def test_gated_scans_adjoint_dot_product(oracle_lib, reverse):
    """<dy, J v> = <J^T dy, v> through the gate: tangents of z enter as f'(z) zd."""
    r = _rng(20)
    T = 203
    z, x = r.standard_normal((3, T)) * 2, r.standard_normal((3, T))
    cu = gen.segments_random(r, T, 4)
    h0 = r.standard_normal((4, 3))
    zd, xd, h0d = r.standard_normal(z.shape), r.standard_normal(z.shape), r.standard_normal(h0.shape)
    dy = r.standard_normal(z.shape)
    g = scipy.special.expit(z)
    _, hd = _tangent_scalar(g, x, h0, g * (1 - g) * zd, xd, h0d, cu, reverse)
    h = oracle_lib.scan_fwd_gated(z, x, h0=h0, cu_seqlens=cu, reverse=reverse)
    dx, dz, dh0 = oracle_lib.scan_bwd_gated(z, h, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    lhs = np.sum(dy * hd)
    rhs = np.sum(dz * zd) + np.sum(dx * xd) + np.sum(dh0 * h0d)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # log space: log_a = -softplus(z), tangent of log_a = -sigmoid(z) zd
    lb = r.standard_normal(z.shape)
    lh0 = r.standard_normal((4, 3))
    lbd, lh0d = r.standard_normal(z.shape), r.standard_normal(lh0.shape)
    la = -np.logaddexp(0.0, z)
    _, hd = _tangent_log(la, lb, lh0, -scipy.special.expit(z) * zd, lbd, lh0d, cu, reverse)
    h = oracle_lib.scan_log_fwd_gated(z, lb, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
    dz, dlb, dlh0 = oracle_lib.scan_log_bwd_gated(z, lb, h, dy, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
    lhs = np.sum(dy * hd)
    rhs = np.sum(dz * zd) + np.sum(dlb * lbd) + np.sum(dlh0 * lh0d)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


# ---------------------------------------------------------------------------
# matrix-affine
# ---------------------------------------------------------------------------
def test_matrix_k1_is_scalar(oracle_lib):
    r = _rng(14)
    g, x = r.uniform(-1, 1, (3, 90)), r.standard_normal((3, 90))
    cu = np.array([0, 30, 90], dtype=np.int32)
    h0 = r.standard_normal((2, 3))
    for reverse in (False, True):
        hs = oracle_lib.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=reverse)
        hm = oracle_lib.matrix_affine_scan_fwd(g[..., None, None], x[..., None, None], h0=h0[..., None, None],
                                               cu_seqlens=cu, reverse=reverse)
        assert np.array_equal(hm[..., 0, 0], hs)


@pytest.mark.parametrize("kv", [(2, 1), (4, 4), (2, 3), (16, 16), (8, 2), (1, 16), (16, 1)])
def test_matrix_brute_force_products(oracle_lib, kv):
    """h_t = (A_t...A_s) h0 + sum_u (A_t...A_{u+1}) B_u with numpy matmul, every segment."""
    k, v = kv
    r = _rng(15 + k + 100 * v)
    T = 20
    A = r.standard_normal((2, T, k, k)) * (0.6 if k <= 4 else 1.2 / np.sqrt(k))
    B = r.standard_normal((2, T, k, v))
    cu = np.array([0, 7, 20], dtype=np.int32)
    h0 = r.standard_normal((2, 2, k, v))
    for reverse in (False, True):
        h = oracle_lib.matrix_affine_scan_fwd(A, B, h0=h0, cu_seqlens=cu, reverse=reverse)
        for row in range(2):
            for s in range(2):
                idx = list(range(cu[s], cu[s + 1]))
                if reverse:
                    idx = idx[::-1]
                for j, t in enumerate(idx):
                    M = np.eye(k)
                    acc = np.zeros((k, v))
                    for i in range(j, -1, -1):
                        acc = acc + M @ B[row, idx[i]]
                        M = M @ A[row, idx[i]]
                    acc = acc + M @ h0[s, row]
                    np.testing.assert_allclose(h[row, t], acc, rtol=1e-12, atol=1e-12)


def test_matrix_rotation_is_complex_scan(oracle_lib):
    """k=2, v=1 with A = r Rot(theta) is multiplication by r e^{i theta}; its adjoint
    (A^T) is multiplication by r e^{-i theta}."""
    d = gen.matrix_rot2(B=1, N=3, T=400)
    A, B, dy = (d[n].astype(np.float64) for n in ("A", "B", "dy"))
    h = oracle_lib.matrix_affine_scan_fwd(A, B)
    a = A[..., 0, 0] + 1j * A[..., 1, 0]
    b = B[..., 0, 0] + 1j * B[..., 1, 0]
    z = np.zeros_like(b)
    st = np.zeros(b.shape[0], dtype=complex)
    for t in range(b.shape[1]):
        st = a[:, t] * st + b[:, t]
        z[:, t] = st
    np.testing.assert_allclose(h[..., 0, 0], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h[..., 1, 0], z.imag, rtol=1e-12, atol=1e-12)
    dA, dB, _ = oracle_lib.matrix_affine_scan_bwd(A, h, dy)
    w = dy[..., 0, 0] + 1j * dy[..., 1, 0]
    lam = np.zeros_like(w)
    st = np.zeros(w.shape[0], dtype=complex)
    for t in range(w.shape[1] - 1, -1, -1):
        nxt = np.conj(a[:, t + 1]) if t + 1 < w.shape[1] else 0.0
        st = w[:, t] + nxt * st
        lam[:, t] = st
    np.testing.assert_allclose(dB[..., 0, 0], lam.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB[..., 1, 0], lam.imag, rtol=1e-12, atol=1e-12)


def test_matrix_reset_gives_B(oracle_lib):
    d = gen.matrix_orth4(B=1, N=2, T=64, p_reset=0.1)
    A, B = d["A"].astype(np.float64), d["B"].astype(np.float64)
    h = oracle_lib.matrix_affine_scan_fwd(A, B, h0=np.ones((1, 2, 4, 4)))
    assert d["reset"].any()
    assert np.array_equal(h[d["reset"]], B[d["reset"]])


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("kv", [(2, 1), (4, 4), (16, 16), (8, 2), (1, 4)])
def test_matrix_adjoint_dot_product(oracle_lib, kv, reverse):
    k, v = kv
    r = _rng(20 + k + 100 * v)
    T = 60
    A = r.standard_normal((3, T, k, k)) * (0.5 if k <= 4 else 1.0 / np.sqrt(k))
    B = r.standard_normal((3, T, k, v))
    cu = np.array([0, 13, 13, 60], dtype=np.int32)
    h0 = r.standard_normal((3, 3, k, v))
    Ad, Bd, h0d = r.standard_normal(A.shape), r.standard_normal(B.shape), r.standard_normal(h0.shape)
    dy = r.standard_normal(B.shape)
    h = oracle_lib.matrix_affine_scan_fwd(A, B, h0=h0, cu_seqlens=cu, reverse=reverse)
    hd = np.zeros_like(h)
    for s in range(3):
        idx = list(range(cu[s], cu[s + 1]))
        if reverse:
            idx = idx[::-1]
        st, std = h0[s].copy(), h0d[s].copy()
        for t in idx:
            std = Ad[:, t] @ st + A[:, t] @ std + Bd[:, t]
            st = A[:, t] @ st + B[:, t]
            hd[:, t] = std
    dA, dB, dh0 = oracle_lib.matrix_affine_scan_bwd(A, h, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    lhs = np.sum(dy * hd)
    rhs = np.sum(dA * Ad) + np.sum(dB * Bd) + np.sum(dh0 * h0d)
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


def test_matrix_block_diagonal_splits(oracle_lib):
    """A block-diagonal 16x16 transition (four 4x4 blocks) acting on a state
    whose rows split the same way is four independent 4x4 scans; v columns of
    the state are v independent scans with the same A (forward and adjoint)."""
    r = _rng(77)
    T = 40
    blocks = r.standard_normal((2, T, 4, 4, 4)) * 0.5  # [row, t, block, 4, 4]
    A = np.zeros((2, T, 16, 16))
    for b in range(4):
        A[:, :, 4 * b:4 * b + 4, 4 * b:4 * b + 4] = blocks[:, :, b]
    B = r.standard_normal((2, T, 16, 3))
    cu = np.array([0, 15, 40], dtype=np.int32)
    h0 = r.standard_normal((2, 2, 16, 3))
    dy = r.standard_normal(B.shape)
    for reverse in (False, True):
        h = oracle_lib.matrix_affine_scan_fwd(A, B, h0=h0, cu_seqlens=cu, reverse=reverse)
        dA, dB, dh0 = oracle_lib.matrix_affine_scan_bwd(A, h, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
        for b in range(4):
            sl = slice(4 * b, 4 * b + 4)
            hb = oracle_lib.matrix_affine_scan_fwd(blocks[:, :, b], B[:, :, sl], h0=h0[:, :, sl], cu_seqlens=cu,
                                                   reverse=reverse)
            np.testing.assert_allclose(h[:, :, sl], hb, rtol=1e-13, atol=1e-13)
            dAb, dBb, dh0b = oracle_lib.matrix_affine_scan_bwd(blocks[:, :, b], hb, dy[:, :, sl], h0=h0[:, :, sl],
                                                               cu_seqlens=cu, reverse=reverse)
            np.testing.assert_allclose(dA[:, :, sl, sl], dAb, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(dB[:, :, sl], dBb, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(dh0[:, :, sl], dh0b, rtol=1e-12, atol=1e-12)
        for c in range(3):
            hc = oracle_lib.matrix_affine_scan_fwd(A, B[..., c:c + 1], h0=h0[..., c:c + 1], cu_seqlens=cu, reverse=reverse)
            np.testing.assert_allclose(h[..., c:c + 1], hc, rtol=1e-13, atol=1e-13)


def test_matrix_finite_differences(oracle_lib):
    r = _rng(30)
    k, v, T = 2, 2, 12
    A = r.standard_normal((1, T, k, k)) * 0.7
    B = r.standard_normal((1, T, k, v))
    h0 = r.standard_normal((1, 1, k, v))
    dy = r.standard_normal(B.shape)
    L = lambda A_, B_, h0_: np.sum(dy * oracle_lib.matrix_affine_scan_fwd(A_, B_, h0=h0_))
    h = oracle_lib.matrix_affine_scan_fwd(A, B, h0=h0)
    dA, dB, dh0 = oracle_lib.matrix_affine_scan_bwd(A, h, dy, h0=h0)
    eps = 1e-6
    for (t, p, q) in [(0, 0, 1), (5, 1, 0), (11, 1, 1)]:
        P, M = A.copy(), A.copy()
        P[0, t, p, q] += eps
        M[0, t, p, q] -= eps
        fd = (L(P, B, h0) - L(M, B, h0)) / (2 * eps)
        assert abs(fd - dA[0, t, p, q]) < 1e-6 * max(1, abs(fd))
    P, M = h0.copy(), h0.copy()
    P[0, 0, 1, 0] += eps
    M[0, 0, 1, 0] -= eps
    fd = (L(A, B, P) - L(A, B, M)) / (2 * eps)
    assert abs(fd - dh0[0, 0, 1, 0]) < 1e-6 * max(1, abs(fd))


# ---------------------------------------------------------------------------
# a reset (zero transition) wipes out a non-finite prefix
# ("Our RG-LRU GPU audit", "Exact real chunk algebra": a reset is a_t = 0)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("reverse", [False, True])
def test_reset_clears_nonfinite_prefix(oracle_lib, reverse):
    """Constant gate a with one zero at p and NaN / +-Inf tokens before it: from
    p on the result is scipy.signal.lfilter of the tokens from p (a fresh start),
    and before p it is lfilter of the poisoned tokens (non-finite from the first
    poison on)."""
    o = oracle_lib
    T, p, a = 300, 170, 0.75
    rng = _rng(41 + reverse)
    x = rng.standard_normal(T)
    g = np.full(T, a)
    x[40], x[90], x[120] = np.nan, np.inf, -np.inf
    g[p] = 0.0
    if reverse:  # time runs backwards: flip the data so the same positions apply
        h = o.scan_fwd(g[::-1].copy(), x[::-1].copy(), reverse=True)[::-1]
    else:
        h = o.scan_fwd(g, x)
    after = scipy.signal.lfilter([1.0], [1.0, -a], x[p:])
    assert np.array_equal(h[p:], after)
    assert np.all(np.isnan(h[40:p]))
    np.testing.assert_allclose(h[:40], scipy.signal.lfilter([1.0], [1.0, -a], x[:40]), rtol=1e-13, atol=0)


def test_reset_at_sequence_start_ignores_nonfinite_h0(oracle_lib):
    """A zero gate on a sequence's first step drops h0, even a NaN or Inf h0:
    the a = 0 special case gives h = x exactly, dx = dy, dh0 = 0."""
    o = oracle_lib
    rng = _rng(43)
    x = rng.standard_normal((3, 50))
    dy = rng.standard_normal((3, 50))
    g = np.zeros((3, 50))
    h0 = np.array([np.nan, np.inf, -np.inf])
    for rev in (False, True):
        h = o.scan_fwd(g, x, h0=h0, reverse=rev)
        assert np.array_equal(h, x)
        dx, dg, dh0 = o.scan_bwd(g, h, dy, h0=h0, reverse=rev)
        assert np.array_equal(dx, dy)
        assert np.array_equal(dh0, np.zeros((1, 3)))
        # dg_t = lam_t * h_{t-1}: h0 enters only the sequence's first step
        first = 49 if rev else 0
        assert np.all(np.isnan(dg[:, first]) | np.isinf(dg[:, first]))
        rest = np.delete(dg, first, axis=1)
        assert np.all(np.isfinite(rest))


@pytest.mark.parametrize("reverse", [False, True])
def test_reset_stops_nonfinite_adjoint(oracle_lib, reverse):
    """Backward with a constant gate a and one zero gate at p (causal): a NaN
    gradient entering after p never reaches t < p, where lam is the reversed
    lfilter of dy (the adjoint recurrence lam_t = dy_t + a lam_{t+1}) over
    [0, p) alone."""
    o = oracle_lib
    T, p, a = 200, 120, 0.5
    rng = _rng(47 + reverse)
    x = rng.standard_normal(T)
    dy = rng.standard_normal(T)
    g = np.full(T, a)
    g[p] = 0.0
    dy[150] = np.nan
    if reverse:
        gg, xx, dd = g[::-1].copy(), x[::-1].copy(), dy[::-1].copy()
        h = o.scan_fwd(gg, xx, reverse=True)
        dx, dg, dh0 = o.scan_bwd(gg, h, dd, reverse=True)
        dx = dx[::-1]
    else:
        h = o.scan_fwd(g, x)
        dx, dg, dh0 = o.scan_bwd(g, h, dy)
    lam_before = scipy.signal.lfilter([1.0], [1.0, -a], dy[:p][::-1])[::-1]
    np.testing.assert_allclose(dx[:p], lam_before, rtol=1e-13, atol=1e-15)
    assert np.all(np.isnan(dx[p:151]))
    assert np.all(np.isfinite(dx[151:]))


def test_reset_equals_sequence_split_with_nonfinite_data(oracle_lib):
    """Inside one sequence, a zero gate at p gives, from p on, exactly what a
    sequence starting at p gives (h0 = 0); the two take different paths through
    the oracle (a gate value against a cu_seqlens boundary)."""
    o = oracle_lib
    rng = _rng(53)
    T, p = 400, 230
    g = rng.uniform(0.2, 1.0, (4, T))
    x = rng.standard_normal((4, T))
    dy = rng.standard_normal((4, T))
    x[:, 100] = np.nan
    x[1, 50] = np.inf
    g[:, p] = 0.0
    h_reset = o.scan_fwd(g, x)
    h_split = o.scan_fwd(g, x, cu_seqlens=[0, p, T])
    assert np.array_equal(h_reset[:, p:], h_split[:, p:])
    # the adjoint of the suffix agrees too, and the prefix's is NaN-free
    dy[:, 350] = np.nan
    dx_r, dg_r, _ = o.scan_bwd(g, h_reset, dy)
    dx_s, dg_s, _ = o.scan_bwd(g, h_split, dy, cu_seqlens=[0, p, T])
    assert np.array_equal(dx_r, dx_s, equal_nan=True)
    assert np.all(np.isfinite(dx_r[:, :p]))


def test_log_reset_drops_h0_and_prefix(oracle_lib):
    """log a = -inf on a sequence's first step drops log_h0 (h = e^{log b}
    exactly there), and the matching linear adjoint has no dlog_h0."""
    o = oracle_lib
    rng = _rng(59)
    la = -np.log1p(np.exp(rng.standard_normal((2, 60))))
    lb = rng.standard_normal((2, 60))
    la[:, 0] = -np.inf
    lh0 = np.array([3.0, -2.0])
    h = o.scan_log_fwd(la, lb, log_h0=lh0)
    h_nol = o.scan_log_fwd(la, lb)
    assert np.array_equal(h, h_nol)
    assert np.array_equal(h[:, 0], np.exp(lb[:, 0]))
    dy = rng.standard_normal((2, 60))
    _, _, dlh0 = o.scan_log_bwd(la, lb, h, dy, log_h0=lh0)
    assert np.array_equal(dlh0, np.zeros((1, 2)))
    # a NaN or Inf log_h0 is dropped the same way, value and gradient
    bad = np.array([np.nan, np.inf])
    assert np.array_equal(o.scan_log_fwd(la, lb, log_h0=bad), h_nol)
    _, _, dlh0 = o.scan_log_bwd(la, lb, h, dy, log_h0=bad)
    assert np.array_equal(dlh0, np.zeros((1, 2)))


def test_matrix_reset_clears_nan_prefix(oracle_lib):
    """k = 2 rotations r Rot(theta) with NaN injections and an all-zero A at p:
    from p on the state equals the complex scan z_t = r e^{i theta} z_{t-1} + B
    of the steps from p (scipy.signal.lfilter with a complex coefficient), and
    the adjoint's lam for t < p equals the reversed lfilter with the conjugate
    coefficient."""
    o = oracle_lib
    T, p = 160, 90
    rng = _rng(61)
    r, th = 0.8, 0.7
    A = np.tile(r * np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]]), (T, 1, 1))
    A[p] = 0.0
    B = rng.standard_normal((T, 2, 1))
    B[30, 0, 0] = np.nan
    h = o.matrix_affine_scan_fwd(A[None], B[None])[0]
    z = scipy.signal.lfilter([1.0], [1.0, -r * complex(math.cos(th), math.sin(th))], B[p:, 0, 0] + 1j * B[p:, 1, 0])
    np.testing.assert_allclose(h[p:, 0, 0], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h[p:, 1, 0], z.imag, rtol=1e-12, atol=1e-12)
    assert np.isnan(h[30, 0, 0]) and np.isfinite(h[30, 1, 0])  # the NaN enters one entry
    assert np.all(np.isnan(h[31:p]))  # and the next rotation spreads it over the state
    dy = rng.standard_normal((T, 2, 1))
    dy[120, 1, 0] = np.nan
    dA, dB, dh0 = o.matrix_affine_scan_bwd(A[None], h[None], dy[None])
    lam = scipy.signal.lfilter([1.0], [1.0, -r * complex(math.cos(th), -math.sin(th))],
                               (dy[:p, 0, 0] + 1j * dy[:p, 1, 0])[::-1])[::-1]
    np.testing.assert_allclose(dB[0, :p, 0, 0], lam.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB[0, :p, 1, 0], lam.imag, rtol=1e-12, atol=1e-12)
    assert np.all(np.isfinite(dh0))
