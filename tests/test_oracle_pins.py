"""Pins for the fp64 oracle, each against something other than the oracle itself.

Sources: the KATA page ("Kernelized Linear Attention: Breaking the Capacity
Wall with Symmetric Cones") -- Eq. 2 (normalised readout), Sec. 2.2
Proposition 1 (convex output gate), Sec. 3.1 (rank-one lift squares the inner
product), Eq. 8 and Sec. 4.1 (packed widths), Sec. 4.1 Eqs. 17-20 (chunkwise
form), Sec. 2.1 Assumption 2 (isometric invariance), App. A (antipodal
identification under the PSD lift); the hebbian-MLP page ("MLPs are Hebbians",
App. B.2.2, Lemma B.2: the bilinear random-feature sketch is unbiased for the
exact quadratic kernel <x, z>^2).  Worked values live in
tests/golden/handworked.json with their derivations.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kata_oracle as orc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "handworked.json")))


def _frac_arr(rows):
    return [[Fraction(a, b) for (a, b) in r] for r in rows]


def _f64(rows):
    return np.array([[float(Fraction(a, b)) for (a, b) in r] for r in rows])


def _unit(g, shape):
    x = g.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ------------------------------------------------------------------ feature map

def test_packed_width_matches_page():
    pw = GOLDEN["packed_width"]
    for d, D in zip(pw["d"], pw["D"]):
        assert orc.feature_dim(d) == D
        assert len(orc.feature_pairs(d)) == D
        assert orc.feature_map(np.ones(d)).shape == (D,)
    assert 64 * 64 == pw["direct_d64"]


def test_packing_order_d3_and_index_formula():
    assert [list(p) for p in orc.feature_pairs(3)] == GOLDEN["feature_order_d3"]["pairs"]
    for d in (1, 2, 5, 16, 32):
        for f, (i, j) in enumerate(orc.feature_pairs(d)):
            assert i <= j
            assert f == i * d - i * (i - 1) // 2 + (j - i)


def test_rank_one_identity_exact_rationals():
    # sum_f w_f (x_i x_j)(y_i y_j) == (x . y)^2 exactly, w from the oracle.
    g = np.random.Generator(np.random.PCG64(11))
    for d in (1, 2, 3, 5, 8):
        pairs = orc.feature_pairs(d)
        w = [Fraction(int(a)) for a in orc.feature_weights(d)]
        for _ in range(5):
            x = [Fraction(int(a), int(b)) for a, b in zip(g.integers(-9, 10, d), g.integers(1, 8, d))]
            y = [Fraction(int(a), int(b)) for a, b in zip(g.integers(-9, 10, d), g.integers(1, 8, d))]
            lhs = sum(wf * x[i] * x[j] * y[i] * y[j] for wf, (i, j) in zip(w, pairs))
            rhs = sum(a * b for a, b in zip(x, y)) ** 2
            assert lhs == rhs


def test_feature_map_worked_example():
    ex = GOLDEN["feature_map_example"]
    phi = orc.feature_map(np.array(ex["x"]))
    want = np.array(ex["phi_rational_part"]) * np.sqrt(2.0) ** np.array(ex["phi_sqrt2_power"])
    np.testing.assert_allclose(phi, want, rtol=0, atol=1e-15)
    e0 = orc.feature_map(np.array([1.0, 0.0]))
    assert abs(phi @ e0 - ex["dot_with_e0"]) < 1e-15


@pytest.mark.parametrize("d", [16, 32])
def test_feature_map_dot_fp64_within_ulps(d):
    g = np.random.Generator(np.random.PCG64(d))
    x = _unit(g, (200, d))
    y = _unit(g, (200, d))
    px, py = orc.feature_map(x), orc.feature_map(y)
    lhs = np.sum(px * py, axis=1)
    rhs = np.sum(x * y, axis=1) ** 2
    scale = np.sum(np.abs(px * py), axis=1)
    assert np.all(np.abs(lhs - rhs) <= 8 * np.finfo(np.float64).eps * scale)


def test_feature_map_matches_bilinear_sketch_mean():
    # hebbian-MLP page, Lemma B.2: E[(a.x)(a.z)(b.x)(b.z)] = <x,z>^2 for iid
    # Gaussian a, b.  The Monte-Carlo mean must agree with phi(x).phi(z)
    # within a few standard errors; a wrong weight or index moves it by O(1).
    g = np.random.Generator(np.random.PCG64(5))
    d, m = 6, 400_000
    for _ in range(3):
        x, z = _unit(g, (2, d))
        A = g.standard_normal((m, d))
        G = g.standard_normal((m, d))
        samples = (A @ x) * (A @ z) * (G @ x) * (G @ z)
        mean, se = samples.mean(), samples.std() / math.sqrt(m)
        exact = orc.feature_map(x) @ orc.feature_map(z)
        assert abs(mean - exact) < 5 * se + 1e-12
    # and a pair with known kernel: x = z gives 1; orthogonal gives 0
    x = np.zeros(d); x[0] = 1
    y = np.zeros(d); y[1] = 1
    assert orc.feature_map(x) @ orc.feature_map(x) == pytest.approx(1.0, abs=1e-15)
    assert orc.feature_map(x) @ orc.feature_map(y) == pytest.approx(0.0, abs=1e-15)


# ------------------------------------------------------------------ worked values

def _example(name):
    ex = GOLDEN[name]
    q = _f64(ex["q"])[None, None]
    k = _f64(ex["k"])[None, None]
    v = _f64(ex["v"])[None, None]
    return ex, q, k, v


def test_three_token_example_quadratic_and_chunked():
    ex, q, k, v = _example("three_token_example")
    want = _f64(ex["out"])
    got = orc.forward_quadratic(q, k, v, eps=0.0)[0, 0]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)
    for C in (1, 2, 3, 8):
        got = orc.forward_chunked(q, k, v, C, eps=0.0)[0, 0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_three_token_example_with_eps():
    ex, q, k, v = _example("three_token_example")
    eps = 0.125
    num = _f64([[tuple(x) for x in r] for r in ex["num"]])
    den = np.array([float(Fraction(a, b)) for a, b in ex["den"]])
    want = num / (den + eps)[:, None]
    got = orc.forward_quadratic(q, k, v, eps=eps)[0, 0]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)
    got = orc.forward_chunked(q, k, v, 2, eps=eps)[0, 0]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_gate_branch_returns_current_value():
    ex, q, k, v = _example("gate_branch_example")
    want = _f64(ex["out"])
    got = orc.forward_quadratic(q, k, v, eps=0.0)[0, 0]
    np.testing.assert_allclose(got, want, rtol=4e-16, atol=0)
    alpha, beta, _, o = orc.convex_gate(q[0, 0], k[0, 0], v[0, 0])
    assert alpha[1] == 0.0 and beta[1] == 1.0
    np.testing.assert_array_equal(o, want)


def test_bruteforce_exact_rationals_tiny():
    # Exact-arithmetic brute force of Eq. 2 with the squared kernel on tiny
    # random rational inputs, T <= 8.
    g = np.random.Generator(np.random.PCG64(3))
    for T, d, dv in ((1, 2, 1), (5, 3, 2), (8, 2, 3)):
        q = [[Fraction(int(a), 7) for a in g.integers(-7, 8, d)] for _ in range(T)]
        k = [[Fraction(int(a), 5) for a in g.integers(-5, 6, d)] for _ in range(T)]
        v = [[Fraction(int(a), 3) for a in g.integers(-9, 10, dv)] for _ in range(T)]
        k[0][0] = Fraction(1)  # keep the first key non-zero
        q[0][0] = Fraction(1)
        eps = Fraction(1, 1000)
        want = []
        for t in range(T):
            c = [sum(a * b for a, b in zip(q[t], k[s])) ** 2 for s in range(t + 1)]
            den = sum(c) + eps
            want.append([sum(c[s] * v[s][j] for s in range(t + 1)) / den for j in range(dv)])
        f = lambda M: np.array([[float(x) for x in r] for r in M])[None, None]
        got = orc.forward_quadratic(f(q), f(k), f(v), eps=float(eps))[0, 0]
        np.testing.assert_allclose(got, f(want)[0, 0], rtol=1e-13, atol=1e-15)


def test_forward_rows_matches_worked_values_and_full_form():
    ex, q, k, v = _example("three_token_example")
    got = orc.forward_rows(q[0, 0], k[0, 0], v[0, 0], [2, 0], eps=0.0)
    np.testing.assert_allclose(got, _f64(ex["out"])[[2, 0]], rtol=0, atol=1e-14)
    g = np.random.Generator(np.random.PCG64(9))
    T = 300
    q, k = _unit(g, (T, 16)), _unit(g, (T, 16))
    v = g.standard_normal((T, 8))
    rows = [0, 1, 63, 64, 150, 299]
    full = orc.forward_quadratic(q[None], k[None], v[None], eps=1e-6)[0]
    np.testing.assert_allclose(orc.forward_rows(q, k, v, rows, 1e-6), full[rows], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ chunked == quadratic

@pytest.mark.parametrize("T", [1, 2, 3, 257])
@pytest.mark.parametrize("C", [1, 3, 32, None])
def test_chunked_equals_quadratic(T, C):
    g = np.random.Generator(np.random.PCG64(T * 100 + (C or 0)))
    q = _unit(g, (2, 1, T, 4))
    k = _unit(g, (2, 1, T, 4))
    v = g.standard_normal((2, 1, T, 3))
    a = orc.forward_quadratic(q, k, v, eps=1e-6, block=7)
    b = orc.forward_chunked(q, k, v, C or T, eps=1e-6)
    np.testing.assert_allclose(b, a, rtol=1e-10, atol=1e-12)


def test_chunk_one_is_the_recurrence():
    # C = 1 leaves no intra-chunk work except the diagonal: it is the additive
    # recurrence read after each update, which pins the exclusive prefix.
    g = np.random.Generator(np.random.PCG64(8))
    T, d, dv = 20, 3, 2
    q, k = _unit(g, (T, d)), _unit(g, (T, d))
    v = g.standard_normal((T, dv))
    S = np.zeros((orc.feature_dim(d), dv))
    z = np.zeros(orc.feature_dim(d))
    rec = []
    for t in range(T):
        S, z, o = orc.decode_step(S, z, q[t], k[t], v[t], eps=1e-6)
        rec.append(o)
    b = orc.forward_chunked(q[None, None], k[None, None], v[None, None], 1, eps=1e-6)[0, 0]
    np.testing.assert_allclose(b, np.array(rec), rtol=1e-11, atol=1e-13)


# ------------------------------------------------------------------ Proposition 1

def test_convex_gate_decomposition_and_bounds():
    g = np.random.Generator(np.random.PCG64(21))
    T, d, dv = 64, 4, 5
    q, k = _unit(g, (T, d)), _unit(g, (T, d))
    v = g.standard_normal((T, dv))
    alpha, beta, zbar, o = orc.convex_gate(q, k, v)
    assert np.all(alpha >= 0) and np.all(beta >= 0)
    np.testing.assert_allclose(alpha + beta, 1.0, rtol=0, atol=1e-14)
    ref = orc.forward_quadratic(q[None], k[None], v[None], eps=0.0)[0]
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    # convex interpolation: each coordinate within the visible min/max (eps = 0)
    for t in range(T):
        lo, hi = v[: t + 1].min(axis=0), v[: t + 1].max(axis=0)
        assert np.all(ref[t] >= lo - 1e-12) and np.all(ref[t] <= hi + 1e-12)


def test_convex_bound_with_eps_after_rescale():
    # With eps > 0, o_t = D_t/(D_t + eps) * (convex combination), so
    # (D_t + eps)/D_t * o_t lies within the visible min/max.
    g = np.random.Generator(np.random.PCG64(22))
    T, d, dv, eps = 50, 16, 4, 1e-6
    q, k = _unit(g, (T, d)), _unit(g, (T, d))
    v = g.standard_normal((T, dv))
    o = orc.forward_quadratic(q[None], k[None], v[None], eps=eps)[0]
    c = (q @ k.T) ** 2 * np.tril(np.ones((T, T)))
    Dt = c.sum(axis=1)
    resc = o * ((Dt + eps) / Dt)[:, None]
    for t in range(T):
        lo, hi = v[: t + 1].min(axis=0), v[: t + 1].max(axis=0)
        tol = 1e-12 * (1 + np.abs(v[: t + 1]).max())
        assert np.all(resc[t] >= lo - tol) and np.all(resc[t] <= hi + tol)
        # and the unscaled read shrinks towards 0 only
        assert np.all(o[t] >= np.minimum(lo, 0) - tol) and np.all(o[t] <= np.maximum(hi, 0) + tol)


# ------------------------------------------------------------------ special cases

def test_d1_is_k_squared_weighted_running_mean():
    g = np.random.Generator(np.random.PCG64(31))
    T = 40
    q = g.choice([-1.0, 1.0], size=(T, 1)) * g.uniform(0.5, 2.0, (T, 1))
    k = g.uniform(-2, 2, (T, 1))
    v = g.standard_normal((T, 3))
    o = orc.forward_quadratic(q[None], k[None], v[None], eps=0.0)[0]
    w = k[:, 0] ** 2
    want = np.cumsum(w[:, None] * v, axis=0) / np.cumsum(w)[:, None]
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-13)


def test_identical_keys_give_running_mean():
    g = np.random.Generator(np.random.PCG64(32))
    T, d, eps = 30, 5, 1e-3
    key = _unit(g, (d,))
    q = _unit(g, (T, d))
    k = np.tile(key, (T, 1))
    v = g.standard_normal((T, 2))
    o = orc.forward_quadratic(q[None], k[None], v[None], eps=eps)[0]
    n = np.arange(1, T + 1)
    qk2 = (q @ key) ** 2
    Dt = n * qk2
    want = np.cumsum(v, axis=0) / n[:, None] * (Dt / (Dt + eps))[:, None]
    np.testing.assert_allclose(o, want, rtol=1e-11, atol=1e-13)


def test_constant_values_are_reproduced():
    g = np.random.Generator(np.random.PCG64(33))
    T, d = 64, 8
    q, k = _unit(g, (T, d)), _unit(g, (T, d))
    cval = np.array([2.5, -1.25, 0.0])
    v = np.tile(cval, (T, 1))
    o = orc.forward_quadratic(q[None], k[None], v[None], eps=0.0)[0]
    np.testing.assert_allclose(o, np.tile(cval, (T, 1)), rtol=1e-13, atol=1e-14)
    o2 = orc.forward_chunked(q[None], k[None], v[None], 16, eps=0.0)[0]
    np.testing.assert_allclose(o2, np.tile(cval, (T, 1)), rtol=1e-12, atol=1e-13)


def test_orthonormal_basis_keys():
    d, dv, eps = 6, 3, 1e-6
    g = np.random.Generator(np.random.PCG64(34))
    k = np.eye(d)
    v = g.standard_normal((d, dv))
    for j in range(d):
        q = np.tile(np.eye(d)[j], (d, 1))
        o = orc.forward_quadratic(q[None], k[None], v[None], eps=eps)[0]
        for t in range(d):
            want = v[j] / (1 + eps) if j <= t else np.zeros(dv)
            np.testing.assert_allclose(o[t], want, rtol=1e-15, atol=0)


# ------------------------------------------------------------------ invariances

def test_invariances():
    g = np.random.Generator(np.random.PCG64(41))
    T, d, dv, eps = 48, 6, 4, 1e-6
    q, k = _unit(g, (T, d)), _unit(g, (T, d))
    v = g.standard_normal((T, dv))
    f = lambda q_, k_, v_: orc.forward_quadratic(q_[None], k_[None], v_[None], eps=eps)[0]
    base = f(q, k, v)
    # antipodal identification: flipping signs of any q_t or k_s
    sq = g.choice([-1.0, 1.0], size=(T, 1))
    sk = g.choice([-1.0, 1.0], size=(T, 1))
    np.testing.assert_allclose(f(q * sq, k * sk, v), base, rtol=1e-12, atol=1e-13)
    # common rotation
    U, _ = np.linalg.qr(g.standard_normal((d, d)))
    np.testing.assert_allclose(f(q @ U.T, k @ U.T, v), base, rtol=1e-10, atol=1e-12)
    # permuting the (k, v) pairs leaves the last read (all visible) unchanged
    perm = g.permutation(T)
    last = f(q, k[perm], v[perm])[-1]
    np.testing.assert_allclose(last, base[-1], rtol=1e-12, atol=1e-13)
    # linearity in v
    v2 = g.standard_normal((T, dv))
    np.testing.assert_allclose(f(q, k, v + 3.0 * v2), base + 3.0 * f(q, k, v2), rtol=1e-11, atol=1e-12)
    # a non-causal dependence would fail this: future tokens do not move o_t
    k3, v3 = k.copy(), v.copy()
    k3[T // 2:] = _unit(g, (T - T // 2, d))
    v3[T // 2:] = g.standard_normal((T - T // 2, dv))
    np.testing.assert_array_equal(f(q, k3, v3)[: T // 2], base[: T // 2])


# ------------------------------------------------------------------ decode

def test_decode_state_closed_form_and_continuation():
    g = np.random.Generator(np.random.PCG64(51))
    T0, n, d, dv, eps = 40, 12, 4, 3, 1e-6
    q, k = _unit(g, (T0 + n, d)), _unit(g, (T0 + n, d))
    v = g.standard_normal((T0 + n, dv))
    S, z = orc.decode_state(k[:T0], v[:T0])
    # state after a history reads out the same as the quadratic form does
    pq = orc.feature_map(q[T0 - 1])
    o_state = (pq @ S) / (pq @ z + eps)
    full = orc.forward_quadratic(q[None], k[None], v[None], eps=eps)[0]
    np.testing.assert_allclose(o_state, full[T0 - 1], rtol=1e-11, atol=1e-13)
    outs = []
    for t in range(T0, T0 + n):
        S, z, o = orc.decode_step(S, z, q[t], k[t], v[t], eps)
        outs.append(o)
    np.testing.assert_allclose(np.array(outs), full[T0:], rtol=1e-11, atol=1e-13)
    S_all, z_all = orc.decode_state(k, v)
    np.testing.assert_allclose(S, S_all, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, z_all, rtol=1e-12, atol=1e-12)
