"""Pins for the oracle's variants of the read, each against something other
than the oracle itself: the KATA-Mg block maps (KATA page, Sec. 4.1, Table 2
state sizes), the linear cone features KATA-Orthant and KATA-Lorentz (App. F.4,
Sec. 2.3) and the gated recurrence GatedKATA (App. F.4, unrolled in Sec. 5.2).
Worked values are hand-derived in tests/golden/handworked.json.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kata_oracle as orc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "handworked.json")))


def _f64(x):
    """Nested [num, den] pairs -> fp64 array (the last axis holds the pairs)."""
    a = np.asarray(x, dtype=np.int64)
    return a[..., 0].astype(np.float64) / a[..., 1]


def _unit(g, shape):
    x = g.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rotation(g, n):
    Q, R = np.linalg.qr(g.standard_normal((n, n)))
    return Q * np.sign(np.diag(R))


# ------------------------------------------------------------------ block maps

def test_block_state_sizes_match_table2():
    ex = GOLDEN["block_state_sizes"]
    for g, state in zip(ex["g"], ex["state"]):
        D = orc.feature_map_blocks(np.ones(ex["d"]), g).shape[-1]
        assert D * ex["dv"] == state


@pytest.mark.parametrize("name", ["block_map_example_m1", "block_map_example_m2"])
def test_block_map_worked_examples(name):
    ex = GOLDEN[name]
    q, k, v, g = _f64(ex["q"]), _f64(ex["k"]), _f64(ex["v"]), ex["g"]
    want, want_full = _f64(ex["out"]), _f64(ex["out_full_map"])
    np.testing.assert_allclose(orc.forward_quadratic(q, k, v, 0.0, g=g), want, rtol=0, atol=1e-15)
    for C in (1, 2, len(q)):
        np.testing.assert_allclose(orc.forward_chunked(q, k, v, C, 0.0, g=g), want, rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.forward_rows(q, k, v, range(len(q)), 0.0, g=g), want, rtol=0,
                               atol=1e-15)
    # the full map differs on these inputs, so the block structure is what is pinned
    np.testing.assert_allclose(orc.forward_quadratic(q, k, v, 0.0), want_full, rtol=0, atol=1e-15)


@pytest.mark.parametrize("d,g", [(4, 2), (8, 4), (64, 2), (64, 4), (6, 3)])
def test_block_features_exact_identity(d, g):
    # sum over block features of w_f x_i x_j y_i y_j == sum_a (x_a . y_a)^2, exactly,
    # with the block layout of feature_map_blocks read back from its own output
    rng = np.random.Generator(np.random.PCG64(d * 10 + g))
    x = [Fraction(int(a), 7) for a in rng.integers(-9, 10, d)]
    y = [Fraction(int(a), 5) for a in rng.integers(-9, 10, d)]
    m = d // g
    pairs = orc.feature_pairs(m)
    lhs = Fraction(0)
    for a in range(g):
        for (i, j) in pairs:
            w = 1 if i == j else 2
            lhs += w * x[a * m + i] * x[a * m + j] * y[a * m + i] * y[a * m + j]
    rhs = sum(sum(x[a * m + i] * y[a * m + i] for i in range(m)) ** 2 for a in range(g))
    assert lhs == rhs
    # and the packed fp64 vectors realise it
    xf = np.array([float(a) for a in x])
    yf = np.array([float(a) for a in y])
    dot = orc.feature_map_blocks(xf, g) @ orc.feature_map_blocks(yf, g)
    assert abs(dot - float(rhs)) <= 1e-13 * max(1.0, abs(float(rhs)))
    # block a's coordinates are the packed lift of x_a
    pb = orc.feature_map_blocks(xf, g)
    D = m * (m + 1) // 2
    for a in range(g):
        np.testing.assert_array_equal(pb[a * D:(a + 1) * D], orc.feature_map(xf[a * m:(a + 1) * m]))


def test_block_map_blockwise_rotation_invariance():
    # psi_Mg is invariant under a separate rotation of each block (applied to q
    # and k alike), but not under a rotation that mixes blocks
    rng = np.random.Generator(np.random.PCG64(5))
    T, d, g, dv = 40, 8, 2, 3
    q, k, v = _unit(rng, (T, d)), _unit(rng, (T, d)), rng.standard_normal((T, dv))
    base = orc.forward_quadratic(q, k, v, 1e-6, g=g)
    U = np.zeros((d, d))
    U[:4, :4] = _rotation(rng, 4)
    U[4:, 4:] = _rotation(rng, 4)
    np.testing.assert_allclose(orc.forward_quadratic(q @ U, k @ U, v, 1e-6, g=g), base, atol=1e-11)
    R = _rotation(rng, d)
    assert np.abs(orc.forward_quadratic(q @ R, k @ R, v, 1e-6, g=g) - base).max() > 1e-3
    # swapping the blocks of both q and k leaves the read; swapping only k's does not
    perm = np.r_[4:8, 0:4]
    np.testing.assert_allclose(orc.forward_quadratic(q[:, perm], k[:, perm], v, 1e-6, g=g), base,
                               atol=1e-13)
    assert np.abs(orc.forward_quadratic(q, k[:, perm], v, 1e-6, g=g) - base).max() > 1e-3


def test_single_block_reduces_to_full_map_of_its_width():
    rng = np.random.Generator(np.random.PCG64(6))
    T, m, dv = 33, 4, 2
    qa, ka, v = _unit(rng, (T, m)), _unit(rng, (T, m)), rng.standard_normal((T, dv))
    q = np.zeros((T, 3 * m))
    k = np.zeros((T, 3 * m))
    q[:, m:2 * m] = qa
    k[:, m:2 * m] = ka
    np.testing.assert_allclose(orc.forward_quadratic(q, k, v, 1e-6, g=3),
                               orc.forward_quadratic(qa, ka, v, 1e-6), atol=1e-14)


@pytest.mark.parametrize("T", [1, 2, 37, 130])
@pytest.mark.parametrize("g", [2, 4])
def test_block_chunked_equals_quadratic(T, g):
    rng = np.random.Generator(np.random.PCG64(T + g))
    q, k, v = _unit(rng, (2, T, 16)), _unit(rng, (2, T, 16)), rng.standard_normal((2, T, 3))
    want = orc.forward_quadratic(q, k, v, 1e-6, g=g)
    for C in (1, 3, 32, T):
        np.testing.assert_allclose(orc.forward_chunked(q, k, v, C, 1e-6, g=g), want, rtol=1e-12,
                                   atol=1e-13)


def test_block_constant_values_closed_form():
    rng = np.random.Generator(np.random.PCG64(8))
    T, d, g = 50, 8, 4
    q, k = _unit(rng, (T, d)), _unit(rng, (T, d))
    v = np.full((T, 2), -1.75)
    o = orc.forward_quadratic(q, k, v, 0.0, g=g)
    np.testing.assert_allclose(o, v, rtol=1e-14)


# ------------------------------------------------------------------ linear cone features

def test_orthant_worked_example():
    ex = GOLDEN["orthant_example"]
    q, k, v = _f64(ex["q"]), _f64(ex["k"]), _f64(ex["v"])
    shift = ex["shift"][0] / ex["shift"][1]
    want = _f64(ex["out"])
    np.testing.assert_allclose(orc.forward_linear_quadratic(q, k, v, "orthant", 0.0, shift), want,
                               atol=1e-15)
    for C in (1, 2):
        np.testing.assert_allclose(orc.forward_linear_chunked(q, k, v, C, "orthant", 0.0, shift), want,
                                   atol=1e-15)


def test_lorentz_worked_example():
    ex = GOLDEN["lorentz_example"]
    q, k, v = _f64(ex["q"]), _f64(ex["k"]), _f64(ex["v"])
    np.testing.assert_array_equal(orc.feature_lorentz(q), _f64(ex["psi_q"]))
    np.testing.assert_array_equal(orc.feature_lorentz(k), _f64(ex["psi_k"]))
    want = _f64(ex["out"])
    np.testing.assert_allclose(orc.forward_linear_quadratic(q, k, v, "lorentz", 0.0), want, atol=1e-15)
    for C in (1, 2):
        np.testing.assert_allclose(orc.forward_linear_chunked(q, k, v, C, "lorentz", 0.0), want,
                                   atol=1e-15)


def test_cone_membership_and_nonnegative_scores():
    rng = np.random.Generator(np.random.PCG64(9))
    x = rng.standard_normal((300, 16)) * 3
    po = orc.feature_orthant(x, 1e-6)
    assert (po >= 1e-6).all()
    np.testing.assert_array_equal(orc.feature_orthant(np.array([-1.0, 2.0, 0.0]), 0.5), [0.5, 2.5, 0.5])
    pl = orc.feature_lorentz(x)
    assert (pl[:, -1] >= np.linalg.norm(pl[:, :-1], axis=1) * (1 - 1e-15)).all()
    assert ((pl @ pl.T) >= -1e-12).all()
    assert ((po @ po.T) > 0).all()


@pytest.mark.parametrize("feature", ["orthant", "lorentz"])
@pytest.mark.parametrize("T", [1, 5, 97])
def test_linear_chunked_equals_quadratic(feature, T):
    rng = np.random.Generator(np.random.PCG64(T))
    q, k, v = _unit(rng, (2, T, 8)), _unit(rng, (2, T, 8)), rng.standard_normal((2, T, 3))
    want = orc.forward_linear_quadratic(q, k, v, feature, 1e-6)
    for C in (1, 3, 32, T):
        np.testing.assert_allclose(orc.forward_linear_chunked(q, k, v, C, feature, 1e-6), want,
                                   rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("feature", ["orthant", "lorentz"])
def test_linear_rows_match_the_full_form(feature):
    rng = np.random.Generator(np.random.PCG64(20))
    T = 70
    q, k, v = _unit(rng, (T, 8)), _unit(rng, (T, 8)), rng.standard_normal((T, 3))
    rows = [0, 5, 31, 69]
    np.testing.assert_allclose(orc.forward_linear_rows(q, k, v, rows, feature, 1e-6),
                               orc.forward_linear_quadratic(q, k, v, feature, 1e-6)[rows], rtol=1e-13,
                               atol=1e-15)


@pytest.mark.parametrize("feature", ["orthant", "lorentz"])
def test_linear_reads_are_convex_combinations(feature):
    # cone features give nonnegative scores, so (D+eps)/D o_t lies inside the visible v's range
    rng = np.random.Generator(np.random.PCG64(12))
    T, d = 60, 8
    q, k, v = _unit(rng, (T, d)), _unit(rng, (T, d)), rng.standard_normal((T, 2))
    eps = 1e-6
    o = orc.forward_linear_quadratic(q, k, v, feature, eps)
    psi = orc.linear_feature(feature)
    c = np.tril(psi(q) @ psi(k).T)
    D = c.sum(axis=1)
    ok = D > 1e-9
    scaled = o[ok] * ((D[ok] + eps) / D[ok])[:, None]
    lo = np.minimum.accumulate(v, axis=0)[ok]
    hi = np.maximum.accumulate(v, axis=0)[ok]
    assert (scaled >= lo - 1e-12).all() and (scaled <= hi + 1e-12).all()


def test_orthant_basis_keys_closed_form():
    # shift 0 and basis keys e_s, queries e_j: c_{t,s} = [s == j], so o_t = v_j/(1+eps) once j <= t
    d, dv, eps = 6, 2, 1e-3
    rng = np.random.Generator(np.random.PCG64(13))
    k = np.eye(d)
    v = rng.standard_normal((d, dv))
    js = rng.integers(0, d, d)
    q = np.eye(d)[js]
    o = orc.forward_linear_quadratic(q, k, v, "orthant", eps, shift=0.0)
    for t in range(d):
        want = v[js[t]] / (1 + eps) if js[t] <= t else np.zeros(dv)
        np.testing.assert_allclose(o[t], want, atol=1e-15)


def test_lorentz_invariant_under_rotation_of_y():
    # psi_L(x) keeps y and its norm, so rotating y (not s) in q and k leaves the read
    rng = np.random.Generator(np.random.PCG64(14))
    T, d = 45, 8
    q, k, v = _unit(rng, (T, d)), _unit(rng, (T, d)), rng.standard_normal((T, 3))
    base = orc.forward_linear_quadratic(q, k, v, "lorentz", 1e-6)
    U = np.eye(d)
    U[:-1, :-1] = _rotation(rng, d - 1)
    np.testing.assert_allclose(orc.forward_linear_quadratic(q @ U, k @ U, v, "lorentz", 1e-6), base,
                               atol=1e-12)
    R = _rotation(rng, d)
    assert np.abs(orc.forward_linear_quadratic(q @ R, k @ R, v, "lorentz", 1e-6) - base).max() > 1e-3


def test_orthant_invariant_under_coordinate_permutation():
    rng = np.random.Generator(np.random.PCG64(15))
    T, d = 45, 8
    q, k, v = _unit(rng, (T, d)), _unit(rng, (T, d)), rng.standard_normal((T, 3))
    base = orc.forward_linear_quadratic(q, k, v, "orthant", 1e-6)
    p = rng.permutation(d)
    np.testing.assert_allclose(orc.forward_linear_quadratic(q[:, p], k[:, p], v, "orthant", 1e-6), base,
                               atol=1e-13)


# ------------------------------------------------------------------ identity feature

def test_identity_worked_example():
    ex = GOLDEN["identity_example"]
    q, k, v = _f64(ex["q"]), _f64(ex["k"]), _f64(ex["v"])
    want = _f64(ex["out"])
    np.testing.assert_allclose(orc.forward_identity_quadratic(q, k, v), want, atol=1e-15)
    np.testing.assert_allclose(orc.forward_identity_rows(q, k, v, [0, 1, 2]), want, atol=1e-15)
    for C in (1, 2, 3):
        np.testing.assert_allclose(orc.forward_identity_chunked(q, k, v, C), want, atol=1e-15)


def test_identity_brute_force_in_rationals():
    # o_t = sum_{s<=t} (q_t . k_s) v_s evaluated in exact rationals
    rng = np.random.Generator(np.random.PCG64(31))
    T, d, dv = 6, 3, 2
    qi, ki_, vi = (rng.integers(-4, 5, (T, n)) for n in (d, d, dv))
    den = 3
    want = []
    for t in range(T):
        acc = [Fraction(0)] * dv
        for s in range(t + 1):
            c = sum(Fraction(int(qi[t, a]), den) * Fraction(int(ki_[s, a]), den) for a in range(d))
            acc = [acc[j] + c * int(vi[s, j]) for j in range(dv)]
        want.append([float(x) for x in acc])
    got = orc.forward_identity_quadratic(qi / den, ki_ / den, vi.astype(np.float64))
    np.testing.assert_allclose(got, np.array(want), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("T", [1, 5, 97, 300])
def test_identity_chunked_equals_quadratic(T):
    rng = np.random.Generator(np.random.PCG64(T + 3))
    q, k, v = rng.standard_normal((2, T, 8)), rng.standard_normal((2, T, 8)), rng.standard_normal((2, T, 3))
    want = orc.forward_identity_quadratic(q, k, v)
    for C in (1, 3, 32, 128, T):
        np.testing.assert_allclose(orc.forward_identity_chunked(q, k, v, C), want, rtol=1e-11, atol=1e-11)


def test_identity_recurrence_token_by_token():
    # Sec. 2 with psi(x) = x: S_t = S_{t-1} + k_t v_t^T, o_t = q_t^T S_t
    rng = np.random.Generator(np.random.PCG64(32))
    T, d, dv = 40, 5, 4
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv))
    S = np.zeros((d, dv))
    want = np.empty((T, dv))
    for t in range(T):
        S = S + np.outer(k[t], v[t])
        want[t] = q[t] @ S
    np.testing.assert_allclose(orc.forward_identity_quadratic(q, k, v), want, rtol=1e-12, atol=1e-12)


def test_identity_is_the_orthant_numerator_on_nonnegative_inputs():
    # with q, k >= 0 and no shift the orthant map is the identity, so the
    # identity read equals the orthant read (eps = 0) times its denominator
    # (the identity read of v = 1)
    rng = np.random.Generator(np.random.PCG64(33))
    T = 50
    q, k, v = np.abs(rng.standard_normal((T, 6))), np.abs(rng.standard_normal((T, 6))), rng.standard_normal((T, 3))
    den = orc.forward_identity_quadratic(q, k, np.ones((T, 1)))
    np.testing.assert_allclose(orc.forward_identity_quadratic(q, k, v),
                               orc.forward_linear_quadratic(q, k, v, "orthant", 0.0, shift=0.0) * den,
                               rtol=1e-12)


def test_identity_basis_keys_causal_and_linear():
    T = d = 6
    k = np.eye(d)
    rng = np.random.Generator(np.random.PCG64(34))
    v = rng.standard_normal((T, 3))
    for j in range(d):
        q = np.tile(np.eye(d)[j], (T, 1))
        o = orc.forward_identity_quadratic(q, k, v)
        for t in range(T):
            np.testing.assert_allclose(o[t], v[j] if j <= t else 0.0, atol=0)
    q, kk = rng.standard_normal((T, 4)), rng.standard_normal((T, 4))
    a = orc.forward_identity_quadratic(q, kk, v)
    b = orc.forward_identity_quadratic(q, kk, 2.0 * v - 1.0)
    np.testing.assert_allclose(b, 2.0 * a - orc.forward_identity_quadratic(q, kk, np.ones_like(v)), atol=1e-12)
    v2 = v.copy()
    v2[4:] = 100.0
    np.testing.assert_array_equal(orc.forward_identity_quadratic(q, kk, v2)[:4], a[:4])


# ------------------------------------------------------------------ gated recurrence

def _three_token():
    ex = GOLDEN["three_token_example"]
    return _f64(ex["q"]), _f64(ex["k"]), _f64(ex["v"]), _f64(ex["num"])


def test_gated_worked_example_half():
    q, k, v, _ = _three_token()
    want = _f64(GOLDEN["gated_example"]["out"])
    lg = np.full(3, np.log(0.5))
    np.testing.assert_allclose(orc.gated_recurrence(q, k, v, lg), want, atol=1e-15)
    np.testing.assert_allclose(orc.forward_gated_quadratic(q, k, v, lg), want, atol=1e-15)
    # gamma_1 multiplies the empty state and changes nothing
    lg1 = lg.copy()
    lg1[0] = -7.0
    np.testing.assert_allclose(orc.forward_gated_quadratic(q, k, v, lg1), want, atol=1e-15)


def test_gated_without_decay_is_the_unnormalised_numerator():
    q, k, v, num = _three_token()
    z = np.zeros(3)
    np.testing.assert_allclose(orc.gated_recurrence(q, k, v, z), num, atol=1e-15)
    np.testing.assert_allclose(orc.forward_gated_quadratic(q, k, v, z), num, atol=1e-15)


@pytest.mark.parametrize("g", [1, 2])
def test_gated_recurrence_equals_unrolled(g):
    rng = np.random.Generator(np.random.PCG64(16 + g))
    T, d, dv = 90, 8, 3
    q, k, v = _unit(rng, (T, d)), _unit(rng, (T, d)), rng.standard_normal((T, dv))
    lg = np.log(1 / (1 + np.exp(-(rng.standard_normal(T) + 2))))
    a = orc.gated_recurrence(q, k, v, lg, g)
    b = orc.forward_gated_quadratic(q, k, v, lg, g)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12 * np.abs(a).max())


def test_gated_strong_decay_keeps_only_the_current_token():
    rng = np.random.Generator(np.random.PCG64(18))
    T, d = 20, 4
    q, k, v = _unit(rng, (T, d)), _unit(rng, (T, d)), rng.standard_normal((T, 2))
    o = orc.forward_gated_quadratic(q, k, v, np.full(T, -60.0))
    c = np.sum(q * k, axis=1) ** 2
    np.testing.assert_allclose(o, c[:, None] * v, rtol=1e-12, atol=1e-300)


def test_gated_causal_and_linear_in_v():
    rng = np.random.Generator(np.random.PCG64(19))
    T, d = 30, 4
    q, k = _unit(rng, (T, d)), _unit(rng, (T, d))
    v1, v2 = rng.standard_normal((T, 2)), rng.standard_normal((T, 2))
    lg = -rng.uniform(0, 0.3, T)
    o1 = orc.forward_gated_quadratic(q, k, v1, lg)
    o2 = orc.forward_gated_quadratic(q, k, v2, lg)
    np.testing.assert_allclose(orc.forward_gated_quadratic(q, k, 2 * v1 - v2, lg), 2 * o1 - o2,
                               atol=1e-12)
    q3, k3, v3, lg3 = q.copy(), k.copy(), v1.copy(), lg.copy()
    q3[20:], k3[20:], v3[20:], lg3[20:] = 0.3, -0.2, 9.0, -0.01
    np.testing.assert_array_equal(orc.forward_gated_quadratic(q3, k3, v3, lg3)[:20], o1[:20])


def test_gated_rows_match_the_full_form():
    rng = np.random.Generator(np.random.PCG64(21))
    T = 64
    q, k, v = _unit(rng, (T, 8)), _unit(rng, (T, 8)), rng.standard_normal((T, 3))
    lg = -rng.uniform(0, 0.2, T)
    rows = [0, 1, 40, 63]
    for g in (1, 2):
        np.testing.assert_allclose(orc.forward_gated_rows(q, k, v, lg, rows, g),
                                   orc.forward_gated_quadratic(q, k, v, lg, g)[rows], rtol=1e-12, atol=1e-14)


def test_gated_decode_continues_the_forward():
    # state of the first 40 tokens, then 25 gated steps == the gated read of all 65
    rng = np.random.Generator(np.random.PCG64(22))
    T, n, d, dv = 40, 25, 4, 3
    q, k, v = _unit(rng, (T + n, d)), _unit(rng, (T + n, d)), rng.standard_normal((T + n, dv))
    lg = -rng.uniform(0, 0.3, T + n)
    want = orc.forward_gated_quadratic(q, k, v, lg)
    S = orc.gated_state(k[:T], v[:T], lg[:T])
    # the state reads out the history's last row: phi(q_T-1)^T S = o_T-1
    np.testing.assert_allclose(orc.feature_map(q[T - 1]) @ S, want[T - 1], rtol=1e-12, atol=1e-13)
    for t in range(T, T + n):
        S, o = orc.decode_step_gated(S, q[t], k[t], v[t], lg[t])
        np.testing.assert_allclose(o, want[t], rtol=1e-11, atol=1e-12)
    # and matches the token-by-token recurrence's state
    np.testing.assert_allclose(S, orc.gated_state(k, v, lg), rtol=1e-12, atol=1e-13)


def test_gated_decode_without_decay_is_the_additive_step():
    rng = np.random.Generator(np.random.PCG64(23))
    d, dv = 5, 2
    S0, z0 = orc.decode_state(_unit(rng, (30, d)), rng.standard_normal((30, dv)))
    q, k, v = _unit(rng, d), _unit(rng, d), rng.standard_normal(dv)
    S1, o = orc.decode_step_gated(S0, q, k, v, 0.0)
    S2, z2, o2 = orc.decode_step(S0, z0, q, k, v, 0.0)
    np.testing.assert_allclose(S1, S2, rtol=1e-14)
    np.testing.assert_allclose(o, o2 * (orc.feature_map(q) @ z2), rtol=1e-12)
