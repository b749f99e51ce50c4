"""fp64 CPU oracle for causal linear attention with KATA's rank-one PSD feature map.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library and imports nothing from it.

Everything here is plain NumPy in float64, written for a reader to check by
eye against the source page, "Kernelized Linear Attention: Breaking the
Capacity Wall with Symmetric Cones" (Ghriss & Chakraborty, arXiv 2607.17419):

  feature_pairs / feature_weights / feature_map
      Sec. 3.1 (rank-one lift psi(u) = u u^T, whose Frobenius inner products
      are squared dot products) and Eq. 8 (n = p(p+1)/2 free coordinates of a
      symmetric matrix).  Packing order and the sqrt(2) off-diagonal weight are
      this library's convention (row-major upper triangle); the page fixes only
      the count.
  forward_quadratic
      Eq. 2 (the linearised readout z_t = psi(q_t)^T S_t / psi(q_t)^T Z_t with
      sums over i <= t) written out as its plain definition: score
      c_{t,s} = (q_t . k_s)^2 for s <= t, o_t = sum c v_s / (sum c + eps).
  forward_chunked
      Sec. 4.1 Eqs. 17-20 and App. D.2 (chunkwise forward: per-chunk feature matrices,
      lower-triangular causal mask, inter-chunk state update, O = diag(D)^-1 N),
      in the page's order: read out with the incoming state, then update it.
  decode_state / decode_step
      Sec. 2, below Eq. 2: additive recurrence S_t = S_{t-1} + psi(k_t) v_t^T,
      Z_t = Z_{t-1} + psi(k_t), read out after the update.
  convex_gate
      Sec. 2.2, Proposition 1 (output-level gating): alpha_t = D_{t-1}/D_t,
      beta_t = c_t/D_t.
  feature_map_blocks, and the g argument of the forward functions
      Sec. 4.1, the KATA-Mg block family: u = (u_1, ..., u_g) in g equal
      blocks of width m = d/g, psi_Mg(u) = (u_1 u_1^T, ..., u_g u_g^T), whose
      inner products are sum_a (q_a . k_a)^2; g = 1 is the full map.
  feature_orthant / feature_lorentz / forward_linear_quadratic /
  forward_linear_rows / forward_linear_chunked
      the linear (D = d) cone features: KATA-Orthant psi(x) = ReLU(x) + shift,
      KATA-Lorentz psi(x) = (y, |y|_2 (1 + s^2)) with y = x_{1:d-1}, s = x_d
      (App. F.4; Sec. 2.3 names both cone families), read with the same
      normalised causal sum, score c_{t,s} = psi(q_t) . psi(k_s) unsquared.
  forward_identity_quadratic / forward_identity_rows / forward_identity_chunked
      the identity feature psi(x) = x with a d x dv state, the first-order
      workload of the associative-scan tables (Sec. 4.2, Tables 10-11):
      o_t = sum_{s<=t} (q_t . k_s) v_s, read without a denominator.
  gated_recurrence / forward_gated_quadratic / forward_gated_rows
      GatedKATA (App. F.4): S_t = gamma_t S_{t-1} + psi(k_t) v_t^T,
      o_t = psi(q_t)^T S_t, no denominator; its unrolled form
      S_t = sum_s (prod_{r=s+1..t} gamma_r) psi(k_s) v_s^T (Sec. 5.2).
      The per-token gate enters as log gamma_t (<= 0), the quantity the page's
      gate projection produces.
  gated_state / decode_step_gated
      the GatedKATA state after a history and one recurrent step of it.

Readings where the page is silent (each also listed in the design notes):
  * eps is added once to the accumulated denominator, o = N / (D + eps); the
    page calls small eps terms a safeguard against a zero denominator
    (App. A) without fixing where they go.
  * the causal mask includes the diagonal (sums run to i = t in Eqs. 1-2).
  * a final partial chunk is zero-padded (App. D.2 and App. E.1 pad it); psi(0) = 0 so the
    padding adds nothing, and padded query rows are discarded.
  * the linear features use the same eps-on-the-denominator read as the PSD
    map (the page's orthant recurrence divides without one; its orthant shift
    keeps that denominator positive, the Lorentz map only makes it >= 0).
  * the gated read has no denominator and no eps, as the page writes it.
  * the identity feature's scores q.k are signed, so its sum can vanish or
    change sign; it is read without a denominator (the d x dv state of the
    page's first-order tables carries no normaliser).
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np


# ------------------------------------------------------------ feature map

def feature_dim(d: int) -> int:
    """Packed width of the symmetric d x d lift: d(d+1)/2 (Eq. 8)."""
    return d * (d + 1) // 2


def feature_pairs(d: int) -> List[Tuple[int, int]]:
    """(i, j), i <= j, of each packed coordinate, row-major upper triangle.

    Index of (i, j) is i*d - i*(i-1)/2 + (j - i).
    """
    return [(i, j) for i in range(d) for j in range(i, d)]


def feature_weights(d: int) -> np.ndarray:
    """Squared weight of each packed coordinate: 1 on the diagonal, 2 off it.

    vec(u u^T) holds each off-diagonal product u_i u_j twice; folding the two
    copies into one packed coordinate scaled by sqrt(2) keeps every Frobenius
    inner product (Sec. 3.1).
    """
    return np.array([1.0 if i == j else 2.0 for (i, j) in feature_pairs(d)])


def feature_map(x: np.ndarray) -> np.ndarray:
    """phi(x)_{(i,j)} = sqrt(w_ij) x_i x_j over the packed upper triangle."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    pairs = feature_pairs(d)
    ii = np.array([p[0] for p in pairs], dtype=np.int64)
    jj = np.array([p[1] for p in pairs], dtype=np.int64)
    scale = np.sqrt(feature_weights(d))
    return x[..., ii] * x[..., jj] * scale


def block_width(d: int, g: int) -> int:
    """m = d/g, the width of each of the g blocks (g must divide d)."""
    if g < 1 or d % g:
        raise ValueError(f"g = {g} does not divide d = {d}")
    return d // g


def feature_map_blocks(x: np.ndarray, g: int) -> np.ndarray:
    """psi_Mg(x): the packed lift of each block x_a = x[a m:(a+1) m], blocks
    in order, so coordinate a*m(m+1)/2 + idx_m(i, j) is sqrt(w_ij) x_{am+i} x_{am+j}.
    Width g m(m+1)/2 (Sec. 4.1); g = 1 is feature_map."""
    x = np.asarray(x, dtype=np.float64)
    m = block_width(x.shape[-1], g)
    return np.concatenate([feature_map(x[..., a * m:(a + 1) * m]) for a in range(g)], axis=-1)


def block_scores(qr: np.ndarray, kr: np.ndarray, g: int) -> np.ndarray:
    """sum_a (q_a . k_a)^2 for every (query row, key row) pair: [rows, keys].

    The block family's kernel, <psi_Mg(q), psi_Mg(k)>; g = 1 gives (q . k)^2."""
    m = block_width(qr.shape[-1], g)
    c = np.zeros((qr.shape[0], kr.shape[0]))
    for a in range(g):
        sl = slice(a * m, (a + 1) * m)
        c = c + (qr[:, sl] @ kr[:, sl].T) ** 2
    return c


# ------------------------------------------------------------ forward

def forward_quadratic(q: np.ndarray, k: np.ndarray, v: np.ndarray, eps: float,
                      block: int = 256, g: int = 1) -> np.ndarray:
    """Plain definition of the causal normalised read, O(T^2) per head.

    q, k: [..., T, d]; v: [..., T, dv]  ->  o: [..., T, dv] (fp64).
    For each t: c_{t,s} = (q_t . k_s)^2 for s <= t (with g blocks:
    sum_a (q_{t,a} . k_{s,a})^2), o_t = sum_s c_{t,s} v_s / (sum_s c_{t,s} + eps).
    Query rows are taken in blocks only to bound memory; each row's sums are
    over the same key set.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    T = q.shape[-2]
    qf = q.reshape((-1, T, q.shape[-1]))
    kf = k.reshape((-1, T, k.shape[-1]))
    vf = v.reshape((-1, T, v.shape[-1]))
    out = np.empty((qf.shape[0], T, vf.shape[-1]), dtype=np.float64)
    for h in range(qf.shape[0]):
        for t0 in range(0, T, block):
            t1 = min(T, t0 + block)
            c = block_scores(qf[h, t0:t1], kf[h, :t1], g)   # [rows, t1]
            rows = np.arange(t0, t1)[:, None]
            cols = np.arange(t1)[None, :]
            c = np.where(cols <= rows, c, 0.0)               # causal, diagonal kept
            num = c @ vf[h, :t1]
            den = c.sum(axis=1, keepdims=True)
            out[h, t0:t1] = num / (den + eps)
    return out.reshape(lead + (T, vf.shape[-1]))


def forward_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows, eps: float,
                 g: int = 1) -> np.ndarray:
    """The same plain definition as forward_quadratic, for selected query rows
    of one head only (for spot checks of long sequences).

    q, k: [T, d]; v: [T, dv]; rows: query positions.  Returns [len(rows), dv]:
    o_t = sum_{s<=t} c_{t,s} v_s / (sum_{s<=t} c_{t,s} + eps), c as in
    forward_quadratic.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((len(rows), v.shape[-1]))
    for n, t in enumerate(rows):
        c = block_scores(q[t][None, :], k[: t + 1], g)[0]
        out[n] = (c @ v[: t + 1]) / (c.sum() + eps)
    return out


def forward_chunked(q: np.ndarray, k: np.ndarray, v: np.ndarray, chunk: int,
                    eps: float, g: int = 1) -> np.ndarray:
    """Chunkwise form, Eqs. 17-20 with the sequential inter-chunk prefix.

    Per head: S = 0 (D x dv), Z = 0 (D).  For each chunk c:
      Psi_Q, Psi_K = phi(Q_c), phi(K_c)                     (C x D)
      P = (Psi_Q Psi_K^T) * M,  M lower-triangular incl. diagonal
      N = Psi_Q S + P V_c;  Den = Psi_Q Z + P 1;  O_c = N / (Den + eps)
      S += Psi_K^T V_c;  Z += Psi_K^T 1
    The final chunk is zero-padded and its padded rows dropped.  phi is the
    packed lift, or psi_Mg with g blocks.
    """
    return _chunked(q, k, v, chunk, eps, lambda x: feature_map_blocks(x, g))


def _chunked(q, k, v, chunk, eps, psi):
    """Eqs. 17-20 for any feature map psi: [rows, d] -> [rows, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    T, d = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    D = psi(np.zeros((1, d))).shape[-1]
    nc = -(-T // chunk)
    Tp = nc * chunk
    qf = np.zeros((int(np.prod(lead, dtype=np.int64)), Tp, d))
    kf = np.zeros_like(qf)
    vf = np.zeros((qf.shape[0], Tp, dv))
    qf[:, :T] = q.reshape((-1, T, d))
    kf[:, :T] = k.reshape((-1, T, d))
    vf[:, :T] = v.reshape((-1, T, dv))
    M = np.tril(np.ones((chunk, chunk)))
    out = np.empty((qf.shape[0], Tp, dv))
    for h in range(qf.shape[0]):
        S = np.zeros((D, dv))
        Z = np.zeros(D)
        for c in range(nc):
            sl = slice(c * chunk, (c + 1) * chunk)
            PQ = psi(qf[h, sl])
            PK = psi(kf[h, sl])
            Vc = vf[h, sl]
            P = (PQ @ PK.T) * M
            N = PQ @ S + P @ Vc
            Den = PQ @ Z + P.sum(axis=1)
            with np.errstate(invalid="ignore", divide="ignore"):  # padded rows only
                out[h, sl] = N / (Den + eps)[:, None]
            S = S + PK.T @ Vc
            Z = Z + PK.sum(axis=0)
    return out[:, :T].reshape(lead + (T, dv))


# ------------------------------------------------------------ linear cone features

def feature_orthant(x: np.ndarray, shift: float) -> np.ndarray:
    """KATA-Orthant: psi(x) = ReLU(x) + shift (every coordinate), D = d."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + shift


def feature_lorentz(x: np.ndarray) -> np.ndarray:
    """KATA-Lorentz: with y = x_{1:d-1} and s = x_d,
    psi(x) = (y, |y|_2 (1 + s^2)), D = d; its last coordinate is >= |y|_2,
    so psi(x) lies in the closed Lorentz cone."""
    x = np.asarray(x, dtype=np.float64)
    y = x[..., :-1]
    s = x[..., -1:]
    return np.concatenate([y, np.sqrt(np.sum(y * y, axis=-1, keepdims=True)) * (1.0 + s * s)], axis=-1)


def linear_feature(name: str, shift: float = 1e-6):
    """The feature map called `name` ("orthant" or "lorentz") as a function of x."""
    if name == "orthant":
        return lambda x: feature_orthant(x, shift)
    if name == "lorentz":
        return feature_lorentz
    raise ValueError(f"unknown linear feature {name!r}")


def forward_linear_quadratic(q: np.ndarray, k: np.ndarray, v: np.ndarray, feature: str,
                             eps: float, shift: float = 1e-6, block: int = 256) -> np.ndarray:
    """Plain definition of the causal normalised read with a linear feature:
    c_{t,s} = psi(q_t) . psi(k_s) for s <= t, o_t = sum c v_s / (sum c + eps)."""
    psi = linear_feature(feature, shift)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    T = q.shape[-2]
    pq = psi(q.reshape((-1, T, q.shape[-1])))
    pk = psi(k.reshape((-1, T, k.shape[-1])))
    vf = v.reshape((-1, T, v.shape[-1]))
    out = np.empty((pq.shape[0], T, vf.shape[-1]))
    for h in range(pq.shape[0]):
        for t0 in range(0, T, block):
            t1 = min(T, t0 + block)
            c = pq[h, t0:t1] @ pk[h, :t1].T
            rows = np.arange(t0, t1)[:, None]
            cols = np.arange(t1)[None, :]
            c = np.where(cols <= rows, c, 0.0)
            out[h, t0:t1] = (c @ vf[h, :t1]) / (c.sum(axis=1, keepdims=True) + eps)
    return out.reshape(lead + (T, vf.shape[-1]))


def forward_linear_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows, feature: str,
                        eps: float, shift: float = 1e-6) -> np.ndarray:
    """forward_linear_quadratic for selected query rows of one head:
    q, k: [T, d]; v: [T, dv]; returns [len(rows), dv]."""
    psi = linear_feature(feature, shift)
    pk = psi(np.asarray(k, dtype=np.float64))
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((len(rows), v.shape[-1]))
    for n, t in enumerate(rows):
        c = pk[: t + 1] @ psi(np.asarray(q[t], dtype=np.float64))
        out[n] = (c @ v[: t + 1]) / (c.sum() + eps)
    return out


def forward_linear_chunked(q: np.ndarray, k: np.ndarray, v: np.ndarray, chunk: int,
                           feature: str, eps: float, shift: float = 1e-6) -> np.ndarray:
    """Eqs. 17-20 with a linear feature (state D x dv with D = d)."""
    return _chunked(q, k, v, chunk, eps, linear_feature(feature, shift))


# ------------------------------------------------------------ identity feature

def forward_identity_quadratic(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                               block: int = 256) -> np.ndarray:
    """The first-order read with the identity feature psi(x) = x and a d x dv
    state, the workload of the page's associative-scan tables (Sec. 4.2,
    Tables 10-11): o_t = sum_{s<=t} (q_t . k_s) v_s.  Its scores are signed,
    so it is read without a denominator (a normalised read could divide by
    zero or flip sign).  q, k: [..., T, d]; v: [..., T, dv] -> [..., T, dv]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    T = q.shape[-2]
    qf = q.reshape((-1, T, q.shape[-1]))
    kf = k.reshape((-1, T, k.shape[-1]))
    vf = v.reshape((-1, T, v.shape[-1]))
    out = np.empty((qf.shape[0], T, vf.shape[-1]))
    for h in range(qf.shape[0]):
        for t0 in range(0, T, block):
            t1 = min(T, t0 + block)
            c = qf[h, t0:t1] @ kf[h, :t1].T
            rows = np.arange(t0, t1)[:, None]
            cols = np.arange(t1)[None, :]
            out[h, t0:t1] = np.where(cols <= rows, c, 0.0) @ vf[h, :t1]
    return out.reshape(lead + (T, vf.shape[-1]))


def forward_identity_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows) -> np.ndarray:
    """forward_identity_quadratic for selected query rows of one head:
    q, k: [T, d]; v: [T, dv]; returns [len(rows), dv]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((len(rows), v.shape[-1]))
    for n, t in enumerate(rows):
        out[n] = (k[: t + 1] @ q[t]) @ v[: t + 1]
    return out


def forward_identity_chunked(q: np.ndarray, k: np.ndarray, v: np.ndarray, chunk: int) -> np.ndarray:
    """Eqs. 17-20 with psi(x) = x and no normalisation, per head: S = 0
    (d x dv); for each chunk c, O_c = Q_c S + ((Q_c K_c^T) * M) V_c, then
    S += K_c^T V_c.  The final chunk is zero-padded, padded rows dropped."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    T, d = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    nc = -(-T // chunk)
    Tp = nc * chunk
    qf = np.zeros((int(np.prod(lead, dtype=np.int64)), Tp, d))
    kf = np.zeros_like(qf)
    vf = np.zeros((qf.shape[0], Tp, dv))
    qf[:, :T] = q.reshape((-1, T, d))
    kf[:, :T] = k.reshape((-1, T, d))
    vf[:, :T] = v.reshape((-1, T, dv))
    M = np.tril(np.ones((chunk, chunk)))
    out = np.empty((qf.shape[0], Tp, dv))
    for h in range(qf.shape[0]):
        S = np.zeros((d, dv))
        for c in range(nc):
            sl = slice(c * chunk, (c + 1) * chunk)
            Qc, Kc, Vc = qf[h, sl], kf[h, sl], vf[h, sl]
            out[h, sl] = Qc @ S + ((Qc @ Kc.T) * M) @ Vc
            S = S + Kc.T @ Vc
    return out[:, :T].reshape(lead + (T, dv))


# ------------------------------------------------------------ gated recurrence

def gated_recurrence(q: np.ndarray, k: np.ndarray, v: np.ndarray, log_gamma: np.ndarray,
                     g: int = 1) -> np.ndarray:
    """GatedKATA token by token, one head: S_t = gamma_t S_{t-1} + psi(k_t) v_t^T,
    o_t = psi(q_t)^T S_t, psi = psi_Mg (g = 1: the full map), S_0 = 0.

    q, k: [T, d]; v: [T, dv]; log_gamma: [T].  O(T D dv): small cases only."""
    pq = feature_map_blocks(q, g)
    pk = feature_map_blocks(k, g)
    v = np.asarray(v, dtype=np.float64)
    gamma = np.exp(np.asarray(log_gamma, dtype=np.float64))
    S = np.zeros((pk.shape[-1], v.shape[-1]))
    out = np.empty((q.shape[0], v.shape[-1]))
    for t in range(q.shape[0]):
        S = gamma[t] * S + np.outer(pk[t], v[t])
        out[t] = pq[t] @ S
    return out


def forward_gated_quadratic(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                            log_gamma: np.ndarray, g: int = 1, block: int = 256) -> np.ndarray:
    """The unrolled GatedKATA read: o_t = sum_{s<=t} (prod_{r=s+1..t} gamma_r)
    c_{t,s} v_s with c from block_scores; the product is exp(L_t - L_s),
    L = running sum of log gamma.

    q, k: [..., T, d]; v: [..., T, dv]; log_gamma: [..., T]  ->  [..., T, dv]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    T = q.shape[-2]
    qf = q.reshape((-1, T, q.shape[-1]))
    kf = k.reshape((-1, T, k.shape[-1]))
    vf = v.reshape((-1, T, v.shape[-1]))
    L = np.cumsum(np.asarray(log_gamma, dtype=np.float64).reshape((-1, T)), axis=-1)
    out = np.empty((qf.shape[0], T, vf.shape[-1]))
    for h in range(qf.shape[0]):
        for t0 in range(0, T, block):
            t1 = min(T, t0 + block)
            c = block_scores(qf[h, t0:t1], kf[h, :t1], g)
            rows = np.arange(t0, t1)[:, None]
            cols = np.arange(t1)[None, :]
            decay = np.exp(np.where(cols <= rows, L[h, t0:t1][:, None] - L[h, :t1][None, :], -np.inf))
            out[h, t0:t1] = (c * decay) @ vf[h, :t1]
    return out.reshape(lead + (T, vf.shape[-1]))


def forward_gated_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, log_gamma: np.ndarray, rows,
                       g: int = 1) -> np.ndarray:
    """forward_gated_quadratic for selected query rows of one head:
    q, k: [T, d]; v: [T, dv]; log_gamma: [T]; returns [len(rows), dv]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L = np.cumsum(np.asarray(log_gamma, dtype=np.float64))
    out = np.empty((len(rows), v.shape[-1]))
    for n, t in enumerate(rows):
        c = block_scores(q[t][None, :], k[: t + 1], g)[0]
        out[n] = (c * np.exp(L[t] - L[: t + 1])) @ v[: t + 1]
    return out


# ------------------------------------------------------------ recurrent decode

def decode_state(k: np.ndarray, v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """State after a history: S = sum_s phi(k_s) v_s^T, z = sum_s phi(k_s).

    k: [..., T, d], v: [..., T, dv]  ->  S [..., D, dv], z [..., D] (fp64),
    the sqrt(2)-weighted packing of feature_map.
    """
    pk = feature_map(k)
    S = np.einsum("...tf,...tc->...fc", pk, np.asarray(v, dtype=np.float64))
    z = pk.sum(axis=-2)
    return S, z


def decode_step(S: np.ndarray, z: np.ndarray, q: np.ndarray, k: np.ndarray,
                v: np.ndarray, eps: float):
    """One token of the additive recurrence, read after the update.

    S [..., D, dv], z [..., D]; q, k [..., d]; v [..., dv].
    S' = S + phi(k) v^T, z' = z + phi(k), o = phi(q)^T S' / (phi(q)^T z' + eps).
    Returns (S', z', o).
    """
    pq = feature_map(q)
    pk = feature_map(k)
    v = np.asarray(v, dtype=np.float64)
    S2 = S + pk[..., :, None] * v[..., None, :]
    z2 = z + pk
    num = np.einsum("...f,...fc->...c", pq, S2)
    den = np.einsum("...f,...f->...", pq, z2)
    return S2, z2, num / (den + eps)[..., None]


def gated_state(k: np.ndarray, v: np.ndarray, log_gamma: np.ndarray) -> np.ndarray:
    """GatedKATA state after a history, the unrolled recurrence (Sec. 5.2):
    S = sum_s (prod_{r=s+1..T} gamma_r) phi(k_s) v_s^T, public packing.
    k: [T, d], v: [T, dv], log_gamma: [T]  ->  S [D, dv]."""
    lg = np.asarray(log_gamma, dtype=np.float64)
    after = np.cumsum(lg[::-1])[::-1] - lg          # sum of log gamma over r > s
    pk = feature_map(k) * np.exp(after)[:, None]
    return pk.T @ np.asarray(v, dtype=np.float64)


def decode_step_gated(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      log_gamma) -> Tuple[np.ndarray, np.ndarray]:
    """One GatedKATA token (App. F.4), read after the update:
    S' = gamma S + phi(k) v^T, o = phi(q)^T S'.  S [..., D, dv]; q, k [..., d];
    v [..., dv]; log_gamma [...].  Returns (S', o)."""
    gamma = np.exp(np.asarray(log_gamma, dtype=np.float64))
    S2 = gamma[..., None, None] * S + feature_map(k)[..., :, None] * np.asarray(v, dtype=np.float64)[..., None, :]
    return S2, np.einsum("...f,...fc->...c", feature_map(q), S2)


# ------------------------------------------------------------ Proposition 1

def convex_gate(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """Proposition 1 quantities for one head at eps = 0.

    q, k: [T, d], v: [T, dv].  Returns (alpha, beta, zbar_prev, o) with
    D_{t-1} = sum_{s<t} c_{t,s}, c_t = c_{t,t}, D_t = D_{t-1} + c_t,
    alpha = D_{t-1}/D_t, beta = c_t/D_t, zbar_prev = sum_{s<t} c v_s / D_{t-1}
    (zero where D_{t-1} = 0), o = alpha zbar_prev + beta v_t.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T = q.shape[0]
    c = (q @ k.T) ** 2
    strict = np.tril(np.ones((T, T)), k=-1)
    cprev = c * strict
    Dprev = cprev.sum(axis=1)
    ct = np.diag(c).copy()
    Dt = Dprev + ct
    with np.errstate(invalid="ignore", divide="ignore"):
        alpha = np.where(Dt > 0, Dprev / Dt, math.nan)
        beta = np.where(Dt > 0, ct / Dt, math.nan)
        zbar = np.where(Dprev[:, None] > 0, (cprev @ v) / Dprev[:, None], 0.0)
    o = alpha[:, None] * zbar + beta[:, None] * v
    return alpha, beta, zbar, o
