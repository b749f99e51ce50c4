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

Readings where the page is silent (each also listed in the design notes):
  * eps is added once to the accumulated denominator, o = N / (D + eps); the
    page calls small eps terms a safeguard against a zero denominator
    (App. A) without fixing where they go.
  * the causal mask includes the diagonal (sums run to i = t in Eqs. 1-2).
  * a final partial chunk is zero-padded (App. D.2 and App. E.1 pad it); psi(0) = 0 so the
    padding adds nothing, and padded query rows are discarded.
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


# ------------------------------------------------------------ forward

def forward_quadratic(q: np.ndarray, k: np.ndarray, v: np.ndarray, eps: float,
                      block: int = 256) -> np.ndarray:
    """Plain definition of the causal normalised read, O(T^2) per head.

    q, k: [..., T, d]; v: [..., T, dv]  ->  o: [..., T, dv] (fp64).
    For each t: c_{t,s} = (q_t . k_s)^2 for s <= t,
    o_t = sum_s c_{t,s} v_s / (sum_s c_{t,s} + eps).  Query rows are taken in
    blocks only to bound memory; each row's sums are over the same key set.
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
            c = (qf[h, t0:t1] @ kf[h, :t1].T) ** 2          # [rows, t1]
            rows = np.arange(t0, t1)[:, None]
            cols = np.arange(t1)[None, :]
            c = np.where(cols <= rows, c, 0.0)               # causal, diagonal kept
            num = c @ vf[h, :t1]
            den = c.sum(axis=1, keepdims=True)
            out[h, t0:t1] = num / (den + eps)
    return out.reshape(lead + (T, vf.shape[-1]))


def forward_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows, eps: float) -> np.ndarray:
    """The same plain definition as forward_quadratic, for selected query rows
    of one head only (for spot checks of long sequences).

    q, k: [T, d]; v: [T, dv]; rows: query positions.  Returns [len(rows), dv]:
    o_t = sum_{s<=t} (q_t.k_s)^2 v_s / (sum_{s<=t} (q_t.k_s)^2 + eps).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((len(rows), v.shape[-1]))
    for n, t in enumerate(rows):
        c = (k[: t + 1] @ q[t]) ** 2
        out[n] = (c @ v[: t + 1]) / (c.sum() + eps)
    return out


def forward_chunked(q: np.ndarray, k: np.ndarray, v: np.ndarray, chunk: int,
                    eps: float) -> np.ndarray:
    """Chunkwise form, Eqs. 17-20 with the sequential inter-chunk prefix.

    Per head: S = 0 (D x dv), Z = 0 (D).  For each chunk c:
      Psi_Q, Psi_K = phi(Q_c), phi(K_c)                     (C x D)
      P = (Psi_Q Psi_K^T) * M,  M lower-triangular incl. diagonal
      N = Psi_Q S + P V_c;  Den = Psi_Q Z + P 1;  O_c = N / (Den + eps)
      S += Psi_K^T V_c;  Z += Psi_K^T 1
    The final chunk is zero-padded and its padded rows dropped.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    T, d = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    D = feature_dim(d)
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
            PQ = feature_map(qf[h, sl])
            PK = feature_map(kf[h, sl])
            Vc = vf[h, sl]
            P = (PQ @ PK.T) * M
            N = PQ @ S + P @ Vc
            Den = PQ @ Z + P.sum(axis=1)
            with np.errstate(invalid="ignore", divide="ignore"):  # padded rows only
                out[h, sl] = N / (Den + eps)[:, None]
            S = S + PK.T @ Vc
            Z = Z + PK.sum(axis=0)
    return out[:, :T].reshape(lead + (T, dv))


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
