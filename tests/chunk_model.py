"""fp64 model of the chunkwise (WY/UT) form of KDA, as the GPU kernels tile it.

Test infrastructure. It shares no code with the oracle (it re-derives the
pre-processing itself) and none with the HIP path. Its job is to pin the chunk
algebra the kernels rely on against the token-by-token oracle: the intra-chunk
tiles, the unit-lower-triangular solve, w/u, the state walk, and the bounded
reference-row factorisation of the decay (aiter PR 4741, Optimizations Applied:
the split path builds its C x C tiles with a bounded construction that stays
NaN-free to 640 nats, while factoring against one per-chunk reference row overflows
fp32 at ~90-115 nats).

Within a chunk of C rows, with G the inclusive in-chunk cumsum of the gate per key
channel (so G is non-increasing down the rows):

    A[r,i] = beta_r sum_c k_r[c] k_i[c] e^{G_r[c]-G_i[c]}      i <  r
    P[r,i] = scale sum_c q_r[c] k_i[c] e^{G_r[c]-G_i[c]}       i <= r
    T = (I + A)^{-1};  W = T diag(beta) (k * e^G);  U = T diag(beta) v
    Delta = U - W S0^T;  O = scale (q * e^G) S0^T + P Delta
    S_C = S0 Diag(e^{G_C}) + Delta^T (k * e^{G_C - G})

Reference-row factorisation: rows are grouped in blocks of ``ref_block``; a row r in
block b uses the block's first row m_b as reference, splitting
e^{G_r - G_i} = e^{G_r - G_{m_b}} * e^{G_{m_b} - G_i}. For i < m_b both factors are
<= 1; for i inside the block the right factor is >= 1 but bounded by the decay over
ref_block - 1 rows, which the kernel keeps below e^80 by choosing ref_block from the
gate's lower bound.
"""
from __future__ import annotations

import numpy as np


def _l2n(x, eps=1e-6):
    n2 = np.einsum("...c,...c->...", x, x)
    return x / np.sqrt(n2 + eps)[..., None]


def _sig(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def ref_block_for(lower_bound: float, limit_nats: float = 80.0) -> int:
    """Largest block in {16, 8, 4, 2, 1} whose in-block decay stays <= limit_nats."""
    lb = abs(float(lower_bound))
    for s in (16, 8, 4, 2):
        if (s - 1) * lb <= limit_nats:
            return s
    return 1


def chunk_tiles(qn, kn, vv, G, beta, scale, ref_block):
    """Per-chunk, per-head tiles for one padded chunk of C rows.

    qn, kn: [C, K] normalised; vv: [C, V]; G: [C, K] in-chunk cumsum; beta: [C].
    Returns a dict with A, P, T, W, U, Qt, Kt, eGC, the largest exponent of any factor
    (``max_pos``) and the smallest left-factor exponent (``min_left``). Right-factor
    exponents below zero only ever underflow towards 0, which is harmless because the
    true product is smaller still.
    """
    C, K = kn.shape
    assert C % ref_block == 0
    Araw = np.zeros((C, C))
    Praw = np.zeros((C, C))
    max_pos = 0.0  # largest exponent of any factor (overflow risk)
    min_left = 0.0  # smallest left-factor exponent (must not underflow: it can meet a large right factor)
    for b in range(C // ref_block):
        m = b * ref_block
        rows = slice(m, m + ref_block)
        ncols = min(C, m + ref_block)
        left_e = G[rows] - G[m]  # <= 0
        right_e = G[m] - G[:ncols]  # <= 0 before m, >= 0 inside the block
        max_pos = max(max_pos, float(np.max(right_e)), float(np.max(left_e)))
        min_left = min(min_left, float(np.min(left_e)))
        Lk = kn[rows] * np.exp(left_e)
        Lq = qn[rows] * np.exp(left_e)
        R = kn[:ncols] * np.exp(right_e)
        Araw[rows, :ncols] = Lk @ R.T
        Praw[rows, :ncols] = Lq @ R.T
    A = np.tril(Araw, -1) * beta[:, None]
    P = np.tril(Praw, 0) * scale
    T = np.linalg.solve(np.eye(C) + A, np.eye(C))
    Tb = T * beta[None, :]
    W = Tb @ (kn * np.exp(G))
    U = Tb @ vv
    Qt = scale * qn * np.exp(G)
    Kt = kn * np.exp(G[-1][None, :] - G)
    return dict(A=A, P=P, T=T, W=W, U=U, Qt=Qt, Kt=Kt, eGC=np.exp(G[-1]), max_pos=max_pos, min_left=min_left)


def chunk_sequence(q, k, v, g_raw, beta_raw, S0, scale, lower_bound, C=32, ref_block=None,
                   eps=1e-6, return_tiles=False):
    """Chunkwise forward of one sequence, all heads.

    q, k, g_raw: [L, H, K]; v: [L, H, V]; beta_raw: [L, H]; S0: [H, V, K].
    Returns (o [L, H, V], S [H, V, K]) and optionally the per-chunk tiles.
    """
    L = q.shape[0]
    H, V, K = S0.shape
    if ref_block is None:
        ref_block = min(ref_block_for(lower_bound), C)
    qn = _l2n(np.asarray(q, np.float64), eps)
    kn = _l2n(np.asarray(k, np.float64), eps)
    g = lower_bound * _sig(g_raw)
    beta = _sig(beta_raw)
    S = np.array(S0, np.float64, copy=True)
    out = np.zeros((L, H, V))
    tiles = []
    for c0 in range(0, L, C):
        n = min(C, L - c0)
        # Padding rows: q = k = v = 0, g = 0, beta = 0 (an exact no-op).
        Qc = np.zeros((C, H, K)); Qc[:n] = qn[c0:c0 + n]
        Kc = np.zeros((C, H, K)); Kc[:n] = kn[c0:c0 + n]
        Vc = np.zeros((C, H, V)); Vc[:n] = v[c0:c0 + n]
        gc = np.zeros((C, H, K)); gc[:n] = g[c0:c0 + n]
        bc = np.zeros((C, H)); bc[:n] = beta[c0:c0 + n]
        G = np.cumsum(gc, axis=0)  # padding rows carry the last valid row's G
        per_head = []
        for h in range(H):
            t = chunk_tiles(Qc[:, h], Kc[:, h], Vc[:, h], G[:, h], bc[:, h], scale, ref_block)
            X = t["W"] @ S[h].T
            Delta = t["U"] - X
            O = t["Qt"] @ S[h].T + t["P"] @ Delta
            S0h = S[h].copy()
            S[h] = S[h] * t["eGC"][None, :] + Delta.T @ t["Kt"]
            out[c0:c0 + n, h] = O[:n]
            if return_tiles:
                t["S0"] = S0h
                t["Delta"] = Delta
                per_head.append(t)
        if return_tiles:
            tiles.append(per_head)
    if return_tiles:
        return out, S, tiles
    return out, S


def affine_chunk_map(t):
    """Chunk transition as S_C = S0 M + B (M: K x K, B: V x K)."""
    M = np.diag(t["eGC"]) - t["W"].T @ t["Kt"]
    B = t["U"].T @ t["Kt"]
    return M, B
