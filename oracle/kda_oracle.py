"""fp64 CPU oracle for chunkwise Kimi Delta Attention (KDA) prefill.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links this
module; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.

What it computes is the plain definition of the method, token by token, in float64
(numpy), with no blocking, chunking or reordering:

* Inputs are packed varlen ``[T, H, D]`` (batch 1) with ``cu_seqlens`` bounds, raw
  pre-activation gate and beta, and a V-first recurrent state
  (aiter PR 4741, "[FlyDSL] Add gfx950 Kimi Delta Attention prefill kernel", Summary).
* Pre-processing folded into the prefill: q/k L2 normalisation, the lower-bounded
  sigmoid gate ``g = lower_bound * sigmoid(g_raw)`` per key channel with
  ``lower_bound = -5`` by default, and ``beta = sigmoid(beta_raw)`` per token-head
  (same page, Optimizations Applied: the fused pack kernel and the 160-nat remark).
* The gated delta rule with per-key-channel decay, state ``S`` in R^{V x K}:
  ``S_t = S_{t-1} Diag(exp g_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T`` and
  ``o_t = scale * S_t q_t``, evaluated as decay, then the delta update with the
  token's own gate, then the read-out.
* State modes: a dense initial/final state ``[N, H, V, K]``, or a paged pool
  ``[slots, H, V, K]`` addressed by ``state_indices`` where ``has_initial_state``
  false starts from zero without reading the slot (aiter PR 5754, Technical Details).
  Any stored state dtype is upcast exactly; accumulation is in float64
  (aiter PR 5249, What).

Readings where the pages say nothing (each listed with its reason in the design notes):
* L2 norm: ``x / sqrt(sum(x^2) + eps)`` with ``eps = 1e-6`` so that a zero padding
  row normalises to zero rather than NaN.
* The gate has no further terms (no per-head A_log / dt_bias / softplus); a caller
  folds any affine pre-transform into ``g_raw``.
* An empty sequence's final state equals its initial state and is written back.
* Grouped value heads (GVA, named for the default pipeline in aiter PR 5754,
  Technical Details): when q and k carry fewer heads (H_qk) than v (H), value head h
  reads q/k head ``h // (H / H_qk)``, i.e. each q/k head serves a run of consecutive
  value heads, as ``repeat_interleave`` along the head axis would lay them out.
* K-first state (same passage; the final-state shape switch between ``(N, H, V, K)``
  and ``(N, H, K, V)`` in the code under review on aiter PR 5249): a stored plane
  ``[K, V]`` is the transpose of the V-first ``[V, K]`` one; the recurrence is unchanged.

Chunk numbering (aiter PR 6912, Changes and Tests): chunks are numbered by their
sequence's position in ``cu_seqlens``; the reference for that numbering is a
``repeat_interleave`` over the per-sequence chunk counts, given here with numpy.
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + e^-x) in float64; +-inf map to 1 and 0."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def l2_normalize(x: np.ndarray, eps: float = L2_EPS) -> np.ndarray:
    """Row-wise ``x / sqrt(sum(x^2) + eps)`` over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def kda_sequence(q, k, v, g_raw, beta_raw, S0, scale, lower_bound, eps=L2_EPS):
    """Run the recurrence over one sequence, all heads at once.

    q, k, g_raw: [L, H, K]; v: [L, H, V]; beta_raw: [L, H]; S0: [H, V, K].
    Returns (o [L, H, V], S_final [H, V, K]) in float64.
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    L = q.shape[0]
    H, V, K = S.shape
    out = np.empty((L, H, V), dtype=np.float64)
    qn = l2_normalize(q, eps)
    kn = l2_normalize(k, eps)
    g = lower_bound * sigmoid(g_raw)  # [L, H, K], per key channel, in (lower_bound, 0)
    beta = sigmoid(beta_raw)  # [L, H]
    decay = np.exp(g)
    for t in range(L):
        S *= decay[t][:, None, :]  # S <- S Diag(e^{g_t}): column c scaled by e^{g_t[c]}
        Sk = np.einsum("hvk,hk->hv", S, kn[t])
        delta = beta[t][:, None] * (v[t] - Sk)  # delta_t = beta_t (v_t - S' k_t)
        S += delta[:, :, None] * kn[t][:, None, :]  # S <- S' + delta_t k_t^T
        out[t] = scale * np.einsum("hvk,hk->hv", S, qn[t])  # o_t = scale S_t q_t
    return out, S


def kda_forward(
    q, k, v, g_raw, beta_raw, cu_seqlens, *, scale, lower_bound,
    initial_state=None, state_cache=None, state_indices=None, has_initial_state=None,
    state_k_first=False, eps=L2_EPS, seqs=None,
):
    """Whole-call oracle over a packed varlen batch.

    Arrays are float64 numpy (exact upcasts of the stored values):
    q, k ``[T, H_qk, K]``; v ``[T, H, V]``; g_raw ``[T, H, K]``; beta_raw ``[T, H]``;
    cu_seqlens ``[N+1]`` ints. H_qk divides H; value head h reads q/k head
    ``h // (H / H_qk)`` (H_qk = H: one q/k head per value head).

    State, one mode at a time:
      * dense: ``initial_state [N, H, V, K]`` (None means zero);
      * paged: ``state_cache [slots, H, V, K]`` with ``state_indices [N]`` and
        ``has_initial_state [N]``; a false flag starts from zero and the slot is
        not read;
      * neither: zero initial state.
    With ``state_k_first`` every stored plane is ``[K, V]`` instead of ``[V, K]``.

    ``seqs`` restricts the work to a subset of sequence ids (for sampled checks).

    Returns ``(out, finals)``: ``out [T, H, V]`` (rows of sequences outside ``seqs``
    are NaN) and ``finals`` a dict ``seq -> final state``, laid out like the stored
    state: ``[H, V, K]``, or ``[H, K, V]`` with ``state_k_first``.
    """
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    N = len(cu) - 1
    T, H, V = v.shape
    H_qk, K = q.shape[1], q.shape[2]
    if H % H_qk != 0 or k.shape[1] != H_qk:
        raise ValueError("q and k must have the same head count, dividing v's")
    if H_qk != H:  # each q/k head serves H / H_qk consecutive value heads
        q = np.repeat(q, H // H_qk, axis=1)
        k = np.repeat(k, H // H_qk, axis=1)

    def to_math(plane):  # stored plane(s) -> [.., V, K]
        plane = np.asarray(plane, dtype=np.float64)
        return np.swapaxes(plane, -1, -2) if state_k_first else plane

    out = np.full((T, H, V), np.nan, dtype=np.float64)
    finals = {}
    if initial_state is not None and state_cache is not None:
        raise ValueError("dense initial_state and a paged state_cache are exclusive")
    for n in (range(N) if seqs is None else seqs):
        a, b = cu[n], cu[n + 1]
        if state_cache is not None:
            if bool(has_initial_state[n]):
                S0 = to_math(state_cache[int(state_indices[n])])
            else:
                S0 = np.zeros((H, V, K))
        elif initial_state is not None:
            S0 = to_math(initial_state[n])
        else:
            S0 = np.zeros((H, V, K))
        o, S = kda_sequence(q[a:b], k[a:b], v[a:b], g_raw[a:b], beta_raw[a:b], S0,
                            scale, lower_bound, eps)
        out[a:b] = o
        finals[n] = np.ascontiguousarray(np.swapaxes(S, -1, -2)) if state_k_first else S
    return out, finals


def chunk_indices(cu_seqlens, chunk: int):
    """Chunk table ``[(seq, chunk_in_seq), ...]`` numbered by position in cu_seqlens.

    Per-sequence chunk counts are ``ceil(len / chunk)`` (zero for an empty sequence);
    sequence ids are ``repeat(arange(N), counts)`` and the in-sequence index is the
    global position minus the repeated exclusive prefix of the counts.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.diff(cu)
    counts = (lens + chunk - 1) // chunk
    seq = np.repeat(np.arange(len(lens), dtype=np.int64), counts)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]) if len(counts) else np.zeros(0, np.int64)
    within = np.arange(int(counts.sum()), dtype=np.int64) - np.repeat(starts, counts)
    return np.stack([seq, within], axis=1).astype(np.int32)
