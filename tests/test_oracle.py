"""Pins for the fp64 oracle: each check ties it to something other than itself.

* brute force: an independent 50-digit evaluation of the closed product form of the
  recurrence on tiny inputs (K != V so that a transposed operand cannot pass);
* closed forms: T = 1, beta = 0, g = 0 with basis keys, zero initial state;
* invariants: zero padding rows are a no-op, resume equals one call, contraction
  with v = 0, exact homogeneity in (S0, v);
* the chunkwise form (with the bounded reference-row factorisation) equals the token
  recurrence for several chunk sizes and at 640 nats per chunk;
* chunk numbering equals a plain loop over sequences, including empty ones.
"""
import math

import mpmath as mp
import numpy as np
import pytest

from oracle import chunk_indices, kda_forward, kda_sequence
from tests import chunk_model

mp.mp.dps = 50


def _rand_case(rng, L, H, K, V, gscale=1.0):
    q = rng.standard_normal((L, H, K))
    k = rng.standard_normal((L, H, K))
    v = rng.standard_normal((L, H, V))
    graw = rng.standard_normal((L, H, K)) * gscale
    braw = rng.standard_normal((L, H))
    S0 = 0.1 * rng.standard_normal((H, V, K))
    return q, k, v, graw, braw, S0


# ---------------------------------------------------------------- brute force (mpmath)
def _mp_norm(x, eps):
    s = mp.fsum([mp.mpf(float(a)) ** 2 for a in x])
    return [mp.mpf(float(a)) / mp.sqrt(s + mp.mpf(eps)) for a in x]


def _mp_sig(x):
    return 1 / (1 + mp.e ** (-mp.mpf(float(x))))


def _brute_force_head(q, k, v, graw, braw, S0, scale, lb, eps=1e-6):
    """Closed product form, evaluated independently for every t (no recurrence).

    With M_s = Diag(e^{g_s}) (I - beta_s k_s k_s^T):
      S_t = S0 M_1 ... M_t + sum_{s<=t} beta_s v_s k_s^T M_{s+1} ... M_t,
      o_t = scale S_t q_t.
    """
    L, K = q.shape
    V = v.shape[1]
    qs = [mp.matrix(_mp_norm(q[t], eps)) for t in range(L)]
    ks = [mp.matrix(_mp_norm(k[t], eps)) for t in range(L)]
    betas = [_mp_sig(braw[t]) for t in range(L)]
    Ms = []
    for t in range(L):
        D = mp.diag([mp.e ** (mp.mpf(lb) * _mp_sig(graw[t][c])) for c in range(K)])
        Ms.append(D * (mp.eye(K) - betas[t] * ks[t] * ks[t].T))
    S0m = mp.matrix(S0.tolist())

    def prod(a, b):  # M_a ... M_b (inclusive, 0-based); identity if a > b
        P = mp.eye(K)
        for s in range(a, b + 1):
            P = P * Ms[s]
        return P

    outs = np.zeros((L, V))
    S_t = None
    for t in range(L):
        S_t = S0m * prod(0, t)
        for s in range(t + 1):
            vs = mp.matrix(v[s].tolist())
            S_t = S_t + betas[s] * vs * ks[s].T * prod(s + 1, t)
        o = S_t * qs[t] * mp.mpf(scale)
        outs[t] = [float(o[i]) for i in range(V)]
    S_final = np.array([[float(S_t[i, j]) for j in range(K)] for i in range(V)]) if L else S0
    return outs, S_final


@pytest.mark.parametrize("seed,L,K,V,lb", [(0, 7, 4, 3, -5.0), (1, 10, 3, 5, -1.0), (2, 12, 4, 4, -20.0)])
def test_brute_force_single_sequence(seed, L, K, V, lb):
    rng = np.random.default_rng(seed)
    q, k, v, graw, braw, S0 = _rand_case(rng, L, 2, K, V)
    scale = 1.0 / math.sqrt(K)
    o, S = kda_sequence(q, k, v, graw, braw, S0, scale, lb)
    for h in range(2):
        ob, Sb = _brute_force_head(q[:, h], k[:, h], v[:, h], graw[:, h], braw[:, h], S0[h], scale, lb)
        assert np.max(np.abs(o[:, h] - ob)) <= 1e-12 * max(1.0, np.max(np.abs(ob)))
        assert np.max(np.abs(S[h] - Sb)) <= 1e-12 * max(1.0, np.max(np.abs(Sb)))


def test_brute_force_varlen_with_empty_and_paged():
    """Three sequences (one empty) through a paged pool with mixed flags."""
    rng = np.random.default_rng(7)
    K, V, H = 4, 3, 1
    lens = [5, 0, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, graw, braw, _ = _rand_case(rng, T, H, K, V)
    pool = rng.standard_normal((6, H, V, K))
    idx = np.array([4, 0, 2])
    flags = np.array([True, True, False])
    pool[2] = np.nan  # flag false: must not be read
    scale = 0.5
    out, finals = kda_forward(q, k, v, graw, braw, cu, scale=scale, lower_bound=-5.0,
                              state_cache=pool, state_indices=idx, has_initial_state=flags)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        S0 = pool[idx[n], 0] if flags[n] else np.zeros((V, K))
        ob, Sb = _brute_force_head(q[a:b, 0], k[a:b, 0], v[a:b, 0], graw[a:b, 0], braw[a:b, 0], S0,
                                   scale, -5.0)
        assert np.allclose(out[a:b, 0], ob, rtol=0, atol=1e-12)
        assert np.allclose(finals[n][0], Sb, rtol=0, atol=1e-12)
        assert not np.any(np.isnan(finals[n]))
    # The empty sequence's final state is its initial state.
    assert np.array_equal(finals[1][0], pool[0, 0])


def test_brute_force_grouped_value_heads():
    """Two q/k heads serving six value heads (three each): value head h reads q/k head
    h // 3. With H_qk = 2 and groups of 3, h // 3 and h % 3 pick different heads for
    every h but 0, so a swapped index cannot pass."""
    rng = np.random.default_rng(21)
    K, V, L, H, H_qk = 4, 3, 6, 6, 2
    q = rng.standard_normal((L, H_qk, K))
    k = rng.standard_normal((L, H_qk, K))
    v = rng.standard_normal((L, H, V))
    graw = rng.standard_normal((L, H, K))
    braw = rng.standard_normal((L, H))
    S0 = 0.1 * rng.standard_normal((1, H, V, K))
    cu = np.array([0, L])
    out, finals = kda_forward(q, k, v, graw, braw, cu, scale=0.5, lower_bound=-5.0, initial_state=S0)
    for h in range(H):
        j = h // (H // H_qk)
        ob, Sb = _brute_force_head(q[:, j], k[:, j], v[:, h], graw[:, h], braw[:, h], S0[0, h], 0.5, -5.0)
        assert np.max(np.abs(out[:, h] - ob)) <= 1e-12
        assert np.max(np.abs(finals[0][h] - Sb)) <= 1e-12


def test_grouped_heads_must_divide():
    rng = np.random.default_rng(22)
    q = rng.standard_normal((2, 4, 4))
    v = rng.standard_normal((2, 6, 4))
    with pytest.raises(ValueError):
        kda_forward(q, q, v, rng.standard_normal((2, 6, 4)), rng.standard_normal((2, 6)), [0, 2],
                    scale=1.0, lower_bound=-5.0)


def test_brute_force_k_first_state():
    """K-first planes [K, V]: the stored initial state is read as its transpose and the
    final state is written back transposed; checked against the brute force on a
    rectangular K != V plane, through a paged pool with mixed flags."""
    rng = np.random.default_rng(23)
    K, V, H = 5, 3, 2
    lens = [4, 0, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, graw, braw, _ = _rand_case(rng, T, H, K, V)
    pool = rng.standard_normal((4, H, K, V))  # K-first planes
    idx = np.array([3, 1, 0])
    flags = np.array([True, True, False])
    pool[0] = np.nan  # flag false: must not be read
    out, finals = kda_forward(q, k, v, graw, braw, cu, scale=0.4, lower_bound=-5.0, state_cache=pool,
                              state_indices=idx, has_initial_state=flags, state_k_first=True)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        assert finals[n].shape == (H, K, V)
        for h in range(H):
            S0 = pool[idx[n], h].T if flags[n] else np.zeros((V, K))
            ob, Sb = _brute_force_head(q[a:b, h], k[a:b, h], v[a:b, h], graw[a:b, h], braw[a:b, h], S0, 0.4, -5.0)
            assert np.allclose(out[a:b, h], ob, rtol=0, atol=1e-12)
            assert np.allclose(finals[n][h], Sb.T, rtol=0, atol=1e-12)
    assert np.array_equal(finals[1], pool[1])  # empty sequence: stored plane round-trips


# ---------------------------------------------------------------- closed forms
def test_closed_form_single_token():
    """T=1: o = scale [S0 (e^g * q^) + beta (v - S0 (e^g * k^)) (k^ . q^)]."""
    rng = np.random.default_rng(11)
    K, V, H = 6, 5, 3
    q, k, v, graw, braw, S0 = _rand_case(rng, 1, H, K, V)
    scale, lb = 0.3, -5.0
    o, S = kda_sequence(q, k, v, graw, braw, S0, scale, lb)
    for h in range(H):
        qn = q[0, h] / np.sqrt(q[0, h] @ q[0, h] + 1e-6)
        kn = k[0, h] / np.sqrt(k[0, h] @ k[0, h] + 1e-6)
        eg = np.exp(lb / (1 + np.exp(-graw[0, h])))
        b = 1 / (1 + np.exp(-braw[0, h]))
        expect = scale * (S0[h] @ (eg * qn) + b * (v[0, h] - S0[h] @ (eg * kn)) * (kn @ qn))
        assert np.max(np.abs(o[0, h] - expect)) <= 1e-15 * max(1, np.max(np.abs(expect))) * 10
        expect_S = (S0[h] * eg[None, :]) + np.outer(b * (v[0, h] - S0[h] @ (eg * kn)), kn)
        assert np.max(np.abs(S[h] - expect_S)) <= 1e-14


def test_closed_form_beta_zero_pure_decay():
    """beta = 0: the state only decays, S_T = S0 Diag(e^{sum g}), o_t = scale S0 e^{G_t} q^_t."""
    rng = np.random.default_rng(12)
    K, V, H, L = 5, 4, 2, 9
    q, k, v, graw, braw, S0 = _rand_case(rng, L, H, K, V)
    braw[:] = -np.inf
    lb = -3.0
    o, S = kda_sequence(q, k, v, graw, braw, S0, 1.0, lb)
    g = lb / (1 + np.exp(-graw))
    G = np.cumsum(g, axis=0)
    for h in range(H):
        assert np.allclose(S[h], S0[h] * np.exp(G[-1, h])[None, :], rtol=1e-13, atol=0)
        for t in range(L):
            qn = q[t, h] / np.sqrt(q[t, h] @ q[t, h] + 1e-6)
            assert np.allclose(o[t, h], S0[h] @ (np.exp(G[t, h]) * qn), rtol=1e-12, atol=1e-15)


def test_closed_form_identity_gate_unit_beta_basis_keys():
    """g = 0, beta = 1, k = e_i: column i of the state is replaced by v (up to eps)."""
    rng = np.random.default_rng(13)
    K, V, H = 4, 3, 1
    order = [2, 0, 3, 2, 1]
    L = len(order)
    q = rng.standard_normal((L, H, K))
    k = np.zeros((L, H, K))
    for t, i in enumerate(order):
        k[t, 0, i] = 1.0
    v = rng.standard_normal((L, H, V))
    graw = np.full((L, H, K), -np.inf)
    braw = np.full((L, H), np.inf)
    S0 = rng.standard_normal((H, V, K))
    o, S = kda_sequence(q, k, v, graw, braw, S0, 1.0, -5.0)
    expect = S0[0].copy()
    for t, i in enumerate(order):
        expect[:, i] = v[t, 0]
    # k^ = e_i / sqrt(1 + 1e-6): column replacement holds to ~1e-6 relative.
    assert np.max(np.abs(S[0] - expect)) <= 3e-6 * np.max(np.abs(expect))


def test_closed_form_zero_state_single_token():
    """S0 = 0, T = 1: o = scale beta (k^ . q^) v."""
    rng = np.random.default_rng(14)
    K, V, H = 8, 6, 2
    q, k, v, graw, braw, _ = _rand_case(rng, 1, H, K, V)
    o, _ = kda_sequence(q, k, v, graw, braw, np.zeros((H, V, K)), 0.7, -5.0)
    for h in range(H):
        qn = q[0, h] / np.sqrt(q[0, h] @ q[0, h] + 1e-6)
        kn = k[0, h] / np.sqrt(k[0, h] @ k[0, h] + 1e-6)
        b = 1 / (1 + np.exp(-braw[0, h]))
        assert np.allclose(o[0, h], 0.7 * b * (kn @ qn) * v[0, h], rtol=1e-13, atol=0)


# ---------------------------------------------------------------- invariants
def test_padding_rows_are_exact_noop():
    """Rows with q = k = v = 0, raw gate = raw beta = -inf leave everything unchanged."""
    rng = np.random.default_rng(21)
    K = V = 16
    H, L = 2, 11
    q, k, v, graw, braw, S0 = _rand_case(rng, L, H, K, V)
    o, S = kda_sequence(q, k, v, graw, braw, S0, 0.25, -5.0)
    ins = [0, 4, 4, 11]  # positions in the original sequence before which to insert
    keep = []
    rows = []
    for t in range(L + 1):
        for _ in range(ins.count(t)):
            rows.append(None)
        if t < L:
            keep.append(len(rows))
            rows.append(t)
    Lp = len(rows)
    qp = np.zeros((Lp, H, K)); kp = np.zeros((Lp, H, K)); vp = np.zeros((Lp, H, V))
    gp = np.full((Lp, H, K), -np.inf); bp = np.full((Lp, H), -np.inf)
    for j, t in enumerate(rows):
        if t is not None:
            qp[j], kp[j], vp[j], gp[j], bp[j] = q[t], k[t], v[t], graw[t], braw[t]
    op, Sp = kda_sequence(qp, kp, vp, gp, bp, S0, 0.25, -5.0)
    assert np.array_equal(op[keep], o)
    assert np.array_equal(Sp, S)


def test_resume_equals_single_call():
    rng = np.random.default_rng(22)
    q, k, v, graw, braw, S0 = _rand_case(rng, 20, 2, 8, 8)
    o, S = kda_sequence(q, k, v, graw, braw, S0, 0.3, -5.0)
    o1, S1 = kda_sequence(q[:7], k[:7], v[:7], graw[:7], braw[:7], S0, 0.3, -5.0)
    o2, S2 = kda_sequence(q[7:], k[7:], v[7:], graw[7:], braw[7:], S1, 0.3, -5.0)
    assert np.array_equal(np.concatenate([o1, o2]), o)
    assert np.array_equal(S2, S)


def test_contraction_with_zero_values():
    """v = 0: each step multiplies S by Diag(e^g)(I - beta k k^T), of norm <= 1."""
    rng = np.random.default_rng(23)
    q, k, v, graw, braw, S0 = _rand_case(rng, 40, 3, 8, 6, gscale=3.0)
    v[:] = 0
    S = S0.copy()
    prev = np.linalg.norm(S.reshape(3, -1), axis=1)
    for t in range(40):
        _, S = kda_sequence(q[t:t + 1], k[t:t + 1], v[t:t + 1], graw[t:t + 1], braw[t:t + 1], S, 1.0, -0.5)
        cur = np.linalg.norm(S.reshape(3, -1), axis=1)
        assert np.all(cur <= prev * (1 + 1e-15))
        prev = cur


def test_homogeneity_exact_in_powers_of_two():
    rng = np.random.default_rng(24)
    q, k, v, graw, braw, S0 = _rand_case(rng, 13, 2, 8, 8)
    o, S = kda_sequence(q, k, v, graw, braw, S0, 0.3, -5.0)
    o2, S2 = kda_sequence(q, k, 4.0 * v, graw, braw, 4.0 * S0, 0.3, -5.0)
    assert np.array_equal(o2, 4.0 * o)
    assert np.array_equal(S2, 4.0 * S)


def test_has_initial_state_false_equals_zero_dense_state():
    rng = np.random.default_rng(25)
    q, k, v, graw, braw, _ = _rand_case(rng, 9, 2, 4, 4)
    cu = np.array([0, 4, 9])
    pool = np.full((3, 2, 4, 4), np.nan)
    o_p, f_p = kda_forward(q, k, v, graw, braw, cu, scale=0.5, lower_bound=-5.0, state_cache=pool,
                           state_indices=np.array([2, 0]), has_initial_state=np.array([False, False]))
    o_d, f_d = kda_forward(q, k, v, graw, braw, cu, scale=0.5, lower_bound=-5.0,
                           initial_state=np.zeros((2, 2, 4, 4)))
    assert np.array_equal(o_p, o_d)
    for n in range(2):
        assert np.array_equal(f_p[n], f_d[n])


def test_gate_and_beta_ranges():
    """g = lb * sigmoid(raw) lies in (lb, 0); sigmoid(0) = 1/2 gives exactly lb/2."""
    from oracle import sigmoid
    x = np.array([-50.0, -3.0, 0.0, 3.0, 50.0])
    s = sigmoid(x)
    assert s[2] == 0.5
    assert np.all((s >= 0) & (s <= 1))
    assert np.all(np.diff(s) > 0) or np.all(np.diff(s) >= 0)
    assert sigmoid(np.array([-np.inf]))[0] == 0.0 and sigmoid(np.array([np.inf]))[0] == 1.0


# ---------------------------------------------------------------- chunk form == token form
@pytest.mark.parametrize("C", [1, 4, 16, 32, 64])
@pytest.mark.parametrize("lb", [-5.0, -20.0])
def test_chunk_form_equals_oracle(C, lb):
    rng = np.random.default_rng(31 + C)
    K = V = 16
    H, L = 2, 75  # ragged: not a multiple of any C > 1 here
    q, k, v, graw, braw, S0 = _rand_case(rng, L, H, K, V)
    graw += 6.0 if lb == -20.0 else 0.0  # saturated gates: ~20 nats per token at lb = -20
    o, S = kda_sequence(q, k, v, graw, braw, S0, 0.25, lb)
    for rb in sorted({1, min(C, chunk_model.ref_block_for(lb))}):
        if C % rb:
            continue
        oc, Sc, tiles = chunk_model.chunk_sequence(q, k, v, graw, braw, S0, 0.25, lb, C=C, ref_block=rb,
                                                   return_tiles=True)
        assert np.max(np.abs(oc - o)) <= 1e-12 * max(1, np.max(np.abs(o)))
        assert np.max(np.abs(Sc - S)) <= 1e-12 * max(1, np.max(np.abs(S)))
        # No factor of the reference-row construction exceeds e^80, and no left factor
        # falls below e^-80 (fp32 and bf16 both hold e^{+-87}).
        assert max(t["max_pos"] for ch in tiles for t in ch) <= 80.0 + 1e-9
        assert min(t["min_left"] for ch in tiles for t in ch) >= -80.0 - 1e-9
        assert np.all(np.isfinite(oc))


def test_chunk_affine_map():
    """Each chunk acts on the state as S -> S M + B (the basis for segmenting a scan)."""
    rng = np.random.default_rng(41)
    K = V = 8
    q, k, v, graw, braw, S0 = _rand_case(rng, 32, 1, K, V)
    _, S, tiles = chunk_model.chunk_sequence(q, k, v, graw, braw, S0, 0.3, -5.0, C=32, return_tiles=True)
    M, B = chunk_model.affine_chunk_map(tiles[0][0])
    assert np.max(np.abs(S0[0] @ M + B - S[0])) <= 1e-13


def test_ref_block_choice():
    assert chunk_model.ref_block_for(-5.0) == 16
    assert chunk_model.ref_block_for(-20.0) == 4
    assert chunk_model.ref_block_for(-60.0) == 2
    assert chunk_model.ref_block_for(-100.0) == 1


# ---------------------------------------------------------------- chunk numbering
def _loop_chunk_table(cu, chunk):
    out = []
    for n in range(len(cu) - 1):
        length = cu[n + 1] - cu[n]
        j = 0
        while j * chunk < length:
            out.append((n, j))
            j += 1
    return np.array(out, dtype=np.int32).reshape(-1, 2)


@pytest.mark.parametrize("lens", [[5, 0, 64, 33], [0, 0, 1], [32], [0], [31, 32, 33, 0, 0, 100]])
def test_chunk_indices_number_empty_sequences(lens):
    cu = np.concatenate([[0], np.cumsum(lens)])
    assert np.array_equal(chunk_indices(cu, 32), _loop_chunk_table(cu, 32))
