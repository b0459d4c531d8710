"""Pins for the fp64 oracle, checked against things other than itself.

The pages print no worked example for this method, so the oracle is pinned by
exact brute force, closed forms and invariants of the recurrence
S_t = S_{t-1} Diag(a_t)(I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t
(Gated DeltaNet / KDA forward).  Each pin is chosen so that a plausible slip in
the oracle (a dropped decay, a flipped sign, q and k swapped, the decay on the
wrong index, the correction before the decay, a transposed state) fails it;
``test_planted_mistakes_are_caught`` plants those slips in copies of the C
source and checks that the suite below catches each of them.
"""
import math
import os
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------------------
# Exact brute force: products of (I - b k k^T) written out in rationals.
# ---------------------------------------------------------------------------

def _mat(rows, cols, val=Fraction(0)):
    return [[val for _ in range(cols)] for _ in range(rows)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0))
             for j in range(p)] for i in range(n)]


def _transition(a, b, k):
    """A_t = Diag(a)(I - b k k^T), K x K, acting on S from the right."""
    K = len(k)
    return [[a[i] * ((1 if i == j else 0) - b * k[i] * k[j]) for j in range(K)]
            for i in range(K)]


def brute_force(q, k, v, beta, a, S0):
    """S_t = S_0 prod_{j<=t} A_j + sum_{s<=t} b_s v_s k_s^T prod_{s<j<=t} A_j.

    All arguments are Fractions; a[t] is the K-vector of gate factors.  Returns
    (o [T][V], S_T [V][K]) exactly.  This is the unrolled closed form of the
    recurrence, not the oracle's step-by-step update.
    """
    T, K, V = len(q), len(q[0]), len(v[0])
    A = [_transition(a[t], beta[t], k[t]) for t in range(T)]
    outs, S_t = [], None
    for t in range(T):
        P = [[Fraction(int(i == j)) for j in range(K)] for i in range(K)]
        for j in range(t + 1):
            P = _matmul(P, A[j])
        S_t = _matmul(S0, P)
        for s in range(t + 1):
            R = [[Fraction(int(i == j)) for j in range(K)] for i in range(K)]
            for j in range(s + 1, t + 1):
                R = _matmul(R, A[j])
            outer = [[beta[s] * v[s][i] * k[s][j] for j in range(K)]
                     for i in range(V)]
            contrib = _matmul(outer, R)
            S_t = [[S_t[i][j] + contrib[i][j] for j in range(K)] for i in range(V)]
        outs.append([sum((S_t[i][j] * q[t][j] for j in range(K)), Fraction(0))
                     for i in range(V)])
    return outs, S_t


def _small_case(rng, T, K, V, per_key, with_h0=True):
    """Random fp32-exact inputs, shaped [1,T,1,*] as the oracle expects."""
    def r(*shape, scale=1.0):
        return (rng.standard_normal(shape) * scale).astype(np.float32)
    q, k, v = r(1, T, 1, K), r(1, T, 1, K, scale=0.6), r(1, T, 1, V)
    beta = (1 / (1 + np.exp(-r(1, T, 1)))).astype(np.float32)
    gs = (1, T, 1, K) if per_key else (1, T, 1)
    g = (-np.log1p(np.exp(-(r(*gs) + 1.0)))).astype(np.float32)
    h0 = r(1, 1, K, V, scale=0.5) if with_h0 else None
    return q, k, v, beta, g, h0


def _to_frac(x):
    return [[Fraction(float(e)) for e in row] for row in x]


@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("T,K,V", [(1, 2, 3), (4, 3, 2), (6, 4, 3)])
def test_exact_bruteforce(oracle_mod, per_key, T, K, V):
    rng = np.random.default_rng(100 + 7 * T + K + (50 if per_key else 0))
    q, k, v, beta, g, h0 = _small_case(rng, T, K, V, per_key)
    o, hT = oracle_mod.token_recurrence(q, k, v, beta, g, h0, nthreads=1)
    # the same gate factors the C oracle forms: libm exp of the fp32 gate
    if per_key:
        a = [[Fraction(math.exp(float(g[0, t, 0, d]))) for d in range(K)]
             for t in range(T)]
    else:
        a = [[Fraction(math.exp(float(g[0, t, 0])))] * K for t in range(T)]
    S0 = [[Fraction(float(h0[0, 0, i, j])) for i in range(K)] for j in range(V)]
    o_ex, S_ex = brute_force(_to_frac(q[0, :, 0]), _to_frac(k[0, :, 0]),
                             _to_frac(v[0, :, 0]),
                             [Fraction(float(b)) for b in beta[0, :, 0]], a, S0)
    o_ex = np.array([[float(x) for x in row] for row in o_ex])
    hT_ex = np.array([[float(S_ex[j][i]) for j in range(V)] for i in range(K)])
    np.testing.assert_allclose(o[0, :, 0], o_ex, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hT[0, 0], hT_ex, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Closed forms and textbook special cases.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("per_key", [False, True])
def test_beta_zero_is_pure_decay(oracle_mod, per_key):
    """beta = 0: S_t = S_0 Diag(exp(sum_{j<=t} g_j)), o_t = S_t q_t."""
    rng = np.random.default_rng(1)
    T, K, V = 9, 5, 3
    q, k, v, beta, g, h0 = _small_case(rng, T, K, V, per_key)
    beta[:] = 0
    o, hT = oracle_mod.token_recurrence(q, k, v, beta, g, h0, nthreads=1)
    G = np.cumsum(g[0, :, 0].astype(np.float64), axis=0)       # [T] or [T,K]
    dec = np.exp(G) if per_key else np.exp(G)[:, None] * np.ones((1, K))
    H0 = h0[0, 0].astype(np.float64)
    for t in range(T):
        Ht = dec[t][:, None] * H0                                # K x V
        np.testing.assert_allclose(o[0, t, 0], Ht.T @ q[0, t, 0], rtol=1e-12,
                                   atol=1e-14)
    np.testing.assert_allclose(hT[0, 0], dec[-1][:, None] * H0, rtol=1e-12)


def test_orthonormal_keys_reduce_to_linear_attention(oracle_mod):
    """g = 0, beta = 1, orthonormal k, S_0 = 0: plain DeltaNet writes each v
    exactly, so S_T = sum_s v_s k_s^T and o_t = sum_{s<=t} (k_s . q_t) v_s."""
    rng = np.random.default_rng(2)
    T, K, V = 6, 8, 5
    Q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Q[:T].astype(np.float32)              # rows: nearly orthonormal in fp32
    q = rng.standard_normal((T, K)).astype(np.float32)
    v = rng.standard_normal((T, V)).astype(np.float32)
    beta = np.ones((1, T, 1), np.float32)
    g = np.zeros((1, T, 1), np.float32)
    o, hT = oracle_mod.token_recurrence(q[None, :, None], k[None, :, None],
                                        v[None, :, None], beta, g, None,
                                        nthreads=1)
    k64, q64, v64 = k.astype(np.float64), q.astype(np.float64), v.astype(np.float64)
    scores = np.tril(q64 @ k64.T)             # [t, s], s <= t
    np.testing.assert_allclose(o[0, :, 0], scores @ v64, atol=2e-6)
    np.testing.assert_allclose(hT[0, 0], k64.T @ v64, atol=2e-6)


@pytest.mark.parametrize("per_key", [False, True])
def test_unit_key_query_equal_reads_back_value(oracle_mod, per_key):
    """beta = 1, |k| = 1 and q = k: the update writes v_t at k_t, so o_t = v_t
    whatever the gate and the history."""
    rng = np.random.default_rng(3)
    T, K, V = 12, 8, 4
    k = np.zeros((1, T, 1, K), np.float32)
    for t in range(T):                        # entries +-1/2 on 4 slots: |k| = 1
        idx = rng.choice(K, 4, replace=False)
        k[0, t, 0, idx] = rng.choice([-0.5, 0.5], 4)
    v = rng.standard_normal((1, T, 1, V)).astype(np.float32)
    beta = np.ones((1, T, 1), np.float32)
    gs = (1, T, 1, K) if per_key else (1, T, 1)
    g = (-rng.random(gs)).astype(np.float32)
    h0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    o, _ = oracle_mod.token_recurrence(k, k, v, beta, g, h0, nthreads=1)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], atol=1e-12)


def test_per_key_gate_uniform_equals_scalar_gate(oracle_mod):
    rng = np.random.default_rng(4)
    T, K, V = 20, 6, 7
    q, k, v, beta, g, h0 = _small_case(rng, T, K, V, False)
    gk = np.repeat(g[..., None], K, axis=-1)
    o1, h1 = oracle_mod.token_recurrence(q, k, v, beta, g, h0, nthreads=1)
    o2, h2 = oracle_mod.token_recurrence(q, k, v, beta, gk, h0, nthreads=1)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(h1, h2)


@pytest.mark.parametrize("per_key", [False, True])
def test_state_passing_splits_the_sequence(oracle_mod, per_key):
    rng = np.random.default_rng(5)
    T, K, V, T1 = 30, 6, 5, 13
    q, k, v, beta, g, h0 = _small_case(rng, T, K, V, per_key)
    o, hT = oracle_mod.token_recurrence(q, k, v, beta, g, h0, nthreads=1)
    sl = lambda x, a, b: np.ascontiguousarray(x[:, a:b])
    oa, ha = oracle_mod.token_recurrence(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1),
                                         sl(beta, 0, T1), sl(g, 0, T1), h0,
                                         nthreads=1)
    ob, hb = oracle_mod.token_recurrence(sl(q, T1, T), sl(k, T1, T), sl(v, T1, T),
                                         sl(beta, T1, T), sl(g, T1, T),
                                         ha.astype(np.float32), nthreads=1)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, atol=1e-6)
    np.testing.assert_allclose(hb, hT, atol=1e-6)


@pytest.mark.parametrize("per_key", [False, True])
def test_linear_in_values_and_initial_state(oracle_mod, per_key):
    rng = np.random.default_rng(6)
    T, K, V = 17, 5, 4
    q, k, v, beta, g, h0 = _small_case(rng, T, K, V, per_key)
    v2 = rng.standard_normal(v.shape).astype(np.float32)
    h2 = rng.standard_normal(h0.shape).astype(np.float32)
    oa, ha = oracle_mod.token_recurrence(q, k, v, beta, g, h0, nthreads=1)
    ob, hb = oracle_mod.token_recurrence(q, k, v2, beta, g, h2, nthreads=1)
    os_, hs = oracle_mod.token_recurrence(q, k, v + v2, beta, g, h0 + h2,
                                          nthreads=1)
    # v + v2 and h0 + h2 are rounded to fp32; compare against the same sums
    np.testing.assert_allclose(os_, oa + ob, atol=1e-5)
    np.testing.assert_allclose(hs, ha + hb, atol=1e-5)


def test_threads_and_head_selection_agree(oracle_mod):
    rng = np.random.default_rng(7)
    B, T, H, K, V = 2, 11, 3, 4, 5
    q = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k = (0.5 * rng.standard_normal((B, T, H, K))).astype(np.float32)
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    beta = rng.random((B, T, H)).astype(np.float32)
    g = (-rng.random((B, T, H))).astype(np.float32)
    h0 = rng.standard_normal((B, H, K, V)).astype(np.float32)
    o1, h1 = oracle_mod.token_recurrence(q, k, v, beta, g, h0, nthreads=1)
    o4, h4 = oracle_mod.token_recurrence(q, k, v, beta, g, h0, nthreads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(h1, h4)
    # a head taken alone sees only its own slice of the [B,T,H,*] layout
    sel = [4, 1]
    os_, hs = oracle_mod.token_recurrence(q, k, v, beta, g, h0, heads=sel)
    for n, bh in enumerate(sel):
        b, h = divmod(bh, H)
        np.testing.assert_array_equal(os_[n], o1[b, :, h])
        np.testing.assert_array_equal(hs[n], h1[b, h])
        one = oracle_mod.token_recurrence(
            q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1],
            beta[b:b + 1, :, h:h + 1], g[b:b + 1, :, h:h + 1], h0[b:b + 1, h:h + 1])
        np.testing.assert_array_equal(one[0][0, :, 0], o1[b, :, h])


def test_empty_sequence_returns_initial_state(oracle_mod):
    rng = np.random.default_rng(8)
    K, V = 4, 3
    z = lambda *s: np.zeros(s, np.float32)
    h0 = rng.standard_normal((1, 2, K, V)).astype(np.float32)
    o, hT = oracle_mod.token_recurrence(z(1, 0, 2, K), z(1, 0, 2, K), z(1, 0, 2, V),
                                        z(1, 0, 2), z(1, 0, 2), h0)
    assert o.shape == (1, 0, 2, V)
    np.testing.assert_array_equal(hT, h0)


# ---------------------------------------------------------------------------
# Chunk form (prepare + scan): pinned to the token recurrence and to closed
# forms of the WY factors.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("chunk,T", [(16, 64), (32, 70), (64, 130), (64, 1),
                                     (16, 16)])
def test_chunk_form_equals_token_recurrence(oracle_mod, per_key, chunk, T):
    rng = np.random.default_rng(9 + T + chunk)
    B, H, K, V = 1, 2, 12, 8
    q = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    beta = rng.random((B, T, H)).astype(np.float32)
    gs = (B, T, H, K) if per_key else (B, T, H)
    g = (-0.3 * rng.random(gs)).astype(np.float32)
    h0 = rng.standard_normal((B, H, K, V)).astype(np.float32)
    o_ref, h_ref = oracle_mod.token_recurrence(q, k, v, beta, g, h0)
    o, hT = oracle_mod.chunk_forward(q, k, v, beta, g, chunk, h0)
    np.testing.assert_allclose(o, o_ref, atol=1e-10)
    np.testing.assert_allclose(hT, h_ref, atol=1e-10)


def test_chunk_size_does_not_change_the_result(oracle_mod):
    rng = np.random.default_rng(10)
    B, T, H, K, V = 1, 96, 1, 8, 8
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K)) / 3
    v = rng.standard_normal((B, T, H, V))
    beta = rng.random((B, T, H))
    g = -rng.random((B, T, H))
    outs = [oracle_mod.chunk_forward(q, k, v, beta, g, c) for c in (8, 32, 96)]
    for o, h in outs[1:]:
        np.testing.assert_allclose(o, outs[0][0], atol=1e-10)
        np.testing.assert_allclose(h, outs[0][1], atol=1e-10)


def test_prepare_orthogonal_keys_closed_form(oracle_mod):
    """Mutually orthogonal keys inside a chunk make the Gram term vanish, so
    the inverse is the identity: w = beta exp(gamma) k and u = beta v."""
    rng = np.random.default_rng(11)
    T, K, V, C = 8, 8, 3, 8
    k = np.eye(K)[rng.permutation(K)][None, :, None, :] * 0.5
    v = rng.standard_normal((1, T, 1, V))
    beta = rng.random((1, T, 1))
    g = -rng.random((1, T, 1))
    gcum, w, u = oracle_mod.chunk_prepare(k, v, beta, g, C)
    gam = np.cumsum(g[0, :, 0])
    np.testing.assert_allclose(gcum[0, :, 0], gam, atol=1e-15)
    np.testing.assert_allclose(w[0, :, 0], (beta[0, :, 0] * np.exp(gam))[:, None]
                               * k[0, :, 0], atol=1e-15)
    np.testing.assert_allclose(u[0, :, 0], beta[0, :, 0][:, None] * v[0, :, 0],
                               atol=1e-15)


def test_prepare_two_token_chunk_by_hand(oracle_mod):
    """Two tokens: A = [[0,0],[a,0]] with a = b2 (k2.k1) e^{g2}; the inverse is
    [[1,0],[-a,1]], so w2 = b2 e^{g1+g2} k2 - a b1 e^{g1} k1, u2 = b2 v2 - a b1 v1."""
    k1, k2 = np.array([0.6, 0.8, 0.0]), np.array([0.0, 0.6, 0.8])
    v1, v2 = np.array([1.0, -2.0]), np.array([0.5, 3.0])
    b1, b2, g1, g2 = 0.25, 0.75, -0.5, -0.125
    k = np.stack([k1, k2])[None, :, None]
    v = np.stack([v1, v2])[None, :, None]
    beta = np.array([b1, b2])[None, :, None]
    g = np.array([g1, g2])[None, :, None]
    gcum, w, u = oracle_mod.chunk_prepare(k, v, beta, g, 2)
    a = b2 * (k2 @ k1) * math.exp(g2)
    np.testing.assert_allclose(gcum[0, :, 0], [g1, g1 + g2], atol=1e-15)
    np.testing.assert_allclose(w[0, 0, 0], b1 * math.exp(g1) * k1, atol=1e-15)
    np.testing.assert_allclose(w[0, 1, 0], b2 * math.exp(g1 + g2) * k2
                               - a * b1 * math.exp(g1) * k1, atol=1e-15)
    np.testing.assert_allclose(u[0, 0, 0], b1 * v1, atol=1e-15)
    np.testing.assert_allclose(u[0, 1, 0], b2 * v2 - a * b1 * v1, atol=1e-15)


def test_scan_with_zero_wy_is_gated_linear_readout(oracle_mod):
    """w = u = 0 makes v' = 0, leaving o_t = (q_t e^{gamma_t}) h and the state
    only decays; with a per-key gate the decay is per row of h."""
    rng = np.random.default_rng(12)
    T, K, V, C = 10, 4, 3, 5
    q = rng.standard_normal((1, T, 1, K))
    k = rng.standard_normal((1, T, 1, K))
    gk = -rng.random((1, T, 1, K))
    gam = np.concatenate([np.cumsum(gk[0, :5, 0], 0), np.cumsum(gk[0, 5:, 0], 0)])
    h0 = rng.standard_normal((1, 1, K, V))
    z = np.zeros((1, T, 1, K)), np.zeros((1, T, 1, V))
    o, hT = oracle_mod.chunk_scan(q, k, z[0], z[1], gam[None, :, None], C, h0)
    H = h0[0, 0]
    H5 = np.exp(gam[4])[:, None] * H
    for t in range(T):
        Hs = H if t < 5 else H5
        np.testing.assert_allclose(o[0, t, 0], (q[0, t, 0] * np.exp(gam[t])) @ Hs,
                                   atol=1e-14)
    np.testing.assert_allclose(hT[0, 0], np.exp(gam[9])[:, None] * H5, atol=1e-14)


def test_rel_err_definition(oracle_mod):
    ref = np.array([3.0, -4.0])               # rms = sqrt(12.5)
    assert oracle_mod.rel_err(np.array([3.5, -4.0]), ref) == pytest.approx(
        0.5 / math.sqrt(12.5))


# ---------------------------------------------------------------------------
# Saved states: the chunk-start state h_c and the per-token delta v_new that a
# backward pass re-reads (the KDA re-scan page's h checkpoints and v_new).
# ---------------------------------------------------------------------------

def brute_force_states(q, k, v, beta, a, S0):
    """Every state S_t (V x K) of the unrolled product form, t = -1 .. T-1."""
    T, K, V = len(q), len(q[0]), len(v[0])
    A = [_transition(a[t], beta[t], k[t]) for t in range(T)]
    states = [S0]
    for t in range(T):
        P = [[Fraction(int(i == j)) for j in range(K)] for i in range(K)]
        for j in range(t + 1):
            P = _matmul(P, A[j])
        S_t = _matmul(S0, P)
        for s in range(t + 1):
            R = [[Fraction(int(i == j)) for j in range(K)] for i in range(K)]
            for j in range(s + 1, t + 1):
                R = _matmul(R, A[j])
            outer = [[beta[s] * v[s][i] * k[s][j] for j in range(K)]
                     for i in range(V)]
            contrib = _matmul(outer, R)
            S_t = [[S_t[i][j] + contrib[i][j] for j in range(K)] for i in range(V)]
        states.append(S_t)
    return states


@pytest.mark.parametrize("per_key", [False, True])
def test_states_exact_bruteforce(oracle_mod, per_key, T=5, K=3, V=2, chunk=2):
    """h_c is S^T just before token c*C; v_new_t is what token t adds to the
    decayed state along k_t: S_t = S_{t-1} Diag(a_t) + v_new_t k_t^T, which
    expands the product form to v_new_t = b_t (v_t - S_{t-1} Diag(a_t) k_t).
    Both from exact rational states of the unrolled product (T = 5 leaves a
    ragged last chunk)."""
    rng = np.random.default_rng(300 + (1 if per_key else 0))
    q, k, v, beta, g, h0 = _small_case(rng, T, K, V, per_key)
    o, hT, hck, vnew = oracle_mod.token_states(q, k, v, beta, g, chunk, h0, nthreads=1)
    assert hck.shape == (1, (T + chunk - 1) // chunk, 1, K, V)
    assert vnew.shape == (1, T, 1, V)
    if per_key:
        a = [[Fraction(math.exp(float(g[0, t, 0, d]))) for d in range(K)]
             for t in range(T)]
    else:
        a = [[Fraction(math.exp(float(g[0, t, 0])))] * K for t in range(T)]
    S0 = [[Fraction(float(h0[0, 0, i, j])) for i in range(K)] for j in range(V)]
    kf, vf = _to_frac(k[0, :, 0]), _to_frac(v[0, :, 0])
    bf = [Fraction(float(b)) for b in beta[0, :, 0]]
    states = brute_force_states(_to_frac(q[0, :, 0]), kf, vf, bf, a, S0)
    for c in range(hck.shape[1]):
        S = states[c * chunk]                       # S_{c C - 1}
        ex = np.array([[float(S[j][i]) for j in range(V)] for i in range(K)])
        np.testing.assert_allclose(hck[0, c, 0], ex, rtol=1e-12, atol=1e-13)
    for t in range(T):
        S = states[t]                               # S_{t-1}
        pred = [sum((S[i][d] * a[t][d] * kf[t][d] for d in range(K)), Fraction(0))
                for i in range(V)]
        ex = np.array([float(bf[t] * (vf[t][i] - pred[i])) for i in range(V)])
        np.testing.assert_allclose(vnew[0, t, 0], ex, rtol=1e-12, atol=1e-13)
    # o and hT are those of the plain recurrence
    o2, h2 = oracle_mod.token_recurrence(q, k, v, beta, g, h0, nthreads=1)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(hT, h2)


@pytest.mark.parametrize("per_key", [False, True])
def test_state_deltas_rebuild_the_next_checkpoint(oracle_mod, per_key):
    """Unrolling S_t = S_{t-1} Diag(a_t) + v_new_t k_t^T over a chunk:
    h_{c+1} = Diag(prod a) h_c + sum_t Diag(prod_{j>t} a_j) k_t v_new_t^T,
    and the same sum over the last chunk gives hT."""
    rng = np.random.default_rng(301)
    T, K, V, C = 23, 6, 4, 8
    q, k, v, beta, g, h0 = _small_case(rng, T, K, V, per_key)
    _, hT, hck, vnew = oracle_mod.token_states(q, k, v, beta, g, C, h0, nthreads=1)
    gg = g[0, :, 0].astype(np.float64)
    if not per_key:
        gg = gg[:, None] * np.ones((1, K))
    kk = k[0, :, 0].astype(np.float64)
    NT = hck.shape[1]
    for c in range(NT):
        s, e = c * C, min(c * C + C, T)
        h = np.exp(gg[s:e].sum(0))[:, None] * hck[0, c, 0]
        for t in range(s, e):
            h += np.outer(np.exp(gg[t + 1:e].sum(0)) * kk[t], vnew[0, t, 0])
        nxt = hck[0, c + 1, 0] if c + 1 < NT else hT[0, 0]
        np.testing.assert_allclose(h, nxt, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("per_key", [False, True])
def test_states_beta_zero(oracle_mod, per_key):
    """beta = 0: nothing is written (v_new = 0) and h_c is h0 decayed by the
    gates of the first c*C tokens."""
    rng = np.random.default_rng(302)
    T, K, V, C = 13, 4, 3, 4
    q, k, v, beta, g, h0 = _small_case(rng, T, K, V, per_key)
    beta[:] = 0
    _, _, hck, vnew = oracle_mod.token_states(q, k, v, beta, g, C, h0, nthreads=1)
    assert np.all(vnew == 0)
    G = np.concatenate([np.zeros((1,) + g.shape[3:]),
                        np.cumsum(g[0, :, 0].astype(np.float64), axis=0)])
    for c in range(hck.shape[1]):
        d = np.exp(G[c * C])
        d = d if per_key else d * np.ones(K)
        np.testing.assert_allclose(hck[0, c, 0], d[:, None] * h0[0, 0], rtol=1e-12)


@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("chunk,T", [(16, 64), (32, 70), (64, 1)])
def test_chunk_form_states_equal_token_states(oracle_mod, per_key, chunk, T):
    """v' = u - w h of the chunk form is the token recurrence's v_new, and
    the chunk scan's chunk-start states are its checkpoints."""
    rng = np.random.default_rng(303 + T + chunk)
    B, H, K, V = 1, 2, 12, 8
    q = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    beta = rng.random((B, T, H)).astype(np.float32)
    gs = (B, T, H, K) if per_key else (B, T, H)
    g = (-0.3 * rng.random(gs)).astype(np.float32)
    h0 = rng.standard_normal((B, H, K, V)).astype(np.float32)
    _, _, hck, vnew = oracle_mod.token_states(q, k, v, beta, g, chunk, h0)
    _, _, hck2, vnew2 = oracle_mod.chunk_forward(q, k, v, beta, g, chunk, h0, states=True)
    np.testing.assert_allclose(hck2, hck, atol=1e-10)
    np.testing.assert_allclose(vnew2, vnew, atol=1e-10)


def test_states_head_selection(oracle_mod):
    rng = np.random.default_rng(304)
    B, T, H, K, V, C = 2, 9, 3, 4, 5, 4
    q = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k = (0.5 * rng.standard_normal((B, T, H, K))).astype(np.float32)
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    beta = rng.random((B, T, H)).astype(np.float32)
    g = (-rng.random((B, T, H))).astype(np.float32)
    h0 = rng.standard_normal((B, H, K, V)).astype(np.float32)
    _, _, hck, vnew = oracle_mod.token_states(q, k, v, beta, g, C, h0, nthreads=3)
    sel = [5, 0]
    _, _, hs, vs = oracle_mod.token_states(q, k, v, beta, g, C, h0, heads=sel)
    for n, bh in enumerate(sel):
        b, h = divmod(bh, H)
        np.testing.assert_array_equal(hs[n], hck[b, :, h])
        np.testing.assert_array_equal(vs[n], vnew[b, :, h])


# ---------------------------------------------------------------------------
# Planted mistakes: each slip below, made in a copy of the C oracle, must be
# caught by the pins above (run on small inputs).
# ---------------------------------------------------------------------------

_MUTANTS = {
    "drop_decay": ("hr[j] *= ad;", ""),
    "flip_error_sign": ("e[j] -= hr[j] * kd;", "e[j] += hr[j] * kd;"),
    "correct_before_decay_order": (
        "hr[j] *= ad;\n                e[j] -= hr[j] * kd;",
        "e[j] -= hr[j] * kd;\n                hr[j] *= ad;"),
    "query_as_key": ("const double bk = bt * kk[d], qd = qq[d];",
                     "const double bk = bt * kk[d], qd = kk[d];"),
    "readout_before_update": ("hr[j] += bk * e[j];\n                if (ot) ot[j] += hr[j] * qd;",
                              "if (ot) ot[j] += hr[j] * qd;\n                hr[j] += bk * e[j];"),
    "drop_beta": ("const double bk = bt * kk[d]", "const double bk = kk[d]"),
    "gate_not_exponentiated": ("a[d] = exp((double)gt[d]);", "a[d] = 1.0 + (double)gt[d];"),
    "per_key_gate_on_value_index": ("hr[j] *= ad;", "hr[j] *= a[j % K];"),
    "state_delta_without_beta": ("vn[j] = bt * e[j];", "vn[j] = e[j];"),
    "checkpoint_one_token_late": ("t % J->chunk == 0", "t % J->chunk == 1 % J->chunk"),
}


def _pins_pass(mod):
    """Run a cheap subset of the pins against a (possibly mutated) module."""
    checks = [
        lambda: [test_exact_bruteforce(mod, pk, 4, 3, 2) for pk in (False, True)],
        lambda: [test_beta_zero_is_pure_decay(mod, pk) for pk in (False, True)],
        lambda: test_orthonormal_keys_reduce_to_linear_attention(mod),
        lambda: [test_unit_key_query_equal_reads_back_value(mod, pk)
                 for pk in (False, True)],
        lambda: [test_states_exact_bruteforce(mod, pk) for pk in (False, True)],
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_planted_mistakes_are_caught(oracle_mod, name, tmp_path):
    import importlib.util
    src = open(oracle_mod._SRC).read()
    old, new = _MUTANTS[name]
    assert old in src, "mutation anchor missing: %s" % name
    mut_dir = tmp_path / "oracle_mut"
    mut_dir.mkdir()
    (mut_dir / "gdn_oracle.c").write_text(src.replace(old, new, 1))
    init = open(os.path.join(os.path.dirname(oracle_mod._SRC), "__init__.py")).read()
    (mut_dir / "__init__.py").write_text(init)
    spec = importlib.util.spec_from_file_location(
        "oracle_mut_" + name, str(mut_dir / "__init__.py"),
        submodule_search_locations=[str(mut_dir)])
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build(force=True)
    assert not _pins_pass(mod), "planted mistake %r was not caught" % name
    # the unmutated oracle passes the same subset
    assert _pins_pass(oracle_mod)


@pytest.mark.parametrize("per_key", [False, True])
def test_rescan_dq_with_state_deltas_is_the_autograd_dq(oracle_mod, per_key):
    """dq of L = sum_t o_t . do_t by autograd of a plain fp64 torch loop
    equals, token by token, the chunk-start term rescan_dq (raw) under the
    gate decay plus the in-chunk writes:
        dq_t = e^{G_t} (h_c do_t) + sum_{s <= t in chunk} e^{G_t - G_s} k_s (vnew_s . do_t)
    with G the chunk-local cumsum (per key column for the per-key gate)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(401)
    T, K, V, C = 19, 5, 3, 6
    q, k, v, beta, g, h0 = _small_case(rng, T, K, V, per_key)
    do = rng.standard_normal((1, T, 1, V)).astype(np.float32)
    _, _, hck, vnew = oracle_mod.token_states(q, k, v, beta, g, C, h0, nthreads=1)
    dq_raw = oracle_mod.rescan_dq(hck, do, C)

    f64 = lambda x: torch.tensor(np.asarray(x, np.float64))
    qt = f64(q[0, :, 0]).requires_grad_(True)
    kt, vt, bt, gt = f64(k[0, :, 0]), f64(v[0, :, 0]), f64(beta[0, :, 0]), f64(g[0, :, 0])
    S = f64(h0[0, 0]).T.clone()                                  # S = h^T, V x K
    loss = 0.0
    for t in range(T):
        a = torch.exp(gt[t])
        S = S * a                                                 # per key column (or scalar)
        e = vt[t] - S @ kt[t]
        S = S + bt[t] * torch.outer(e, kt[t])
        loss = loss + (S @ qt[t]) @ f64(do[0, t, 0])
    loss.backward()
    dq = qt.grad.numpy()

    gg = g[0, :, 0].astype(np.float64)
    if not per_key:
        gg = gg[:, None] * np.ones((1, K))
    kk = k[0, :, 0].astype(np.float64)
    dd = do[0, :, 0].astype(np.float64)
    for t in range(T):
        s0 = (t // C) * C
        G = np.cumsum(gg[s0:t + 1], axis=0)                       # G[j] = sum up to s0 + j
        x = np.exp(G[-1]) * dq_raw[0, t, 0]
        for s in range(s0, t + 1):
            x += np.exp(G[-1] - G[s - s0]) * kk[s] * (vnew[0, s, 0] @ dd[t])
        np.testing.assert_allclose(x, dq[t], rtol=1e-9, atol=1e-11)


def _np_loss(q, k, v, beta, g, h0, do, dhT):
    """L = sum_t o_t . do_t + sum hT * dhT by a plain numpy fp64 loop, written
    apart from the oracle's (independent of its C and torch code)."""
    q, k, v, beta, g, h0, do, dhT = (np.asarray(x, np.float64) for x in (q, k, v, beta, g, h0, do, dhT))
    B, T, H, K = q.shape
    L = 0.0
    for b in range(B):
        for h in range(H):
            S = h0[b, h].T.copy()
            for t in range(T):
                S = S * np.exp(g[b, t, h])               # scalar, or per key column
                e = v[b, t, h] - S @ k[b, t, h]
                S = S + beta[b, t, h] * np.outer(e, k[b, t, h])
                L += (S @ q[b, t, h]) @ do[b, t, h]
            L += np.sum(S.T * dhT[b, h])
    return L


@pytest.mark.parametrize("per_key", [False, True])
def test_token_backward_matches_finite_differences(oracle_mod, per_key):
    """Every gradient of token_backward against central differences of an
    independently written loss (step 1e-5 in fp64: error ~1e-10)."""
    pytest.importorskip("torch")
    rng = np.random.default_rng(503 + per_key)
    B, T, H, K, V = 1, 6, 2, 3, 2
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    g = -rng.uniform(0.05, 0.5, (B, T, H, K) if per_key else (B, T, H))
    h0 = 0.3 * rng.standard_normal((B, H, K, V))
    do = rng.standard_normal((B, T, H, V))
    dhT = rng.standard_normal((B, H, K, V))
    grads = oracle_mod.token_backward(q, k, v, beta, g, do, h0, dhT)
    args = [q, k, v, beta, g, h0]
    eps = 1e-5
    for i, (x, gx) in enumerate(zip(args, grads)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap = list(args); ap[i] = xp
            am = list(args); am[i] = xm
            fd[idx] = (_np_loss(*ap, do, dhT) - _np_loss(*am, do, dhT)) / (2 * eps)
        np.testing.assert_allclose(gx, fd, rtol=1e-6, atol=1e-8, err_msg="input %d" % i)


def test_token_backward_forward_value_is_the_recurrence(oracle_mod):
    """The loss token_backward differentiates is the C recurrence's: with
    do = one-hot and no dhT, dq at that token is S_t^T e_j (row j of S_t),
    and the C oracle's o_t = S_t q_t, so dq_t . q_t = o_t[j]."""
    pytest.importorskip("torch")
    rng = np.random.default_rng(509)
    B, T, H, K, V = 1, 5, 1, 4, 3
    q = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k = rng.standard_normal((B, T, H, K)).astype(np.float32)
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (B, T, H)).astype(np.float32)
    g = -rng.uniform(0.05, 0.5, (B, T, H)).astype(np.float32)
    h0 = (0.3 * rng.standard_normal((B, H, K, V))).astype(np.float32)
    o, _ = oracle_mod.token_recurrence(q, k, v, beta, g, h0)
    for t in range(T):
        for j in range(V):
            do = np.zeros((B, T, H, V))
            do[0, t, 0, j] = 1.0
            dq = oracle_mod.token_backward(q, k, v, beta, g, do, h0)[0]
            assert abs(dq[0, t, 0] @ q[0, t, 0].astype(np.float64) - o[0, t, 0, j]) < 1e-10
