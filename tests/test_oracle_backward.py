"""Pins for the oracle's chunk-form backward (``oracle.chunk_backward``).

``token_backward`` (autograd of the token recurrence) is pinned to central
differences of an independently written loss in test_oracle_pins.py; here the
chunk form is checked against it, against a closed form, and its
intermediates against what they mean:
* every gradient equals token_backward's, both gates, ragged T, several chunk
  sizes, with and without h0 and dhT;
* beta = 0 (the state only decays): closed forms for dq, dk, dv, dbeta's
  absence of a delta term, dh0 and dg;
* dhe[c], the gradient of chunk c's end state, is the dh0 of the backward of
  the remaining tokens started from that state (token_backward on the
  suffix), and dv = beta * dR.
A slip in the chunk algebra (a decay on the wrong side, a dropped term of the
gate gradient, T where T^T belongs) moves one of these by far more than the
tolerance.
"""
import numpy as np
import pytest

pytest.importorskip("torch")


def _case(rng, B, T, H, K, V, per_key, h0=True, dhT=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    g = -rng.uniform(0.02, 0.6, (B, T, H, K) if per_key else (B, T, H))
    h0v = 0.3 * rng.standard_normal((B, H, K, V)) if h0 else None
    do = rng.standard_normal((B, T, H, V))
    dhTv = rng.standard_normal((B, H, K, V)) if dhT else None
    return q, k, v, beta, g, h0v, do, dhTv


NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("T,C,h0,dhT", [(13, 4, True, True), (16, 8, False, True),
                                        (11, 3, True, False), (7, 8, False, False)])
def test_chunk_backward_equals_token_backward(oracle_mod, per_key, T, C, h0, dhT):
    rng = np.random.default_rng(700 + T + C + 2 * per_key)
    q, k, v, beta, g, h0v, do, dhTv = _case(rng, 2, T, 2, 5, 4, per_key, h0, dhT)
    ref = oracle_mod.token_backward(q, k, v, beta, g, do, h0v, dhTv)
    got = oracle_mod.chunk_backward(q, k, v, beta, g, do, C, h0v, dhTv)
    for name, x, r in zip(NAMES, got[:6], ref):
        if r is None:
            assert x is None
            continue
        np.testing.assert_allclose(x, r, rtol=1e-10, atol=1e-12, err_msg=name)


def test_chunk_backward_beta_zero_closed_form(oracle_mod):
    """beta = 0: S_t = e^{G_t} S_0 (G_t the cumsum of g up to t), so
    o_t = e^{G_t} h0^T q_t and hT = e^{G_T} h0.  Then dq_t = e^{G_t} h0 do_t,
    dk = dv = 0, dh0 = sum_t e^{G_t} q_t do_t^T + e^{G_T} dhT and
    dg_j = sum_{t >= j} e^{G_t} q_t . (h0 do_t) + e^{G_T} <h0, dhT>."""
    rng = np.random.default_rng(711)
    q, k, v, beta, g, h0, do, dhT = _case(rng, 1, 10, 1, 4, 3, False)
    beta[:] = 0.0
    dq, dk, dv, db, dg, dh0, _ = oracle_mod.chunk_backward(q, k, v, beta, g, do, 4, h0, dhT)
    G = np.cumsum(g[0, :, 0])
    H0 = h0[0, 0]
    dq_ref = np.stack([np.exp(G[t]) * H0 @ do[0, t, 0] for t in range(10)])
    np.testing.assert_allclose(dq[0, :, 0], dq_ref, rtol=1e-12, atol=1e-14)
    assert np.abs(dk).max() < 1e-14 and np.abs(dv).max() < 1e-14
    dh0_ref = sum(np.exp(G[t]) * np.outer(q[0, t, 0], do[0, t, 0]) for t in range(10)) + np.exp(G[-1]) * dhT[0, 0]
    np.testing.assert_allclose(dh0[0, 0], dh0_ref, rtol=1e-12, atol=1e-14)
    per_t = np.array([np.exp(G[t]) * q[0, t, 0] @ (H0 @ do[0, t, 0]) for t in range(10)])
    dg_ref = np.cumsum(per_t[::-1])[::-1] + np.exp(G[-1]) * np.sum(H0 * dhT[0, 0])
    np.testing.assert_allclose(dg[0, :, 0], dg_ref, rtol=1e-12, atol=1e-14)
    # dbeta is the delta's weight: (v_t - S~_t k_t) . (the state gradient's pull on it)
    assert np.isfinite(db).all()


@pytest.mark.parametrize("per_key", [False, True])
def test_chunk_backward_intermediates(oracle_mod, per_key):
    """dhe[c] is the dh0 of the suffix after chunk c started from that
    chunk's end state; the last is dhT.  dv = beta * dR."""
    rng = np.random.default_rng(721 + per_key)
    T, C = 17, 4
    q, k, v, beta, g, h0, do, dhT = _case(rng, 1, T, 2, 4, 3, per_key)
    *_, extra = oracle_mod.chunk_backward(q, k, v, beta, g, do, C, h0, dhT)
    dhe, dR = extra["dhe"], extra["dR"]
    NT = (T + C - 1) // C
    assert dhe.shape == (1, NT, 2, 4, 3)
    np.testing.assert_allclose(dhe[:, -1], dhT, rtol=0, atol=0)
    _, _, hck, _ = oracle_mod.token_states(q.astype(np.float32), k.astype(np.float32),
                                           v.astype(np.float32), beta.astype(np.float32),
                                           g.astype(np.float32), C, h0.astype(np.float32))
    # the state at chunk c's end is the checkpoint of chunk c + 1; redo the
    # checkpoints in fp64 from the fp32-rounded inputs the C oracle saw
    f = lambda x: x.astype(np.float32).astype(np.float64)
    q, k, v, beta, g, h0, do = (f(x) for x in (q, k, v, beta, g, h0, do))
    *_, extra = oracle_mod.chunk_backward(q, k, v, beta, g, do, C, h0, dhT)
    dhe, dR = extra["dhe"], extra["dR"]
    for c in range(NT - 1):
        e = (c + 1) * C
        sl = lambda x: x[:, e:]
        ref = oracle_mod.token_backward(sl(q), sl(k), sl(v), sl(beta), sl(g), sl(do),
                                        hck[:, c + 1], dhT)
        np.testing.assert_allclose(dhe[:, c], ref[5], rtol=1e-7, atol=1e-9, err_msg="chunk %d" % c)
    dv = oracle_mod.chunk_backward(q, k, v, beta, g, do, C, h0, dhT)[2]
    np.testing.assert_allclose(dv, beta[..., None] * dR, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("per_key", [False, True])
def test_chunk_backward_with_the_exact_saved_states(oracle_mod, per_key):
    """Handed the exact chunk-start states and deltas (token_states), the
    chunk backward gives token_backward's gradients; handed rounded ones it
    moves by about the rounding."""
    rng = np.random.default_rng(731 + per_key)
    T, C = 14, 4
    q, k, v, beta, g, h0, do, dhT = _case(rng, 1, T, 2, 4, 3, per_key)
    f = lambda x: x.astype(np.float32).astype(np.float64)
    q, k, v, beta, g, h0 = (f(x) for x in (q, k, v, beta, g, h0))
    _, _, hck, vnew = oracle_mod.token_states(q.astype(np.float32), k.astype(np.float32),
                                              v.astype(np.float32), beta.astype(np.float32),
                                              g.astype(np.float32), C, h0.astype(np.float32))
    ref = oracle_mod.token_backward(q, k, v, beta, g, do, h0, dhT)
    got = oracle_mod.chunk_backward(q, k, v, beta, g, do, C, h0, dhT, hck=hck, vnew=vnew)
    for name, x, r in zip(NAMES, got[:6], ref):
        np.testing.assert_allclose(x, r, rtol=1e-9, atol=1e-11, err_msg=name)
    rnd = oracle_mod.chunk_backward(q, k, v, beta, g, do, C, h0, dhT, hck=hck.astype(np.float16),
                                    vnew=vnew.astype(np.float16))
    moved = max(oracle_mod.rel_err(x, r) for x, r in zip(rnd[:2], ref[:2]))
    assert 1e-5 < moved < 1e-2
