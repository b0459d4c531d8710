"""CPU model of how the kernels split the chunk's decays, at ordinary and
strong gates.

Inside a chunk the decayed products need e^(gcum_r - gcum_s) for s <= r,
which is at most 1 for any gate g <= 0.  A matrix-core product can only take
such a factor as a row factor times a column factor, and those two must not
overflow where their product is a decay.  The kernels therefore:

* off the diagonal (16-row tiles I > J) split the exponent at the boundary
  after block J, which lies between every r of block I and s of block J:
  e^(gcum_r - gend_J) * e^(gend_J - gcum_s), both factors <= 1;
* on a diagonal tile take each entry's decay e^(gcum_r - gcum_s) directly
  (scalar gate), or split it at the boundary between r and s found by halving
  the 16-row block (per-key gate), again both factors <= 1.

These tests compute the factors in float32 exactly as the kernels form them,
build A and P from them, run the rest of the chunk form in fp64 and compare
with the fp64 token recurrence (the oracle).  With exact factors the bar is
the fp32-io one, 1e-4: a float32 cumsum of gates that reach hundreds in
magnitude carries ~1e-5 of absolute error into each exponent.  The previous
split (at the first row of each 16-row block, or around the chunk's middle
row) is modelled beside it to show that these gates break it: the tests
fail on a model that lets a growth factor into a product (inf and NaN reach
A, which then makes the triangular solve fail or the output non-finite).
"""
import numpy as np
import pytest

import oracle
from chunked_gated_delta_prepare_amd.inputs import make_inputs

F32 = np.float32


# ---------------------------------------------------------------------------
# gate recipes: the workloads' logsigmoid(N(0,1) + bias) at lower biases, a
# key channel pinned at g = -20, sparse hard resets, and a scalar gate near -8
# ---------------------------------------------------------------------------

def strong_inputs(B, T, H, K, V, gate, recipe, seed, io="fp32", h0=True):
    bias = {"b1": 1.0, "b0": 0.0, "bm2": -2.0, "m8": -8.0, "pin20": 3.0, "reset": 3.0}[recipe]
    inp = make_inputs(B, T, H, K, V, io=io, gate=gate, gate_bias=bias, h0=h0, seed=seed)
    g = inp["g"].numpy().copy()
    rng = np.random.default_rng(seed + 7777)
    if recipe == "pin20":
        g[..., :4] = -20.0                     # four key channels decay by e^-20 per token
    if recipe == "reset":
        hit = rng.random(g.shape) < 1.0 / 24.0
        g[hit] = -60.0                         # a hard forget now and then
    inp["g"] = __import__("torch").from_numpy(g)
    return inp


# ---------------------------------------------------------------------------
# the kernels' factors (float32), per chunk; gam is the chunk-local cumsum
# ---------------------------------------------------------------------------

def decay_split_scalar(gam):
    """E[r, s] as the scalar-gate kernels form it (float32)."""
    gam = gam.astype(F32)
    n = gam.shape[0]
    nb = (n + 15) // 16
    gpad = np.concatenate([gam, np.full(16 * nb - n, gam[-1], F32)])
    gend = gpad[15::16]                                     # gcum at each block's last row
    E = np.zeros((n, n), F32)
    with np.errstate(over="ignore", invalid="ignore"):
        for r in range(n):
            for s in range(r + 1):
                I, J = r // 16, s // 16
                if I == J:
                    E[r, s] = np.exp(np.minimum(gam[r] - gam[s], F32(0)))
                else:
                    efac = np.exp(np.minimum(gam[r] - gend[J], F32(0)))
                    einv = np.exp(gend[J] - gam[s])
                    E[r, s] = efac * einv
    return E


def decay_split_scalar_old(gam):
    """The previous split: referenced to the first row of s's block."""
    gam = gam.astype(F32)
    n = gam.shape[0]
    E = np.zeros((n, n), F32)
    with np.errstate(over="ignore", invalid="ignore"):
        for r in range(n):
            for s in range(r + 1):
                ref = gam[16 * (s // 16)]
                E[r, s] = np.exp(gam[r] - ref) * np.exp(ref - gam[s])
    return E


def split_point(r, s):
    """For s < r in one chunk: the boundary the per-key kernel splits their
    decay at, as the last row before it.  Off-diagonal 16-row blocks: the end
    of s's block; inside a 16-row block: the end of the half (quarter, ...)
    holding s at the first halving that separates r and s."""
    if r // 16 != s // 16:
        return 16 * (s // 16) + 15
    lo, size = 16 * (s // 16), 16
    while size > 1:
        half = size // 2
        if (r - lo) >= half > (s - lo):
            return lo + half - 1
        if (s - lo) >= half:
            lo += half
        size = half
    raise AssertionError("r and s coincide")


def decay_split_key(gam, fp16_operands=True):
    """Per-key E[r, s, d] = row factor * column factor around split_point,
    both <= 1, each rounded into the operand format (fp16: the factor times a
    unit-scale key or query; below fp16's smallest subnormal it flushes)."""
    gam = gam.astype(F32)
    n, K = gam.shape
    E = np.zeros((n, n, K), np.float64)
    for r in range(n):
        E[r, r] = 1.0
        for s in range(r):
            m = split_point(r, s)
            fr = np.exp(gam[r] - gam[m])                     # <= 1
            fc = np.exp(gam[m] - gam[s])                     # <= 1
            if fp16_operands:
                fr = fr.astype(np.float16).astype(np.float64)
                fc = fc.astype(np.float16).astype(np.float64)
            E[r, s] = fr * fc
    return E


def decay_split_key_old(gam):
    """The previous split: every row referenced to the chunk's middle row,
    factors rounded to fp16."""
    gam = gam.astype(F32)
    n, K = gam.shape
    m = n // 2 - 1
    with np.errstate(over="ignore", invalid="ignore"):
        up = np.exp(gam - gam[m]).astype(np.float16).astype(np.float64)
        dn = np.exp(gam[m] - gam).astype(np.float16).astype(np.float64)
        E = up[:, None, :] * dn[None, :, :]
    return E


# ---------------------------------------------------------------------------
# the chunk form with a given decay model; everything else exact (fp64)
# ---------------------------------------------------------------------------

def chunk_forward_with(q, k, v, beta, g, C, h0, decay):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    beta, g = np.asarray(beta, np.float64), np.asarray(g, np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    per_key = g.ndim == 4
    o = np.zeros((B, T, H, V))
    hT = np.zeros((B, H, K, V))
    for b in range(B):
        for hh in range(H):
            S = np.zeros((K, V)) if h0 is None else np.array(h0[b, hh], np.float64)
            for s0 in range(0, T, C):
                e0 = min(s0 + C, T)
                qc, kc, vc = q[b, s0:e0, hh], k[b, s0:e0, hh], v[b, s0:e0, hh]
                bc = beta[b, s0:e0, hh]
                gam = np.cumsum(g[b, s0:e0, hh], axis=0)
                E = decay(gam)
                if per_key:
                    G = np.einsum("rd,sd,rsd->rs", kc, kc, E)
                    P = np.einsum("rd,sd,rsd->rs", qc, kc, E)
                    ed, el = np.exp(gam), np.exp(gam[-1])
                    kx = kc * ed
                    qx = qc * ed
                    kg = kc * np.exp(gam[-1][None, :] - gam)
                else:
                    G = (kc @ kc.T) * E
                    P = (qc @ kc.T) * E
                    ed, el = np.exp(gam), np.exp(gam[-1])
                    kx, qx = kc * ed[:, None], qc * ed[:, None]
                    kg = kc * np.exp(gam[-1] - gam)[:, None]
                A = np.tril(bc[:, None] * G, -1)
                vp = np.linalg.solve(np.eye(e0 - s0) + A, bc[:, None] * (vc - kx @ S))
                o[b, s0:e0, hh] = qx @ S + np.tril(P) @ vp
                S = (el[:, None] if per_key else el) * S + kg.T @ vp
            hT[b, hh] = S
    return o, hT


def _run(inp, C, decay):
    f = lambda x: None if x is None else x.float().numpy()
    args = [f(inp[n]) for n in ("q", "k", "v", "beta", "g")]
    o_ref, h_ref = oracle.token_recurrence(*args, f(inp["h0"]))
    o, hT = chunk_forward_with(*args, C, f(inp["h0"]), decay)
    return o, hT, o_ref, h_ref


def _assert_close(o, hT, o_ref, h_ref, tol):
    assert np.isfinite(o).all() and np.isfinite(hT).all(), "non-finite output"
    ro, rh = oracle.rel_err(o, o_ref), oracle.rel_err(hT, h_ref)
    assert ro <= tol and rh <= tol, "o %.2e  hT %.2e" % (ro, rh)


# ---------------------------------------------------------------------------
# scalar gate
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("recipe,C", [("m8", 64), ("m8", 32), ("reset", 64)])
def test_scalar_gate_split_is_exact(recipe, C):
    inp = strong_inputs(1, 2 * C + 23, 2, 32, 16, "head", recipe, seed=31)
    E = lambda gam: decay_split_scalar(gam)
    _assert_close(*_run(inp, C, E), tol=1e-4)


def test_scalar_gate_factors_never_grow():
    rng = np.random.default_rng(5)
    for g in (np.full(64, -8.0), -np.abs(rng.normal(8, 3, 64)), np.where(rng.random(64) < 0.1, -100.0, -0.01)):
        gam = np.cumsum(g).astype(F32)
        gend = gam[15::16]
        for r in range(64):
            for s in range(r + 1):
                if r // 16 != s // 16:
                    assert gam[r] - gend[s // 16] <= 0 and gend[s // 16] - gam[s] <= 0


def test_old_scalar_split_overflows_at_g_minus_8():
    """The split at the first row of each block multiplies by a growth factor
    e^(sum of up to 15 gates): at g near -8 that overflows fp32 and the model
    of the old kernel fails the same check."""
    inp = strong_inputs(1, 96, 1, 32, 16, "head", "m8", seed=32)
    with pytest.raises((AssertionError, np.linalg.LinAlgError)):
        _assert_close(*_run(inp, 64, decay_split_scalar_old), tol=2e-2)


# ---------------------------------------------------------------------------
# per-key gate
# ---------------------------------------------------------------------------

def test_split_point_lies_between():
    for C in (32, 64):
        for r in range(C):
            for s in range(r):
                m = split_point(r, s)
                assert s <= m < r, (r, s, m)


@pytest.mark.parametrize("recipe", ["b1", "b0", "bm2", "pin20", "reset"])
@pytest.mark.parametrize("C", [64, 32])
def test_key_gate_split_is_exact(recipe, C):
    inp = strong_inputs(1, C + 19, 2, 32, 16, "key", recipe, seed=33)
    _assert_close(*_run(inp, C, lambda gam: decay_split_key(gam, fp16_operands=False)), tol=1e-4)


@pytest.mark.parametrize("recipe", ["b1", "b0", "bm2", "pin20", "reset"])
def test_key_gate_split_with_fp16_factors(recipe):
    """The factors rounded to fp16 (as operands are): finite and within the
    bf16-io bar."""
    inp = strong_inputs(1, 64 + 19, 2, 32, 16, "key", recipe, seed=34)
    _assert_close(*_run(inp, 64, lambda gam: decay_split_key(gam, fp16_operands=True)), tol=5e-3)


@pytest.mark.parametrize("recipe", ["b1", "b0"])
def test_old_key_split_breaks(recipe):
    """The middle-row reference with fp16 operands: growth factors up to
    e^(32 |g|) overflow fp16 at ordinary per-key decays."""
    inp = strong_inputs(1, 64 + 19, 2, 32, 16, "key", recipe, seed=35)
    with pytest.raises((AssertionError, np.linalg.LinAlgError)):
        _assert_close(*_run(inp, 64, decay_split_key_old), tol=2e-2)
