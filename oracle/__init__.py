"""fp64 CPU oracle for the chunked gated delta rule forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing here is part of the product: only the tests,
the smoke check and the CPU-baseline leg of the benchmark import this package.
It shares no code with the HIP library and never loads it.

These functions mirror the library entry points:

* ``token_recurrence`` -- the plain definition (C, fp64, one token at a time),
  the reference for ``gdn_forward``.  See ``gdn_oracle.c`` for the recurrence.
  ``token_states`` also records the per-chunk start states and the per-token
  state deltas, the reference for ``gdn_forward_states``; ``rescan_dq`` forms
  dq's chunk-start-state term from them, the reference for ``gdn_rescan_dq``
  and ``gdn_chunk_dq``.  ``token_backward`` differentiates the recurrence
  (every input's gradient), the reference for ``gdn_backward``;
  ``chunk_backward`` reaches the same gradients by the chunk form (a reverse
  scan of the state's gradient, then per-chunk products) and also returns
  that scan's intermediates.
* ``chunk_prepare`` -- the per-chunk WY factors (gate cumsum, the strictly lower
  decayed Gram matrix, its unit-triangular inverse, then w and u), the
  reference for ``gdn_prepare``.  Steps follow the TileOPs "Reuse P as beta
  tiles in gated deltanet fused prepare" page (the A_g build, the inverse held
  in S_shared, then w = A_g^-1 k_beta and u = A_g^-1 v_beta), with the gate
  factor folded into w as the chunk algebra requires (see ``chunk_prepare``).
* ``chunk_scan`` -- the serial inter-chunk scan given w, u and the cumsum, the
  reference for ``gdn_scan``.  Steps follow the per-chunk algebra in the
  docstring of the kernel_fun KDA re-scan page (bwd_scan.py, KdaB1ScanKernel):
  v' = u - w h, then h <- exp(gd) h + kg^T v', plus the output read-out.

All three work on numpy arrays in the library's layouts: q, k, w [B,T,H,K];
v, u, o [B,T,H,V]; beta [B,T,H]; g, gcum [B,T,H] (one gate per head) or
[B,T,H,K] (one gate per key dimension); h0, hT [B,H,K,V] with
hT[b,h,i,j] = S_T[j,i].
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into liboracle.so with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
             "-o", tmp, _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            i64, vp = ctypes.c_int64, ctypes.c_void_p
            f = lib.gdn_oracle_states_f64
            f.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                          vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, i64, vp, vp,
                          ctypes.c_int]
            f.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _recurrence(q, k, v, beta, g, h0, heads, nthreads, want_o, want_hT, chunk):
    q, k, v, beta, g = map(_f32, (q, k, v, beta, g))
    B, T, H, K = q.shape
    V = v.shape[-1]
    if k.shape != (B, T, H, K) or v.shape != (B, T, H, V):
        raise ValueError("q/k/v shapes disagree")
    if beta.shape != (B, T, H):
        raise ValueError("beta must be [B,T,H]")
    if g.shape == (B, T, H):
        per_key = 0
    elif g.shape == (B, T, H, K):
        per_key = 1
    else:
        raise ValueError("g must be [B,T,H] or [B,T,H,K]")
    h0c = None if h0 is None else _f32(h0)
    if h0c is not None and h0c.shape != (B, H, K, V):
        raise ValueError("h0 must be [B,H,K,V]")
    if heads is None:
        sel, n = None, B * H
    else:
        sel = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
        n = sel.size
    o = np.empty((n, T, V), np.float64) if want_o else None
    hT = np.empty((n, K, V), np.float64) if want_hT else None
    hck = vnew = None
    if chunk is not None:
        if chunk < 1:
            raise ValueError("chunk must be >= 1")
        hck = np.empty((n, (T + chunk - 1) // chunk, K, V), np.float64)
        vnew = np.empty((n, T, V), np.float64)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = _load().gdn_oracle_states_f64(
        B, T, H, K, V, per_key, ptr(q), ptr(k), ptr(v), ptr(beta), ptr(g),
        ptr(h0c), n, ptr(sel), ptr(o), ptr(hT), int(chunk or 0), ptr(hck),
        ptr(vnew), int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_states_f64 failed with code %d" % rc)
    if heads is None:
        if o is not None:
            o = o.reshape(B, H, T, V).transpose(0, 2, 1, 3)
        if hT is not None:
            hT = hT.reshape(B, H, K, V)
        if hck is not None:
            hck = hck.reshape(B, H, -1, K, V).transpose(0, 2, 1, 3, 4)
            vnew = vnew.reshape(B, H, T, V).transpose(0, 2, 1, 3)
    return o, hT, hck, vnew


def token_recurrence(q, k, v, beta, g, h0=None, heads=None, nthreads=None,
                     want_o=True, want_hT=True):
    """Token-by-token fp64 recurrence.

    Inputs are anything numpy can view as float32 holding the exact values the
    GPU sees (bf16 widens exactly).  ``heads`` optionally selects flat head
    indices b*H + h.  Returns ``(o, hT)`` as float64 arrays: with ``heads`` None
    they are [B,T,H,V] and [B,H,K,V]; otherwise head-major [n,T,V], [n,K,V].
    """
    o, hT, _, _ = _recurrence(q, k, v, beta, g, h0, heads, nthreads, want_o, want_hT, None)
    return o, hT


def token_states(q, k, v, beta, g, chunk, h0=None, heads=None, nthreads=None):
    """The token recurrence with the states a backward pass re-reads.

    Returns ``(o, hT, hck, vnew)``: o and hT as ``token_recurrence``; ``hck``
    the state h (K x V) at the start of every chunk of ``chunk`` tokens,
    before that chunk's first token is applied, [B,NT,H,K,V] with
    NT = ceil(T / chunk) (the KDA re-scan page's h checkpoints); ``vnew`` the
    delta beta_t (v_t - (decayed state)^T k_t) that token t writes into the
    state, [B,T,H,V] (the page's v_new, v' = u - w h of the chunk form).
    With ``heads`` the outputs are head-major: [n,T,V], [n,K,V], [n,NT,K,V],
    [n,T,V].
    """
    return _recurrence(q, k, v, beta, g, h0, heads, nthreads, True, True, int(chunk))


def rescan_dq(hck, do, chunk):
    """The chunk-start-state term of dq that the backward's re-scan forms
    (the KDA re-scan page, bwd_scan.py module docstring: DQ = do h_c^T, raw:
    no gate and no scale, those are applied by the later stage): for token t
    of chunk c, dq[t] = h_c do_t, with h_c (K x V) the state at the chunk's
    start, the checkpoints of ``token_states``.

    hck [B,NT,H,K,V], do [B,T,H,V] -> [B,T,H,K] fp64.
    """
    hck = np.asarray(hck, np.float64)
    do = np.asarray(do, np.float64)
    B, T, H, V = do.shape
    K = hck.shape[3]
    dq = np.zeros((B, T, H, K), np.float64)
    for c in range(hck.shape[1]):
        s, e = c * chunk, min(c * chunk + chunk, T)
        # [B,H,K,V] x [B,t,H,V] -> [B,t,H,K]
        dq[:, s:e] = np.einsum("bhkv,bthv->bthk", hck[:, c], do[:, s:e])
    return dq


# --------------------------------------------------------------------------
# Chunk form.  Per (batch, head) and per chunk of C tokens (the last chunk may
# be shorter).  Notation: gamma = chunk-local inclusive cumsum of g.
# --------------------------------------------------------------------------

def token_backward(q, k, v, beta, g, do, h0=None, dhT=None):
    """Gradients of the forward pass by reverse-mode differentiation of the
    token recurrence, the method's plain definition (decay, then the delta
    correction, then o_t = S_t q_t; the same steps as ``token_recurrence``),
    in fp64 with torch autograd on the CPU.  This is what the backward's WY
    stage of the kernel_fun KDA re-scan page (its dq/dk/dv/dbeta/dg outputs)
    computes by the chunk form.

    For L = sum_t o_t . do_t + sum hT * dhT (dhT optional), returns
    ``(dq, dk, dv, dbeta, dg, dh0)`` as float64 arrays in the inputs' layouts
    (dh0 is None without h0).  A Python loop over tokens: small inputs only.
    """
    import torch
    f64 = lambda x: torch.tensor(np.asarray(x, np.float64))
    qt, kt, vt, bt, gt = (f64(x).requires_grad_(True) for x in (q, k, v, beta, g))
    B, T, H, K = qt.shape
    V = vt.shape[-1]
    per_key = gt.dim() == 4
    h0t = f64(h0).requires_grad_(True) if h0 is not None else None
    S = h0t.transpose(-1, -2) if h0t is not None else torch.zeros(B, H, V, K, dtype=torch.float64)
    dot = f64(do)
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(T):
        a = torch.exp(gt[:, t])
        S = S * (a[:, :, None, :] if per_key else a[:, :, None, None])
        e = vt[:, t] - torch.einsum("bhvk,bhk->bhv", S, kt[:, t])
        S = S + bt[:, t, :, None, None] * e[..., :, None] * kt[:, t][..., None, :]
        loss = loss + (torch.einsum("bhvk,bhk->bhv", S, qt[:, t]) * dot[:, t]).sum()
    if dhT is not None:
        loss = loss + (S.transpose(-1, -2) * f64(dhT)).sum()
    loss.backward()
    grads = [x.grad.numpy() for x in (qt, kt, vt, bt, gt)]
    return tuple(grads) + (h0t.grad.numpy() if h0t is not None else None,)


def _chunks(T, C):
    for s in range(0, T, C):
        yield s, min(s + C, T)


def _pair_decay(gam):
    """exp(gam_r - gam_s) for every pair of rows of a chunk (gam [n] or
    [n, K]), with the exponent of the pairs s > r set to 0: those entries are
    always masked out (tril), and their growth factor would otherwise
    overflow to inf under strong decays (inf * 0 is NaN inside a product).
    The pairs s <= r are the plain exponential, for either sign of g."""
    n = gam.shape[0]
    d = gam[:, None] - gam[None, :]
    keep = (np.arange(n)[:, None] >= np.arange(n)[None, :])
    if d.ndim == 3:
        keep = keep[:, :, None]
    return np.exp(np.where(keep, d, 0.0))


def chunk_prepare(k, v, beta, g, chunk):
    """WY factors per chunk, fp64.  Returns ``(gcum, w, u)``.

    Follows the prepare kernel of the TileOPs gated deltanet page:
      1. gamma: the chunk-local cumulative sum of the log gate (inclusive of
         the current token; the KDA re-scan page stages the same cumsum, g2).
      2. A_g: strictly lower triangular, A[r,s] = beta_r * sum_d k[r,d] k[s,d]
         exp(gamma[r,d] - gamma[s,d]) for s < r (scalar gate: one exponent).
      3. The inverse of (I + A_g), unit lower triangular (the page's
         S_shared; it gets there by a Neumann series, here by an exact solve).
      4. k_beta = k * beta, v_beta = v * beta; w = inv @ (k_beta * exp(gamma)),
         u = inv @ v_beta.
    The exp(gamma) factor on k_beta is the reading under which the scan's
    v' = u - w h is taken against the chunk-start state, which the KDA page
    states ("kg carries the v~ scaling so v' stores un-decayed"); without it
    the chunk form disagrees with the token recurrence.
    """
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    g = np.asarray(g, np.float64)
    B, T, H, K = k.shape
    per_key = g.ndim == 4
    gcum = np.zeros_like(g)
    w = np.zeros(k.shape, np.float64)
    u = np.zeros(v.shape, np.float64)
    for b in range(B):
        for h in range(H):
            for s, e in _chunks(T, chunk):
                n = e - s
                kc = k[b, s:e, h]                       # [n,K]
                vc = v[b, s:e, h]                       # [n,V]
                bc = beta[b, s:e, h]                    # [n]
                gc = g[b, s:e, h]                       # [n] or [n,K]
                gam = np.cumsum(gc, axis=0)
                gcum[b, s:e, h] = gam
                if per_key:
                    # A[r,s] = beta_r sum_d k_rd k_sd exp(gam_rd - gam_sd)
                    dec = _pair_decay(gam)                        # [n,n,K]
                    G = np.einsum("rd,sd,rsd->rs", kc, kc, dec)
                    ke = kc * np.exp(gam)
                else:
                    G = (kc @ kc.T) * _pair_decay(gam)
                    ke = kc * np.exp(gam)[:, None]
                A = np.tril(bc[:, None] * G, -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                w[b, s:e, h] = Tm @ (ke * bc[:, None])
                u[b, s:e, h] = Tm @ (vc * bc[:, None])
    return gcum, w, u


def chunk_scan(q, k, w, u, gcum, chunk, h0=None, states=False):
    """Serial scan over chunks, fp64.  Returns ``(o, hT)``, and with
    ``states`` also the chunk-start states [B,NT,H,K,V] and v' [B,T,H,V]:
    ``(o, hT, hck, vnew)``.

    Per chunk with start state h (K x V), following the re-scan page's
    per-chunk algebra (there with h checkpoints and dq, which are not part of
    the forward output):
      v' = u - w h                         (the page's "v' = u - WH")
      o  = (q * exp(gamma)) h + tril_incl((q k^T) * decay) v'
      h  <- exp(gamma_last) * h + (k * exp(gamma_last - gamma))^T v'
    where decay[r,s] = exp(gamma_r - gamma_s) (per key dimension for KDA) and
    the causal mask keeps s <= r (o_t is read from the updated state).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    w = np.asarray(w, np.float64)
    u = np.asarray(u, np.float64)
    gcum = np.asarray(gcum, np.float64)
    B, T, H, K = q.shape
    V = u.shape[-1]
    per_key = gcum.ndim == 4
    o = np.zeros((B, T, H, V), np.float64)
    hT = np.zeros((B, H, K, V), np.float64)
    NT = (T + chunk - 1) // chunk
    hck = np.zeros((B, NT, H, K, V), np.float64) if states else None
    vnew = np.zeros((B, T, H, V), np.float64) if states else None
    for b in range(B):
        for hh in range(H):
            S = (np.zeros((K, V)) if h0 is None
                 else np.array(h0[b, hh], np.float64))
            for s, e in _chunks(T, chunk):
                qc, kc = q[b, s:e, hh], k[b, s:e, hh]
                wc, uc = w[b, s:e, hh], u[b, s:e, hh]
                gam = gcum[b, s:e, hh]
                vp = uc - wc @ S
                if states:
                    hck[b, s // chunk, hh] = S
                    vnew[b, s:e, hh] = vp
                if per_key:
                    dec = _pair_decay(gam)
                    P = np.einsum("rd,sd,rsd->rs", qc, kc, dec)
                    qd = qc * np.exp(gam)
                    kg = kc * np.exp(gam[-1][None, :] - gam)
                    last = np.exp(gam[-1])[:, None]
                else:
                    P = (qc @ kc.T) * _pair_decay(gam)
                    qd = qc * np.exp(gam)[:, None]
                    kg = kc * np.exp(gam[-1] - gam)[:, None]
                    last = np.exp(gam[-1])
                o[b, s:e, hh] = qd @ S + np.tril(P) @ vp
                S = last * S + kg.T @ vp
            hT[b, hh] = S
    if states:
        return o, hT, hck, vnew
    return o, hT


def chunk_forward(q, k, v, beta, g, chunk, h0=None, states=False):
    """chunk_prepare followed by chunk_scan."""
    gcum, w, u = chunk_prepare(k, v, beta, g, chunk)
    return chunk_scan(q, k, w, u, gcum, chunk, h0, states)


def chunk_backward(q, k, v, beta, g, do, chunk, h0=None, dhT=None, hck=None, vnew=None):
    """Gradients of the forward pass in the chunk form, fp64: the reverse
    state-gradient scan and the per-chunk gradient stage that the backward's
    WY stage computes (the kernel_fun KDA re-scan page, module docstring: the
    re-scan's h checkpoints and v' feed the later stage, which forms dq, dk,
    dv, dbeta and dg).  The same loss as ``token_backward``:
    L = sum_t o_t . do_t + sum hT * dhT.

    Per chunk, with gamma the chunk-local inclusive cumsum of g (per key
    column; a scalar gate is every column alike), b = exp(gamma),
    c = exp(gamma_last - gamma), E_rsd = exp(gamma_rd - gamma_sd), start
    state h and v' = D from the forward:
      A_rs = beta_r sum_d k_rd k_sd E_rsd (s < r),  T = (I + A)^-1
      P_rs = sum_d q_rd k_sd E_rsd (s <= r)
      R = diag(beta) (V - (K * b) h),  D = T R
      o = (Q * b) h + P D,  h' = diag(exp(gamma_last)) h + (K * c)^T D
    Reverse, from dh' (the gradient of the chunk-end state):
      dD = P^T dO + (K * c) dh',  dR = T^T dD
      dh = diag(exp(gamma_last)) dh' + (Q * b)^T dO - (K * b * beta)^T dR
    and the chunk's gradients from dP = tril_incl(dO D^T),
    dA = -strict_tril(dR D^T), Z = dO h^T, Y = dR h^T, W = D dh'^T (each
    term differentiates one factor above; dg is the reverse cumsum of the
    gradient of gamma, the last row also taking gamma_last's).

    With ``hck`` [B,NT,H,K,V] and ``vnew`` [B,T,H,V] (the forward's saved
    chunk-start states and deltas, as token_states returns them, possibly
    rounded) the per-chunk gradients take h and D from them, as a backward
    that is handed saved states does; the reverse scan needs neither.

    Returns ``(dq, dk, dv, dbeta, dg, dh0, extra)`` with dh0 None without h0
    and ``extra`` a dict of the intermediates: ``dR`` [B,T,H,V] and ``dhe``
    [B,NT,H,K,V], the gradient of each chunk's end state (dhT for the last).
    """
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    beta = np.asarray(beta, np.float64)
    g = np.asarray(g, np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    per_key = g.ndim == 4
    NT = (T + chunk - 1) // chunk
    dq, dk = np.zeros_like(q), np.zeros_like(k)
    dv = np.zeros_like(v)
    dbeta = np.zeros_like(beta)
    dg = np.zeros_like(g)
    dh0 = np.zeros((B, H, K, V)) if h0 is not None else None
    dR_all = np.zeros((B, T, H, V))
    dhe = np.zeros((B, NT, H, K, V))
    spans = list(_chunks(T, chunk))
    for b in range(B):
        for hh in range(H):
            # forward: chunk-start states and each chunk's factors
            S = np.zeros((K, V)) if h0 is None else np.array(h0[b, hh], np.float64)
            saved = []
            for s, e in spans:
                n = e - s
                qc, kc, vc = q[b, s:e, hh], k[b, s:e, hh], v[b, s:e, hh]
                bc = beta[b, s:e, hh]
                gc = g[b, s:e, hh]
                gam = np.cumsum(gc if per_key else np.repeat(gc[:, None], K, 1), axis=0)   # [n,K]
                # E_rsd (the entries s > r are only ever multiplied by masked-out
                # zeros; _pair_decay keeps them finite)
                E = _pair_decay(gam)                                                  # [n,n,K]
                lower = np.tril(np.ones((n, n)), -1)
                A = lower * bc[:, None] * np.einsum("rd,sd,rsd->rs", kc, kc, E)
                P = np.tril(np.einsum("rd,sd,rsd->rs", qc, kc, E))
                Tm = np.linalg.inv(np.eye(n) + A)
                bq = np.exp(gam)
                cq = np.exp(gam[-1][None, :] - gam)
                R = bc[:, None] * (vc - (kc * bq) @ S)
                D = Tm @ R
                ci = s // chunk
                saved.append((S if hck is None else np.asarray(hck[b, ci, hh], np.float64), gam, E, A, P, Tm,
                              D if vnew is None else np.asarray(vnew[b, s:e, hh], np.float64)))
                S = np.exp(gam[-1])[:, None] * S + (kc * cq).T @ D
            # reverse
            dH = np.zeros((K, V)) if dhT is None else np.array(dhT[b, hh], np.float64)
            for ci in range(len(spans) - 1, -1, -1):
                s, e = spans[ci]
                n = e - s
                Sc, gam, E, A, P, Tm, D = saved[ci]
                qc, kc, vc = q[b, s:e, hh], k[b, s:e, hh], v[b, s:e, hh]
                bc = beta[b, s:e, hh]
                doc = do[b, s:e, hh]
                bq = np.exp(gam)
                cq = np.exp(gam[-1][None, :] - gam)
                gl = np.exp(gam[-1])
                dhe[b, ci, hh] = dH
                dD = P.T @ doc + (kc * cq) @ dH
                dR = Tm.T @ dD
                dP = np.tril(doc @ D.T)
                dA = -np.tril(dR @ D.T, -1)
                Z = doc @ Sc.T
                Y = dR @ Sc.T
                W = D @ dH.T
                # dq, dk through P and A (per key column d)
                tP = np.einsum("rs,rd,sd,rsd->rsd", dP, qc, kc, E)
                tA = np.einsum("rs,r,rd,sd,rsd->rsd", dA, bc, kc, kc, E)
                dqc = bq * Z + np.einsum("rs,sd,rsd->rd", dP, kc, E)
                dkc = (np.einsum("rs,rd,rsd->sd", dP, qc, E)
                       + np.einsum("rs,r,sd,rsd->rd", dA, bc, kc, E)
                       + np.einsum("rs,r,rd,rsd->sd", dA, bc, kc, E)
                       - bc[:, None] * bq * Y + cq * W)
                dvc = bc[:, None] * dR
                dbc = (np.einsum("rv,rv->r", dR, vc) - np.einsum("rd,rd,rd->r", bq, kc, Y)
                       + np.einsum("rs,rd,sd,rsd->r", dA, kc, kc, E))
                dgam = (bq * qc * Z - bc[:, None] * bq * kc * Y
                        + tP.sum(1) - tP.sum(0) + tA.sum(1) - tA.sum(0) - cq * kc * W)
                dgam[-1] += (cq * kc * W).sum(0) + gl * np.einsum("dv,dv->d", Sc, dH)
                dgc = np.cumsum(dgam[::-1], axis=0)[::-1]
                dq[b, s:e, hh] = dqc
                dk[b, s:e, hh] = dkc
                dv[b, s:e, hh] = dvc
                dbeta[b, s:e, hh] = dbc
                dg[b, s:e, hh] = dgc if per_key else dgc.sum(1)
                dR_all[b, s:e, hh] = dR
                dH = gl[:, None] * dH + (qc * bq).T @ doc - (kc * bq * bc[:, None]).T @ dR
            if dh0 is not None:
                dh0[b, hh] = dH
    return dq, dk, dv, dbeta, dg, dh0, {"dR": dR_all, "dhe": dhe}


def rel_err(x, ref):
    """max |x - ref| / rms(ref), the parity measure used throughout."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    if rms == 0.0:
        return float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return float(np.max(np.abs(x - ref)) / rms)
