"""chunked_gated_delta_prepare_amd -- Python binding for libgdn.

Forward pass of the chunked gated delta rule (Gated DeltaNet with one gate
per head, Kimi-Delta-Attention with one gate per key dimension) on AMD
MI355X.  Every step runs in the HIP kernels of ``libgdn.so``; this module only
checks tensors, allocates outputs with torch and passes raw pointers and the
current HIP stream through the C ABI declared in ``include/libgdn.h``.

Entry points (same names as the C ABI):
    prepare(k, v, beta, g, chunk)                 -> (w, u, gcum)
    scan(q, k, w, u, gcum, chunk, h0=None)        -> (o, hT)
    forward(q, k, v, beta, g, chunk, h0=None)     -> (o, hT)
    forward_states(q, k, v, beta, g, chunk, h0=None)
                                                  -> (o, hT, hck, vnew)
    forward_varlen(q, k, v, beta, g, cu_seqlens, chunk, h0=None)
                                                  -> (o, hT [N,H,K,V])
    rescan_dq(q, k, v, beta, g, do, chunk, h0=None)
                                                  -> (hT, hck, vnew, dq)
Layouts: q, k [B,T,H,K]; v [B,T,H,V]; beta [B,T,H]; g [B,T,H] or [B,T,H,K];
h0/hT [B,H,K,V] fp32.  q, k, v are bf16 or fp32 (same dtype); o is the io
dtype unless ``o_dtype`` says otherwise.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["prepare", "scan", "forward", "forward_states", "forward_varlen", "rescan_dq",
           "workspace_bytes", "wait_timeouts",
           "load_library",
           "GdnError", "LIB_PATH", "POISON_LIB_PATH", "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
# the debug build (build.py, poison=True): the same entry points, with every
# pipelined kernel filling its LDS stages with NaN once their last reader is
# done, so that a read that runs ahead of its write shows up as NaN
POISON_LIB_PATH = os.path.join(_HERE, "libgdn_poison.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_GATE_HEAD, GDN_GATE_KEY = 0, 1
STATUS = {
    0: "GDN_OK", 1: "GDN_ERR_NULL_ARG", 2: "GDN_ERR_BAD_SHAPE",
    3: "GDN_ERR_UNSUPPORTED", 4: "GDN_ERR_ALIGNMENT", 5: "GDN_ERR_LDS_BUDGET",
    6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_HIP",
}
EXPORTS = ["gdn_prepare", "gdn_scan", "gdn_forward", "gdn_forward_states",
           "gdn_forward_varlen", "gdn_rescan_dq", "gdn_chunk_dq", "gdn_workspace_bytes",
           "gdn_workspace_bytes_varlen", "gdn_status_str", "gdn_abi_version",
           "gdn_wait_timeouts", "gdn_forward_noalloc", "gdn_forward_split",
           "gdn_workspace_bytes_split", "gdn_backward", "gdn_workspace_bytes_backward",
           "gdn_forward_split_point"]
NOALLOC_SCRATCH_BYTES = 32 << 20
ABI_VERSION = 10


class GdnError(RuntimeError):
    def __init__(self, call, status, message):
        super().__init__("%s failed: %s" % (call, message))
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("K", ctypes.c_int64), ("V", ctypes.c_int64), ("chunk", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
                ("gate", ctypes.c_int32)]


_lib = None
_lock = threading.Lock()


def load_library(path: str | None = None):
    """Load libgdn.so (built in-tree by build.py).  Raises if it is missing:
    there is no fallback implementation."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                "libgdn.so not found at %s; build it with "
                "`python -m chunked_gated_delta_prepare_amd.build`" % p)
        lib = ctypes.CDLL(p)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        pp = ctypes.POINTER(Problem)
        lib.gdn_prepare.argtypes = [pp] + [vp] * 8
        lib.gdn_scan.argtypes = [pp] + [vp] * 9
        lib.gdn_forward.argtypes = [pp] + [vp] * 9 + [sz, vp]
        lib.gdn_forward_states.argtypes = [pp] + [vp] * 11 + [sz, vp]
        lib.gdn_forward_varlen.argtypes = [pp, vp, ctypes.c_int64] + [vp] * 9 + [sz, vp]
        lib.gdn_rescan_dq.argtypes = [pp] + [vp] * 12 + [sz, vp]
        lib.gdn_chunk_dq.argtypes = [pp] + [vp] * 4
        lib.gdn_forward_noalloc.argtypes = [pp] + [vp] * 9
        lib.gdn_forward_split.argtypes = [pp, ctypes.c_int64] + [vp] * 9 + [sz, vp]
        lib.gdn_workspace_bytes_split.argtypes = [pp, ctypes.c_int64]
        lib.gdn_workspace_bytes_split.restype = sz
        lib.gdn_forward_split_point.argtypes = [pp]
        lib.gdn_forward_split_point.restype = ctypes.c_int64
        lib.gdn_backward.argtypes = [pp] + [vp] * 16 + [sz, vp]
        lib.gdn_workspace_bytes_backward.argtypes = [pp]
        lib.gdn_workspace_bytes_backward.restype = sz
        for f in (lib.gdn_prepare, lib.gdn_scan, lib.gdn_forward, lib.gdn_forward_states,
                  lib.gdn_forward_varlen, lib.gdn_rescan_dq, lib.gdn_chunk_dq,
                  lib.gdn_forward_noalloc, lib.gdn_forward_split, lib.gdn_backward):
            f.restype = ctypes.c_int
        lib.gdn_workspace_bytes.argtypes = [pp]
        lib.gdn_workspace_bytes.restype = sz
        lib.gdn_workspace_bytes_varlen.argtypes = [pp, ctypes.c_int64]
        lib.gdn_workspace_bytes_varlen.restype = sz
        lib.gdn_status_str.argtypes = [ctypes.c_int]
        lib.gdn_status_str.restype = ctypes.c_char_p
        lib.gdn_abi_version.argtypes = []
        lib.gdn_abi_version.restype = ctypes.c_int
        lib.gdn_wait_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
        lib.gdn_wait_timeouts.restype = ctypes.c_int
        if lib.gdn_abi_version() != ABI_VERSION:
            raise RuntimeError("libgdn ABI %d, binding expects %d"
                               % (lib.gdn_abi_version(), ABI_VERSION))
        if path is None:
            _lib = lib
        return lib


def _torch():
    import torch
    return torch


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float32:
        return GDN_F32
    if dt == torch.bfloat16:
        return GDN_BF16
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % dt)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _check(call, rc):
    if rc != 0:
        lib = load_library()
        raise GdnError(call, rc, lib.gdn_status_str(rc).decode())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _problem(q_or_k, v, chunk, gate_per_key, o_dtype):
    B, T, H, K = q_or_k.shape
    V = v.shape[-1] if v is not None else K
    io = _dtype_code(q_or_k.dtype)
    return Problem(B, T, H, K, V, int(chunk), io, _dtype_code(o_dtype),
                   GDN_GATE_KEY if gate_per_key else GDN_GATE_HEAD)


def _gate_kind(g, B, T, H, K):
    if tuple(g.shape) == (B, T, H):
        return False
    if tuple(g.shape) == (B, T, H, K):
        return True
    raise ValueError("g must be [B,T,H] or [B,T,H,K], got %s" % (tuple(g.shape),))


def workspace_bytes(B, T, H, K, V, chunk, io_dtype, gate_per_key=False, o_dtype=None):
    io = _dtype_code(io_dtype)
    od = _dtype_code(o_dtype or io_dtype)
    pr = Problem(B, T, H, K, V, chunk, io, od, GDN_GATE_KEY if gate_per_key else GDN_GATE_HEAD)
    return int(load_library().gdn_workspace_bytes(ctypes.byref(pr)))


def forward_split_point(B, T, H, K, V, chunk, io_dtype, gate_per_key=False, o_dtype=None):
    """gdn_forward_split_point: the token at which gdn_forward cuts each
    stream into two segments run side by side, or 0 for a single pass."""
    pr = Problem(B, T, H, K, V, int(chunk), _dtype_code(io_dtype), _dtype_code(o_dtype or io_dtype),
                 GDN_GATE_KEY if gate_per_key else GDN_GATE_HEAD)
    return int(load_library().gdn_forward_split_point(ctypes.byref(pr)))


def wait_timeouts(reset=False):
    """Count of bounded LDS waits inside the bf16-io kernels that gave up on
    the current device since the last reset (gdn_wait_timeouts; synchronous).
    A launch during which it grew produced results that must not be trusted."""
    lib = load_library()
    n = ctypes.c_uint32(0)
    _check("gdn_wait_timeouts", lib.gdn_wait_timeouts(ctypes.byref(n), 1 if reset else 0))
    return int(n.value)


def prepare(k, v, beta, g, chunk, *, w=None, u=None, gcum=None, stream=None):
    """WY factors per chunk: returns (w [B,T,H,K], u [B,T,H,V], gcum) fp32."""
    torch = _torch()
    lib = load_library()
    B, T, H, K = k.shape
    V = v.shape[-1]
    per_key = _gate_kind(g, B, T, H, K)
    _need(k, "k")
    _need(v, "v", k.dtype, (B, T, H, V))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(g, "g", torch.float32)
    dev = k.device
    if w is None:
        w = torch.empty(B, T, H, K, device=dev, dtype=torch.float32)
    if u is None:
        u = torch.empty(B, T, H, V, device=dev, dtype=torch.float32)
    if gcum is None:
        gcum = torch.empty_like(g)
    _need(w, "w", torch.float32, (B, T, H, K))
    _need(u, "u", torch.float32, (B, T, H, V))
    _need(gcum, "gcum", torch.float32, tuple(g.shape))
    pr = _problem(k, v, chunk, per_key, k.dtype)
    rc = lib.gdn_prepare(ctypes.byref(pr), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                         _ptr(w), _ptr(u), _ptr(gcum), _stream(stream))
    _check("gdn_prepare", rc)
    return w, u, gcum


def scan(q, k, w, u, gcum, chunk, h0=None, *, o_dtype=None, o=None, hT=None,
         output_final_state=True, stream=None):
    """Inter-chunk scan from WY factors: returns (o, hT or None)."""
    torch = _torch()
    lib = load_library()
    B, T, H, K = q.shape
    V = u.shape[-1]
    per_key = _gate_kind(gcum, B, T, H, K)
    _need(q, "q")
    _need(k, "k", q.dtype, (B, T, H, K))
    _need(w, "w", torch.float32, (B, T, H, K))
    _need(u, "u", torch.float32, (B, T, H, V))
    _need(gcum, "gcum", torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, H, K, V))
    od = o_dtype or q.dtype
    if o is None:
        o = torch.empty(B, T, H, V, device=q.device, dtype=od)
    _need(o, "o", od, (B, T, H, V))
    if hT is None and output_final_state:
        hT = torch.empty(B, H, K, V, device=q.device, dtype=torch.float32)
    if hT is not None:
        _need(hT, "hT", torch.float32, (B, H, K, V))
    pr = _problem(q, u, chunk, per_key, od)
    rc = lib.gdn_scan(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(w), _ptr(u), _ptr(gcum),
                      _ptr(h0), _ptr(o), _ptr(hT), _stream(stream))
    _check("gdn_scan", rc)
    return o, hT


def _workspace(lib, pr, device, workspace, n_seqs=0, split=False):
    """The workspace the call needs (gdn_workspace_bytes), allocated with
    torch when the caller passes none; returns (tensor or None, bytes).
    For the scalar gate only gdn_forward uses one (its sequence split:
    ``split``); the other entry points need none."""
    torch = _torch()
    if pr.gate == GDN_GATE_HEAD and not split:
        need = 0
    else:
        need = int(lib.gdn_workspace_bytes_varlen(ctypes.byref(pr), ctypes.c_int64(n_seqs)) if n_seqs
                   else lib.gdn_workspace_bytes(ctypes.byref(pr)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, ctypes.c_size_t(ws_bytes)


def forward(q, k, v, beta, g, chunk, h0=None, *, o_dtype=None, o=None, hT=None,
            output_final_state=True, workspace=None, stream=None, library=None):
    """Whole forward pass: returns (o [B,T,H,V], hT [B,H,K,V] fp32 or None).
    ``library``: a library from load_library(path) to call instead of
    libgdn.so (the debug build at POISON_LIB_PATH)."""
    return _forward(q, k, v, beta, g, chunk, h0, o_dtype, o, hT, output_final_state,
                    workspace, stream, noalloc=False, library=library)


def forward_noalloc(q, k, v, beta, g, chunk, h0=None, *, o=None, hT=None, stream=None):
    """gdn_forward_noalloc: the forward pass with the per-key gate's workspace
    taken from the library's static device scratch (at most
    NOALLOC_SCRATCH_BYTES) instead of an allocation.  The library call itself
    allocates nothing; o and hT, which the caller must pass, are written in
    place and returned."""
    if o is None:
        raise ValueError("forward_noalloc writes into a caller-provided o")
    return _forward(q, k, v, beta, g, chunk, h0, o.dtype, o, hT, hT is not None, None, stream,
                    noalloc=True)


def _forward(q, k, v, beta, g, chunk, h0, o_dtype, o, hT, output_final_state, workspace,
             stream, noalloc, library=None):
    torch = _torch()
    lib = library or load_library()
    B, T, H, K = q.shape
    V = v.shape[-1]
    per_key = _gate_kind(g, B, T, H, K)
    _need(q, "q")
    _need(k, "k", q.dtype, (B, T, H, K))
    _need(v, "v", q.dtype, (B, T, H, V))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(g, "g", torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, H, K, V))
    od = o_dtype or q.dtype
    if o is None:
        o = torch.empty(B, T, H, V, device=q.device, dtype=od)
    _need(o, "o", od, (B, T, H, V))
    if hT is None and output_final_state:
        hT = torch.empty(B, H, K, V, device=q.device, dtype=torch.float32)
    if hT is not None:
        _need(hT, "hT", torch.float32, (B, H, K, V))
    pr = _problem(q, v, chunk, per_key, od)
    if noalloc:
        rc = lib.gdn_forward_noalloc(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                     _ptr(g), _ptr(h0), _ptr(o), _ptr(hT), _stream(stream))
        _check("gdn_forward_noalloc", rc)
        return o, hT
    workspace, ws_bytes = _workspace(lib, pr, q.device, workspace, split=True)
    rc = lib.gdn_forward(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                         _ptr(h0), _ptr(o), _ptr(hT), _ptr(workspace), ws_bytes, _stream(stream))
    _check("gdn_forward", rc)
    return o, hT


def forward_split(q, k, v, beta, g, chunk, t_split, h0=None, *, o_dtype=None, o=None, hT=None,
                  output_final_state=True, workspace=None, stream=None):
    """gdn_forward_split: the scalar-gate forward (bf16 io, chunk 64) with each
    stream cut at token t_split into two segments that run at the same time;
    returns (o, hT or None) like forward."""
    torch = _torch()
    lib = load_library()
    B, T, H, K = q.shape
    V = v.shape[-1]
    if _gate_kind(g, B, T, H, K):
        raise GdnError("gdn_forward_split", 3, "the split forward takes the scalar gate only")
    _need(q, "q")
    _need(k, "k", q.dtype, (B, T, H, K))
    _need(v, "v", q.dtype, (B, T, H, V))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(g, "g", torch.float32, (B, T, H))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, H, K, V))
    od = o_dtype or q.dtype
    if o is None:
        o = torch.empty(B, T, H, V, device=q.device, dtype=od)
    _need(o, "o", od, (B, T, H, V))
    if hT is None and output_final_state:
        hT = torch.empty(B, H, K, V, device=q.device, dtype=torch.float32)
    if hT is not None:
        _need(hT, "hT", torch.float32, (B, H, K, V))
    pr = _problem(q, v, chunk, False, od)
    need = int(lib.gdn_workspace_bytes_split(ctypes.byref(pr), ctypes.c_int64(t_split)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.gdn_forward_split(ctypes.byref(pr), ctypes.c_int64(t_split), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(beta), _ptr(g), _ptr(h0), _ptr(o), _ptr(hT), _ptr(workspace),
                               ctypes.c_size_t(ws_bytes), _stream(stream))
    _check("gdn_forward_split", rc)
    return o, hT


def forward_states(q, k, v, beta, g, chunk, h0=None, *, o_dtype=None, o=None, hT=None,
                   hck=None, vnew=None, output_final_state=True, workspace=None, stream=None,
                   library=None):
    """Forward pass that also saves the chunk-start states and the per-token
    deltas: returns (o, hT or None, hck [B,NT,H,K,V], vnew [B,T,H,V]), with
    hck and vnew in the o dtype and NT = ceil(T / chunk).  ``library`` as
    for forward."""
    torch = _torch()
    lib = library or load_library()
    B, T, H, K = q.shape
    V = v.shape[-1]
    per_key = _gate_kind(g, B, T, H, K)
    _need(q, "q")
    _need(k, "k", q.dtype, (B, T, H, K))
    _need(v, "v", q.dtype, (B, T, H, V))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(g, "g", torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, H, K, V))
    od = o_dtype or q.dtype
    nt = (T + int(chunk) - 1) // int(chunk) if chunk > 0 else 0
    if o is None:
        o = torch.empty(B, T, H, V, device=q.device, dtype=od)
    if hck is None:
        hck = torch.empty(B, nt, H, K, V, device=q.device, dtype=od)
    if vnew is None:
        vnew = torch.empty(B, T, H, V, device=q.device, dtype=od)
    _need(o, "o", od, (B, T, H, V))
    _need(hck, "hck", od, (B, nt, H, K, V))
    _need(vnew, "vnew", od, (B, T, H, V))
    if hT is None and output_final_state:
        hT = torch.empty(B, H, K, V, device=q.device, dtype=torch.float32)
    if hT is not None:
        _need(hT, "hT", torch.float32, (B, H, K, V))
    pr = _problem(q, v, chunk, per_key, od)
    if T == 0:
        rc = lib.gdn_forward_states(ctypes.byref(pr), None, None, None, None, None,
                                    _ptr(h0), None, _ptr(hT), None, None, None,
                                    ctypes.c_size_t(0), _stream(stream))
    else:
        workspace, ws_bytes = _workspace(lib, pr, q.device, workspace)
        rc = lib.gdn_forward_states(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                    _ptr(g), _ptr(h0), _ptr(o), _ptr(hT), _ptr(hck),
                                    _ptr(vnew), _ptr(workspace), ws_bytes, _stream(stream))
    _check("gdn_forward_states", rc)
    return o, hT, hck, vnew


def forward_varlen(q, k, v, beta, g, cu_seqlens, chunk, h0=None, *, o_dtype=None, o=None,
                   hT=None, output_final_state=True, workspace=None, stream=None, library=None):
    """Forward pass over packed sequences: q, k [1,T,H,K], v [1,T,H,V], beta
    [1,T,H], g [1,T,H] or [1,T,H,K]; cu_seqlens an int32 device tensor of
    N + 1 token offsets; h0 [N,H,K,V] fp32 or None.  Returns (o [1,T,H,V],
    hT [N,H,K,V] or None).  ``library`` as for forward."""
    torch = _torch()
    lib = library or load_library()
    B, T, H, K = q.shape
    V = v.shape[-1]
    if B != 1:
        raise ValueError("packed sequences use a batch of 1, got %d" % B)
    per_key = _gate_kind(g, B, T, H, K)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must hold N + 1 >= 2 offsets")
    N = cu_seqlens.numel() - 1
    _need(q, "q")
    _need(k, "k", q.dtype, (B, T, H, K))
    _need(v, "v", q.dtype, (B, T, H, V))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(g, "g", torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (N, H, K, V))
    od = o_dtype or q.dtype
    if o is None:
        o = torch.empty(B, T, H, V, device=q.device, dtype=od)
    _need(o, "o", od, (B, T, H, V))
    if hT is None and output_final_state:
        hT = torch.empty(N, H, K, V, device=q.device, dtype=torch.float32)
    if hT is not None:
        _need(hT, "hT", torch.float32, (N, H, K, V))
    pr = _problem(q, v, chunk, per_key, od)
    workspace, ws_bytes = _workspace(lib, pr, q.device, workspace, n_seqs=N)
    rc = lib.gdn_forward_varlen(ctypes.byref(pr), _ptr(cu_seqlens), ctypes.c_int64(N),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0),
                                _ptr(o), _ptr(hT), _ptr(workspace), ws_bytes, _stream(stream))
    _check("gdn_forward_varlen", rc)
    return o, hT


def chunk_dq(do, hck, chunk, *, dq=None, stream=None):
    """dq's chunk-start-state term from saved states: dq[t] = h_c do_t (raw)
    for token t of chunk c, with do [B,T,H,V] bf16 and hck [B,NT,H,K,V] bf16
    or fp32 as forward_states returns it.  Returns dq [B,T,H,K] fp32,
    written (a given dq is overwritten, not accumulated into)."""
    torch = _torch()
    lib = load_library()
    B, T, H, V = do.shape
    K = hck.shape[3]
    nt = (T + int(chunk) - 1) // int(chunk) if chunk > 0 else 0
    _need(do, "do", torch.bfloat16)
    _need(hck, "hck", None, (B, nt, H, K, V))
    if hck.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("hck must be bfloat16 or float32, got %s" % hck.dtype)
    if dq is None:
        dq = torch.empty(B, T, H, K, device=do.device, dtype=torch.float32)
    _need(dq, "dq", torch.float32, (B, T, H, K))
    pr = Problem(B, T, H, K, V, int(chunk), _dtype_code(do.dtype), _dtype_code(hck.dtype),
                 GDN_GATE_HEAD)
    rc = lib.gdn_chunk_dq(ctypes.byref(pr), _ptr(do) if T else None, _ptr(hck) if T else None,
                          _ptr(dq) if T else None, _stream(stream))
    _check("gdn_chunk_dq", rc)
    return dq


def rescan_dq(q, k, v, beta, g, do, chunk, h0=None, *, o_dtype=None, hT=None, hck=None,
              vnew=None, dq=None, output_final_state=True, workspace=None, stream=None):
    """The backward's forward re-scan with bf16 io: returns (hT or None,
    hck [B,NT,H,K,V], vnew [B,T,H,V], dq [B,T,H,K] fp32) with
    dq[t] = h_c do_t (raw, the chunk-start-state term).  g is [B,T,H] (one
    gate per head) or [B,T,H,K] (one per key dimension, chunk 64 only).  A
    given dq is accumulated into; a new one starts from zero."""
    torch = _torch()
    lib = load_library()
    B, T, H, K = q.shape
    V = v.shape[-1]
    per_key = _gate_kind(g, B, T, H, K)
    _need(q, "q")
    _need(k, "k", q.dtype, (B, T, H, K))
    _need(v, "v", q.dtype, (B, T, H, V))
    _need(do, "do", q.dtype, (B, T, H, V))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(g, "g", torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, H, K, V))
    od = o_dtype or q.dtype
    nt = (T + int(chunk) - 1) // int(chunk) if chunk > 0 else 0
    if hck is None:
        hck = torch.empty(B, nt, H, K, V, device=q.device, dtype=od)
    if vnew is None:
        vnew = torch.empty(B, T, H, V, device=q.device, dtype=od)
    if dq is None:
        dq = torch.zeros(B, T, H, K, device=q.device, dtype=torch.float32)
    _need(hck, "hck", od, (B, nt, H, K, V))
    _need(vnew, "vnew", od, (B, T, H, V))
    _need(dq, "dq", torch.float32, (B, T, H, K))
    if hT is None and output_final_state:
        hT = torch.empty(B, H, K, V, device=q.device, dtype=torch.float32)
    if hT is not None:
        _need(hT, "hT", torch.float32, (B, H, K, V))
    pr = _problem(q, v, chunk, per_key, od)
    if T == 0:
        rc = lib.gdn_rescan_dq(ctypes.byref(pr), None, None, None, None, None, _ptr(h0), None,
                               _ptr(hT), None, None, None, None, ctypes.c_size_t(0),
                               _stream(stream))
    else:
        workspace, ws_bytes = _workspace(lib, pr, q.device, workspace)
        rc = lib.gdn_rescan_dq(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                               _ptr(h0), _ptr(do), _ptr(hT), _ptr(hck), _ptr(vnew), _ptr(dq),
                               _ptr(workspace), ws_bytes, _stream(stream))
    _check("gdn_rescan_dq", rc)
    return hT, hck, vnew, dq


def backward(q, k, v, beta, g, do, chunk, hck, vnew, dhT=None, *, want_dh0=True, dq=None, dk=None,
             dv=None, dbeta=None, dg=None, dh0=None, workspace=None, stream=None):
    """Gradients of the forward (bf16 io; g [B,T,H] one gate per head or
    [B,T,H,K] one per key dimension) for the loss sum_t o_t . do_t +
    sum hT * dhT, from the bf16 hck and vnew that forward_states (or
    rescan_dq) saved for the same inputs and chunk.  Returns (dq, dk, dv,
    dbeta, dg, dh0 or None), fp32, dg in g's shape.  The workspace
    (gdn_workspace_bytes_backward bytes) is allocated when not given; after
    the call it starts with v's gradient before the beta factor [B,T,H,V]
    and the gradient of every chunk's end state [B,NT,H,K,V], both fp32."""
    torch = _torch()
    lib = load_library()
    B, T, H, K = q.shape
    V = v.shape[-1]
    per_key = _gate_kind(g, B, T, H, K)
    gshape = (B, T, H, K) if per_key else (B, T, H)
    nt = (T + int(chunk) - 1) // int(chunk) if chunk > 0 else 0
    for t, name, dt, shp in ((q, "q", torch.bfloat16, None), (k, "k", torch.bfloat16, (B, T, H, K)),
                             (v, "v", torch.bfloat16, (B, T, H, V)),
                             (do, "do", torch.bfloat16, (B, T, H, V)),
                             (beta, "beta", torch.float32, (B, T, H)), (g, "g", torch.float32, gshape),
                             (hck, "hck", torch.bfloat16, (B, nt, H, K, V)),
                             (vnew, "vnew", torch.bfloat16, (B, T, H, V))):
        _need(t, name, dt, shp)
    if dhT is not None:
        _need(dhT, "dhT", torch.float32, (B, H, K, V))
    dev = q.device
    f32 = dict(device=dev, dtype=torch.float32)
    dq = torch.empty(B, T, H, K, **f32) if dq is None else dq
    dk = torch.empty(B, T, H, K, **f32) if dk is None else dk
    dv = torch.empty(B, T, H, V, **f32) if dv is None else dv
    dbeta = torch.empty(B, T, H, **f32) if dbeta is None else dbeta
    dg = torch.empty(*gshape, **f32) if dg is None else dg
    if dh0 is None and want_dh0:
        dh0 = torch.empty(B, H, K, V, **f32)
    for t, name, shp in ((dq, "dq", (B, T, H, K)), (dk, "dk", (B, T, H, K)), (dv, "dv", (B, T, H, V)),
                         (dbeta, "dbeta", (B, T, H)), (dg, "dg", gshape)):
        _need(t, name, torch.float32, shp)
    if dh0 is not None:
        _need(dh0, "dh0", torch.float32, (B, H, K, V))
    pr = _problem(q, v, chunk, per_key, torch.bfloat16)
    need = int(lib.gdn_workspace_bytes_backward(ctypes.byref(pr)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
    _need(workspace, "workspace")
    rc = lib.gdn_backward(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(do),
                          _ptr(dhT), _ptr(hck), _ptr(vnew), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta),
                          _ptr(dg), _ptr(dh0), _ptr(workspace),
                          ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                          _stream(stream))
    _check("gdn_backward", rc)
    return dq, dk, dv, dbeta, dg, dh0
