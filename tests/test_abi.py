"""Host-only checks of the C ABI: the library loads, exports every function
include/libgdn.h declares, and rejects bad arguments before enqueuing any
GPU work (every call below returns during validation, so none needs a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgdn.h")


@pytest.fixture(scope="module")
def lib():
    import chunked_gated_delta_prepare_amd as gdn
    if not os.path.exists(gdn.LIB_PATH):
        from chunked_gated_delta_prepare_amd import build
        build.build()
    return gdn.load_library()


@pytest.fixture(scope="module")
def gdn():
    import chunked_gated_delta_prepare_amd as m
    return m


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(gdn_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(
        ["gdn_prepare", "gdn_scan", "gdn_forward", "gdn_forward_states",
         "gdn_forward_varlen", "gdn_rescan_dq", "gdn_chunk_dq", "gdn_workspace_bytes",
         "gdn_workspace_bytes_varlen", "gdn_status_str", "gdn_abi_version",
         "gdn_wait_timeouts", "gdn_forward_noalloc", "gdn_forward_split",
         "gdn_workspace_bytes_split", "gdn_backward", "gdn_workspace_bytes_backward",
         "gdn_forward_split_point"])


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_debug_build_exports_the_same_boundary(gdn):
    """libgdn_poison.so (LDS stages filled with NaN on release) is a drop-in
    for libgdn.so: same symbols, same ABI version."""
    if not os.path.exists(gdn.POISON_LIB_PATH):
        from chunked_gated_delta_prepare_amd import build
        build.build(poison=True)
    dbg = gdn.load_library(gdn.POISON_LIB_PATH)
    for name in _declared_functions():
        assert hasattr(dbg, name), name
    assert dbg.gdn_abi_version() == gdn.ABI_VERSION


def test_binding_exports_match_header(gdn):
    assert sorted(gdn.EXPORTS) == _declared_functions()


def test_abi_version_and_status_strings(lib, gdn):
    assert lib.gdn_abi_version() == gdn.ABI_VERSION
    for code, name in gdn.STATUS.items():
        assert lib.gdn_status_str(code).decode().startswith(name)
    assert b"unknown" in lib.gdn_status_str(99)


def test_header_enums_match_binding(gdn):
    src = open(HEADER).read()
    for code, name in gdn.STATUS.items():
        assert re.search(r"\b%s = %d\b" % (name, code), src), name
    assert re.search(r"GDN_F32 = 0", src) and re.search(r"GDN_BF16 = 1", src)
    assert re.search(r"GDN_GATE_HEAD = 0", src) and re.search(r"GDN_GATE_KEY = 1", src)
    assert re.search(r"#define GDN_ABI_VERSION %d\b" % gdn.ABI_VERSION, src)


def _problem(gdn, B=1, T=64, H=1, K=64, V=64, chunk=64, io=1, o=1, gate=0):
    return gdn.Problem(B, T, H, K, V, chunk, io, o, gate)


FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10008)


def _fwd(lib, pr, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, h0=None, o=FAKE,
         hT=None, ws=FAKE, ws_bytes=1 << 40):
    return lib.gdn_forward(ctypes.byref(pr), q, k, v, beta, g, h0, o, hT, ws,
                           ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("field,value,status", [
    ("K", 96, 3), ("V", 32, 3), ("chunk", 16, 3), ("chunk", 128, 3),
    ("io_dtype", 7, 3), ("o_dtype", 5, 3), ("gate", 2, 3),
    ("B", 0, 2), ("H", 0, 2), ("T", -1, 2), ("K", 0, 2), ("chunk", 0, 2),
])
def test_bad_problem_rejected(lib, gdn, field, value, status):
    pr = _problem(gdn)
    setattr(pr, field, value)
    assert _fwd(lib, pr) == status
    assert lib.gdn_workspace_bytes(ctypes.byref(pr)) == 0


def test_fp32_io_with_bf16_output_rejected(lib, gdn):
    assert _fwd(lib, _problem(gdn, io=0, o=1)) == 3


def test_null_problem_and_pointers(lib, gdn):
    assert lib.gdn_forward(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                           FAKE, ctypes.c_size_t(1 << 40), None) == 1
    pr = _problem(gdn)
    for name in ("q", "k", "v", "beta", "g", "o"):
        assert _fwd(lib, pr, **{name: None}) == 1, name
    assert lib.gdn_prepare(ctypes.byref(pr), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                           None) == 1
    assert lib.gdn_scan(ctypes.byref(pr), FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                        None, None) == 1


def test_alignment_rejected(lib, gdn):
    pr = _problem(gdn)
    assert _fwd(lib, pr, q=MISALIGNED) == 4
    assert _fwd(lib, pr, h0=MISALIGNED) == 4
    assert _fwd(lib, pr, hT=MISALIGNED) == 4


def test_workspace_sizes(lib, gdn):
    # the scalar gate keeps every intermediate on chip; the per-key gate's
    # kernel over all chunks leaves a slot per (chunk, head) in the
    # workspace: Tmb and P ([C][C] each, operand type) and, with bf16 io, the
    # re-scan's operand tiles ([C][K] fp16, three) and e^gl ([K] fp32)
    for io, slot in ((1, 2 * 64 * 64 * 2 + 3 * 64 * 64 * 2 + 64 * 4), (0, 2 * 64 * 64 * 4)):
        pr = _problem(gdn, B=2, T=100, H=3, K=64, V=128, gate=0, io=io, o=io)
        assert lib.gdn_workspace_bytes(ctypes.byref(pr)) == 0
        assert lib.gdn_workspace_bytes_varlen(ctypes.byref(pr), ctypes.c_int64(4)) == 0
        pr = _problem(gdn, B=2, T=100, H=3, K=64, V=128, gate=1, io=io, o=io)
        assert lib.gdn_workspace_bytes(ctypes.byref(pr)) == 2 * 2 * 3 * slot
        pr1 = _problem(gdn, B=1, T=100, H=3, K=64, V=128, gate=1, io=io, o=io)
        assert lib.gdn_workspace_bytes_varlen(ctypes.byref(pr1), ctypes.c_int64(4)) == \
            (2 + 4) * 3 * slot
        assert lib.gdn_workspace_bytes_varlen(ctypes.byref(pr1), ctypes.c_int64(0)) == 0
    # T = 0: nothing to form
    assert lib.gdn_workspace_bytes(ctypes.byref(_problem(gdn, T=0, gate=1))) == 0


def test_key_gate_workspace_checked_before_launch(lib, gdn):
    pr = _problem(gdn, B=1, T=200, H=2, K=128, V=128, gate=1)
    need = lib.gdn_workspace_bytes(ctypes.byref(pr))
    assert need > 0
    assert _fwd(lib, pr, ws=None, ws_bytes=0) == 6
    assert _fwd(lib, pr, ws_bytes=need - 1) == 6
    assert _fwd(lib, pr, ws=MISALIGNED, ws_bytes=need) == 4
    assert _fwd_states(lib, pr, ws=None, ws_bytes=0) == 6
    assert _rescan(lib, pr, ws_bytes=need - 16) == 6
    pv = _problem(gdn, B=1, T=200, H=2, K=128, V=128, gate=1)
    needv = lib.gdn_workspace_bytes_varlen(ctypes.byref(pv), ctypes.c_int64(2))
    assert _fwd_varlen(lib, pv, ws_bytes=needv - 1) == 6
    # fp32 io at K = 128, chunk 64 (the four-wave kernel without its own
    # Gram tiles) now fits; it asks for its workspace like any other shape
    p32 = _problem(gdn, io=0, o=0, gate=1, K=128, V=128, chunk=64)
    assert _fwd(lib, p32, ws=None, ws_bytes=0) == 6
    assert _fwd_states(lib, p32, ws=None, ws_bytes=0) == 6


def test_noalloc_refuses_oversize_before_launch(lib, gdn):
    # the static scratch holds GDN_NOALLOC_SCRATCH_BYTES; a per-key problem
    # that needs more is refused before the device is touched
    C, K = 64, 128
    per = 2 * C * C * 2 + 3 * C * K * 2 + K * 4          # bf16 io slot bytes
    nt = gdn.NOALLOC_SCRATCH_BYTES // per
    fits = _problem(gdn, B=1, T=nt * C, H=1, K=K, V=128, gate=1, chunk=C)
    assert lib.gdn_workspace_bytes(ctypes.byref(fits)) == nt * per <= gdn.NOALLOC_SCRATCH_BYTES
    over = _problem(gdn, B=1, T=nt * C + 1, H=1, K=K, V=128, gate=1, chunk=C)
    assert lib.gdn_workspace_bytes(ctypes.byref(over)) > gdn.NOALLOC_SCRATCH_BYTES
    st = lib.gdn_forward_noalloc(ctypes.byref(over), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                 None, None)
    assert st == 6
    assert lib.gdn_forward_noalloc(ctypes.byref(over), None, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                   None, None) == 1


def _split(lib, pr, t_split, ws=FAKE, ws_bytes=1 << 40, h0=None, hT=None):
    return lib.gdn_forward_split(ctypes.byref(pr), ctypes.c_int64(t_split), FAKE, FAKE, FAKE, FAKE,
                                 FAKE, h0, FAKE, hT, ws, ctypes.c_size_t(ws_bytes), None)


def test_split_forward_checks(lib, gdn):
    pr = _problem(gdn, B=2, T=300, H=4, K=128, V=64, chunk=64)
    need = lib.gdn_workspace_bytes_split(ctypes.byref(pr), ctypes.c_int64(192))
    assert need == 2 * 4 * 128 * 64 * 4 * 3 + 2 * 4 * 128 * 128 * 4 + 2 * (300 - 192) * 4 * 128 * 2
    assert _split(lib, pr, 192, ws=None, ws_bytes=0) == 1
    assert _split(lib, pr, 192, ws_bytes=need - 1) == 6
    for bad in (0, 300, 100, -64, 320):
        assert _split(lib, pr, bad) == 2, bad
        assert lib.gdn_workspace_bytes_split(ctypes.byref(pr), ctypes.c_int64(bad)) == 0
    # scalar gate, bf16 io and chunk 64 only
    assert _split(lib, _problem(gdn, T=300, gate=1), 128) == 3
    assert _split(lib, _problem(gdn, T=300, io=0, o=0), 128) == 3
    assert _split(lib, _problem(gdn, T=300, chunk=32), 128) == 3
    assert _split(lib, pr, 192, h0=MISALIGNED) == 4


def _bwd(lib, pr, ws=FAKE, ws_bytes=1 << 40, **kw):
    names = ("q", "k", "v", "beta", "g", "dout", "dhT", "hck", "vnew", "dq", "dk", "dv", "dbeta",
             "dg", "dh0")
    args = [kw.get(n, None if n in ("dhT", "dh0") else FAKE) for n in names]
    return lib.gdn_backward(ctypes.byref(pr), *args, ws, ctypes.c_size_t(ws_bytes), None)


def test_backward_checks(lib, gdn):
    pr = _problem(gdn, B=2, T=300, H=4, K=128, V=64, chunk=64)
    need = lib.gdn_workspace_bytes_backward(ctypes.byref(pr))
    assert need == 2 * 300 * 4 * 64 * 4 + 2 * 5 * 4 * 128 * 64 * 4 + 2 * 5 * 4 * (8 * 64 * 64 + 16 * 64 + 16)
    assert _bwd(lib, pr, ws=None, ws_bytes=0) == 6
    assert _bwd(lib, pr, ws_bytes=need - 1) == 6
    assert _bwd(lib, pr, ws=MISALIGNED) == 4
    for name in ("q", "k", "v", "beta", "g", "dout", "hck", "vnew", "dq", "dk", "dv", "dbeta", "dg"):
        assert _bwd(lib, pr, **{name: None}) == 1, name
        assert _bwd(lib, pr, **{name: MISALIGNED}) == 4, name
    for name in ("dhT", "dh0"):
        assert _bwd(lib, pr, **{name: MISALIGNED}) == 4, name
    # the per-key gate's workspace also holds Gamma per key in its slots and
    # dP, dA per (chunk, head)
    prk = _problem(gdn, B=2, T=300, H=4, K=128, V=64, chunk=64, gate=1)
    slot = 8 * 64 * 64 + 64 * 128 * 4 + 64 * 4 + 128 * 4
    assert lib.gdn_workspace_bytes_backward(ctypes.byref(prk)) == (
        2 * 300 * 4 * 64 * 4 + 2 * 5 * 4 * 128 * 64 * 4 + 2 * 5 * 4 * slot + 2 * 5 * 4 * 2 * 64 * 64 * 4)
    # bf16 io and bf16 saved states only
    assert _bwd(lib, _problem(gdn, T=300, io=0, o=0)) == 3
    assert _bwd(lib, _problem(gdn, T=300, o=0)) == 3
    assert _bwd(lib, _problem(gdn, K=96)) == 3
    assert lib.gdn_workspace_bytes_backward(None) == 0
    # an fp32 row of a stream past 4 GiB
    assert _bwd(lib, _problem(gdn, T=1 << 22, H=512, K=128, V=128)) == 3


def test_lds_budget_reported_before_launch(lib, gdn):
    # fp32 operands at K = 128 with 64-token chunks need more than 160 KiB of
    # LDS in the scan: reported as a status, never attempted.
    pr = _problem(gdn, B=1, T=0, H=1, K=128, V=128, chunk=64, io=0, o=0)
    pr.T = 64
    st = lib.gdn_scan(ctypes.byref(pr), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                      None, None)
    assert st == 5


def _fwd_states(lib, pr, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, h0=None, o=FAKE,
                hT=None, hck=FAKE, vnew=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.gdn_forward_states(ctypes.byref(pr), q, k, v, beta, g, h0, o, hT, hck,
                                  vnew, ws, ctypes.c_size_t(ws_bytes), None)


def test_forward_states_validates_before_launch(lib, gdn):
    pr = _problem(gdn)
    for name in ("q", "k", "v", "beta", "g", "o", "hck", "vnew"):
        assert _fwd_states(lib, pr, **{name: None}) == 1, name
    for name in ("q", "o", "hck", "vnew", "h0", "hT"):
        assert _fwd_states(lib, pr, **{name: MISALIGNED}) == 4, name
    bad = _problem(gdn, K=96)
    assert _fwd_states(lib, bad) == 3
    assert lib.gdn_forward_states(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                  FAKE, FAKE, FAKE, ctypes.c_size_t(0), None) == 1


def test_forward_states_empty_sequence_needs_no_buffers(lib, gdn):
    # T = 0 with no final state requested: nothing to write, nothing enqueued
    pr = _problem(gdn, T=0)
    assert _fwd_states(lib, pr, q=None, k=None, v=None, beta=None, g=None, o=None,
                       hck=None, vnew=None) == 0


def _fwd_varlen(lib, pr, cu=FAKE, n=2, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, h0=None,
                o=FAKE, hT=None, ws=FAKE, ws_bytes=1 << 40):
    return lib.gdn_forward_varlen(ctypes.byref(pr), cu, ctypes.c_int64(n), q, k, v, beta, g,
                                  h0, o, hT, ws, ctypes.c_size_t(ws_bytes), None)


def test_forward_varlen_validates_before_launch(lib, gdn):
    pr = _problem(gdn, B=1, T=200)
    assert _fwd_varlen(lib, pr, cu=None) == 1
    assert _fwd_varlen(lib, pr, cu=ctypes.c_void_p(0x10002)) == 4
    assert _fwd_varlen(lib, _problem(gdn, B=2, T=200)) == 2     # packed means B = 1
    assert _fwd_varlen(lib, pr, n=0) == 2
    assert _fwd_varlen(lib, pr, n=(1 << 24) + 1) == 2
    for name in ("q", "k", "v", "beta", "g", "o"):
        assert _fwd_varlen(lib, pr, **{name: None}) == 1, name
    assert _fwd_varlen(lib, pr, h0=MISALIGNED) == 4
    assert _fwd_varlen(lib, _problem(gdn, B=1, T=200, K=96)) == 3
    # no tokens and no final state: nothing to do
    assert _fwd_varlen(lib, _problem(gdn, B=1, T=0), q=None, k=None, v=None, beta=None,
                       g=None, o=None) == 0


def test_streams_beyond_32bit_offsets_rejected(lib, gdn):
    # one (batch, head) stream of q addressed with 32-bit byte offsets: T*H*K*2
    # bytes must stay below 4 GiB; 2^20 tokens of 16 heads of 128 reach it
    pr = _problem(gdn, B=1, T=1 << 20, H=16, K=128, V=128)
    assert _fwd(lib, pr) == 3
    assert _fwd_states(lib, pr) == 3
    assert _fwd_varlen(lib, pr) == 3
    # one token fewer fits
    ok = _problem(gdn, B=1, T=(1 << 20) - 1, H=16, K=128, V=128)
    assert lib.gdn_workspace_bytes(ctypes.byref(ok)) == 0


def _rescan(lib, pr, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, h0=None, do=FAKE, hT=None,
            hck=FAKE, vnew=FAKE, dq=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.gdn_rescan_dq(ctypes.byref(pr), q, k, v, beta, g, h0, do, hT, hck, vnew, dq,
                             ws, ctypes.c_size_t(ws_bytes), None)


def test_rescan_dq_validates_before_launch(lib, gdn):
    pr = _problem(gdn)
    for name in ("q", "k", "v", "beta", "g", "do", "hck", "vnew", "dq"):
        assert _rescan(lib, pr, **{name: None}) == 1, name
    assert _rescan(lib, pr, dq=MISALIGNED) == 4
    assert _rescan(lib, _problem(gdn, io=0, o=0)) == 3        # bf16 io only
    assert _rescan(lib, _problem(gdn, T=0), q=None, k=None, v=None, beta=None, g=None, do=None,
                   hck=None, vnew=None, dq=None) == 0


def test_rescan_dq_is_not_routed_to_the_four_wave_kernel(lib, gdn, monkeypatch):
    # with the pipelined kernels switched off for bf16 io, the re-scan has no
    # kernel: it returns GDN_ERR_UNSUPPORTED before any launch instead of
    # running a forward that leaves dq untouched
    monkeypatch.setenv("GDN_FORWARD_FOUR_WAVE", "1")
    assert _rescan(lib, _problem(gdn)) == 3
    assert _rescan(lib, _problem(gdn, gate=1)) == 3



def _chunk_dq(lib, pr, do=FAKE, hck=FAKE, dq=FAKE):
    return lib.gdn_chunk_dq(ctypes.byref(pr), do, hck, dq, None)


def test_chunk_dq_validates_before_launch(lib, gdn):
    pr = _problem(gdn)
    for name in ("do", "hck", "dq"):
        assert _chunk_dq(lib, pr, **{name: None}) == 1, name
    assert _chunk_dq(lib, pr, dq=MISALIGNED) == 4
    assert _chunk_dq(lib, pr, hck=MISALIGNED) == 4
    assert _chunk_dq(lib, _problem(gdn, io=0, o=0)) == 3        # bf16 dO only
    assert _chunk_dq(lib, _problem(gdn, K=96)) == 3
    assert _chunk_dq(lib, _problem(gdn, chunk=16)) == 3
    # a chunk's rows of 2^17 heads of fp32 dq pass 32-bit offsets
    assert _chunk_dq(lib, _problem(gdn, B=1, T=64, H=1 << 17, K=128, V=128)) == 3
    # no tokens: nothing to do, no buffers needed
    assert _chunk_dq(lib, _problem(gdn, T=0), do=None, hck=None, dq=None) == 0


def test_wait_timeouts_rejects_null(lib, gdn):
    # validated before the device word is touched: no GPU needed
    assert lib.gdn_wait_timeouts(None, 0) == 1


def test_forward_split_point(lib, gdn, monkeypatch):
    """Where gdn_forward cuts its streams: F = B H V/64 single-pass streams
    leave 256 - F compute units idle; the second segment's S = B H (V/64 +
    K/64) streams run there in R = ceil(S / (256 - F)) rounds, so the cut is
    T R / (R + 1) rounded to a chunk; only for the scalar gate, bf16 io,
    chunk 64, and R = 1 from 128 chunks or R = 2 from 256 chunks."""
    monkeypatch.delenv("GDN_FORWARD_NO_SPLIT", raising=False)
    sp = lambda **kw: lib.gdn_forward_split_point(ctypes.byref(_problem(gdn, **kw)))
    big = dict(B=1, T=65536, H=64, K=128, V=128)
    # F = 128, S = 256: R = 2, 2/3 of 65536 = 43690.7 -> 683 chunks
    assert sp(**big) == 683 * 64
    assert sp(B=1, T=16384, H=64, K=128, V=128) == 171 * 64          # 10922.7 -> 171 chunks
    assert sp(B=1, T=16384 - 64, H=64, K=128, V=128) == 0            # 255 chunks at R = 2
    assert sp(B=1, T=8192, H=8, K=128, V=128) == 4096                # F = 16, S = 32: R = 1
    assert sp(B=1, T=8192 - 64, H=8, K=128, V=128) == 0              # 127 chunks
    assert sp(B=4, T=4096, H=16, K=128, V=128) == 0                  # 64 chunks
    assert sp(B=1, T=65536, H=128, K=128, V=128) == 0                # F = 256: no idle unit
    assert sp(B=1, T=65536, H=96, K=128, V=128) == 0                 # F = 192: R = 6
    assert sp(B=1, T=65536, H=64, K=64, V=128) == 683 * 64           # S = 192: R = 2
    assert sp(B=1, T=65536, H=64, K=128, V=64) == 32768              # F = 64, S = 192: R = 1, T / 2
    assert sp(B=1, T=65537, H=8, K=128, V=128) == 32768              # a ragged last chunk
    for kw in (dict(chunk=32), dict(io=0, o=0), dict(gate=1)):
        assert sp(**big, **kw) == 0, kw
    assert lib.gdn_forward_split_point(None) == 0
    # the workspace gdn_forward asks for is the split's
    pr = _problem(gdn, **big)
    assert lib.gdn_workspace_bytes(ctypes.byref(pr)) == lib.gdn_workspace_bytes_split(
        ctypes.byref(pr), ctypes.c_int64(683 * 64)) > 0
    monkeypatch.setenv("GDN_FORWARD_NO_SPLIT", "1")
    assert sp(**big) == 0 and lib.gdn_workspace_bytes(ctypes.byref(pr)) == 0
