"""The debug build and the launch trace.

libgdn_poison.so is libgdn built with GDN_POISON_LDS: each pipelined kernel
fills an LDS stage with NaN as soon as its last reader is done with it (the
chain's operand slot at the end of its chunk, the prepare's row factors, split
A blocks and fp16 diagonal inverses at the end of its prepare).  A read that
runs ahead of the write it must wait for -- a missing or misplaced barrier or
arrival count -- then returns NaN instead of the previous chunk's values.
With every wait in place the debug build computes exactly what the production
build computes, so the tests compare the two bit for bit, over enough chunks
for the two-slot LDS ring to wrap several times (NT >= 6, three times its
depth), for both gates, both chunk sizes and both key sizes, the instances
that save states and read packed sequences, and also check the outputs
against the oracle.

GDN_TRACE=1 prints each entry point's problem and each launch's plan (kernel
instance, grid, workgroup, LDS, registers, scratch) to stderr.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def poison_lib():
    assert os.path.exists(gdn.POISON_LIB_PATH), "the debug library is built beside libgdn.so"
    return gdn.load_library(gdn.POISON_LIB_PATH)


def _inputs(B, T, H, K, V, gate, seed):
    inp = make_inputs(B, T, H, K, V, io="bf16", gate=gate, gate_bias=2.0 if gate == "head" else 3.0,
                      h0=True, seed=seed)
    d = _dev()
    return inp, {k: (None if v is None else v.to(d)) for k, v in inp.items()}


def _same(a, b, what):
    assert a.dtype == b.dtype and a.shape == b.shape, what
    assert torch.isfinite(a.float()).all(), "%s: non-finite values in the debug build" % what
    assert torch.equal(a, b), "%s: debug build differs from libgdn (max |diff| %.3e)" % (
        what, (a.float() - b.float()).abs().max().item())


CASES = [("head", 128, 128, 64), ("head", 64, 64, 32), ("head", 128, 64, 32),
         ("key", 128, 128, 64), ("key", 64, 128, 32)]


@pytest.mark.parametrize("gate,K,V,C", CASES, ids=lambda c: str(c))
def test_poison_build_matches_production(poison_lib, gate, K, V, C):
    B, T, H = 2, 6 * C + 19, 2
    inp, d = _inputs(B, T, H, K, V, gate, seed=5 + K + C)
    for od in (torch.bfloat16, torch.float32):
        ref = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"], o_dtype=od)
        got = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"], o_dtype=od,
                          library=poison_lib)
        torch.cuda.synchronize()
        _same(got[0], ref[0], "o (%s)" % od)
        _same(got[1], ref[1], "hT (%s)" % od)
    o_ref, h_ref = oracle.token_recurrence(inp["q"].float().numpy(), inp["k"].float().numpy(),
                                           inp["v"].float().numpy(), inp["beta"].numpy(),
                                           inp["g"].numpy(), inp["h0"].numpy())
    assert oracle.rel_err(got[0].cpu().numpy(), o_ref) <= 2e-2
    assert oracle.rel_err(got[1].cpu().numpy(), h_ref) <= 2e-2


@pytest.mark.parametrize("gate", ["head", "key"])
def test_poison_build_states_and_packed_sequences(poison_lib, gate):
    K = V = 128
    C = 64
    B, T, H = 1, 7 * C + 5, 2
    inp, d = _inputs(B, T, H, K, V, gate, seed=17)
    ref = gdn.forward_states(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"])
    got = gdn.forward_states(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"], library=poison_lib)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "hT", "hck", "vnew"), got, ref):
        _same(a, b, "states " + name)
    # three packed sequences, one shorter than a chunk
    cu = torch.tensor([0, 3 * C + 7, 3 * C + 7 + 40, T], dtype=torch.int32, device=_dev())
    h0n = torch.randn(3, H, K, V, device=_dev()) * 0.1
    ref = gdn.forward_varlen(d["q"], d["k"], d["v"], d["beta"], d["g"], cu, C, h0n)
    got = gdn.forward_varlen(d["q"], d["k"], d["v"], d["beta"], d["g"], cu, C, h0n, library=poison_lib)
    torch.cuda.synchronize()
    _same(got[0], ref[0], "varlen o")
    _same(got[1], ref[1], "varlen hT")


def test_trace_prints_the_plan(monkeypatch, capfd):
    B, T, H, K, V, C = 1, 130, 2, 128, 128, 64
    _, d = _inputs(B, T, H, K, V, "head", seed=3)
    _, dk = _inputs(B, T, H, K, V, "key", seed=4)
    monkeypatch.delenv("GDN_TRACE", raising=False)
    capfd.readouterr()
    gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"])
    torch.cuda.synchronize()
    assert "gdn_trace" not in capfd.readouterr().err
    monkeypatch.setenv("GDN_TRACE", "1")
    gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"])
    gdn.forward(dk["q"], dk["k"], dk["v"], dk["beta"], dk["g"], C, dk["h0"])
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    lines = [x for x in err.splitlines() if x.startswith("gdn_trace")]
    entries = [x for x in lines if x.startswith("gdn_trace gdn_forward:")]
    assert len(entries) == 2, err
    assert "B=1 T=130 H=2 K=128 V=128 chunk=64 io=bf16 o=bf16 gate=head V tiles=2 status=0" in entries[0]
    assert "gate=key" in entries[1]
    launches = [x for x in lines if " launch " in x]
    # the scalar gate: one pipelined launch of B * H * V/64 workgroups of 512
    # threads; the per-key gate: the Gram kernel, then its pipelined re-scan
    assert "forward_pipe_kernel<64, 128" in launches[0] and "grid=4 block=512" in launches[0], launches
    assert "kda_gram_kernel<64, 128" in launches[1], launches
    assert "forward_pipe_kda_kernel<64, 128" in launches[2] and "grid=4" in launches[2], launches
    for x in launches:
        lds = int(x.split("lds=")[1].split()[0])
        regs = int(x.split("regs=")[1].split()[0])
        assert lds > 0 and regs > 0 and "scratch=0" in x, x
    monkeypatch.setenv("GDN_TRACE", "0")
    gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"])
    torch.cuda.synchronize()
    assert "gdn_trace" not in capfd.readouterr().err
