"""GPU parity of gdn_chunk_dq (dq's chunk-start-state term from saved states,
through the C ABI) against the fp64 oracle.

The inputs are seeded synthetic states and dO (the kernel takes any states),
so the oracle sees exactly what the kernel sees.  Bar: max |dq - dq_ref| /
rms(dq_ref) <= 1e-4 (bf16 states multiply exactly and accumulate in fp32;
fp32 states enter as bf16 high and low parts, ~16 bits).  The end-to-end
check against gdn_rescan_dq, which forms the same term fused into the
re-scan, is held to the same bar with fp32 states on both sides.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs, WORKLOADS

pytestmark = pytest.mark.gpu

TOL = 1e-4
TDT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _np(t):
    return t.detach().float().cpu().numpy()


def _synthetic(B, T, H, K, V, C, hdt, seed):
    gen = torch.Generator().manual_seed(int(seed))
    nt = (T + C - 1) // C
    hck = (0.5 * torch.randn(B, nt, H, K, V, generator=gen)).to(TDT[hdt]).contiguous()
    do = torch.randn(B, T, H, V, generator=gen).to(torch.bfloat16).contiguous()
    return hck, do


CASES = [
    # B, T, H, K, V, chunk, state dtype
    (2, 333, 3, 128, 128, 64, "bf16"),
    (1, 200, 2, 64, 64, 32, "fp32"),
    (1, 97, 2, 128, 64, 32, "bf16"),       # dk != dv, ragged tail
    (1, 130, 4, 64, 128, 64, "fp32"),      # dv > dk
    (3, 64, 2, 128, 128, 64, "fp32"),      # one whole chunk
    (1, 1, 1, 128, 128, 64, "bf16"),       # a single token
    (2, 31, 5, 64, 64, 32, "bf16"),        # shorter than a chunk
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "B%dT%dH%dK%dV%dC%d_%s" % c)
def test_chunk_dq_matches_oracle(cfg):
    B, T, H, K, V, C, hdt = cfg
    print("case chunk_dq", cfg, flush=True)
    hck, do = _synthetic(B, T, H, K, V, C, hdt, seed=B * 100 + T + K + V + C)
    dev = _dev()
    # a dq full of garbage: the call writes every element
    dq0 = torch.full((B, T, H, K), float("nan"), device=dev)
    dq = gdn.chunk_dq(do.to(dev), hck.to(dev), C, dq=dq0)
    torch.cuda.synchronize()
    ref = oracle.rescan_dq(hck.double().numpy(), do.double().numpy(), C)
    got = _np(dq)
    assert np.isfinite(got).all()
    rel = oracle.rel_err(got, ref)
    print("  dq rel %.3e" % rel, flush=True)
    assert rel <= TOL


def test_chunk_dq_is_deterministic_and_empty_is_a_no_op():
    hck, do = _synthetic(2, 300, 4, 128, 128, 64, "bf16", seed=5)
    dev = _dev()
    a = gdn.chunk_dq(do.to(dev), hck.to(dev), 64)
    b = gdn.chunk_dq(do.to(dev), hck.to(dev), 64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    e = gdn.chunk_dq(torch.empty(1, 0, 2, 64, device=dev, dtype=torch.bfloat16),
                     torch.empty(1, 0, 2, 64, 64, device=dev), 64)
    torch.cuda.synchronize()
    assert e.shape == (1, 0, 2, 64)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_forward_states_then_chunk_dq_is_the_fused_rescan(gate):
    # the unfused pair (saved states, then the product) and the fused
    # re-scan form the same term; fp32 states on both sides
    B, T, H, K, V, C = 1, 300, 2, 128, 128, 64
    inp = make_inputs(B, T, H, K, V, io="bf16", gate=gate, gate_bias=3.0, h0=True, seed=41)
    d = {n: t.to(_dev()) for n, t in inp.items()}
    gen = torch.Generator().manual_seed(42)
    do = torch.randn(B, T, H, V, generator=gen).to(torch.bfloat16).to(_dev())
    _, _, hck, _ = gdn.forward_states(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"],
                                      o_dtype=torch.float32)
    _, hck2, _, dq_fused = gdn.rescan_dq(d["q"], d["k"], d["v"], d["beta"], d["g"], do, C,
                                         d["h0"], o_dtype=torch.float32)
    # the product itself, on the fused kernel's own states
    dq_unfused = gdn.chunk_dq(do, hck2, C)
    dq_states = gdn.chunk_dq(do, hck, C)
    torch.cuda.synchronize()
    rel = oracle.rel_err(_np(dq_unfused), _np(dq_fused))
    print("fused vs unfused dq rel %.3e" % rel, flush=True)
    assert rel <= TOL
    # the two kernels' states are separately compiled instances of the
    # re-scan, whose fp32 roundings may differ and travel through the fp16
    # operands: a quarter of the forward's 2e-2 bar, as for o and hT
    assert oracle.rel_err(_np(hck2), _np(hck)) <= 5e-3
    assert oracle.rel_err(_np(dq_states), _np(dq_fused)) <= 5e-3


@pytest.mark.parametrize("name", ["gdn_t4k", "gdn_c32_d64"])
def test_chunk_dq_full_size_sampled(name):
    # the workload's shapes, synthetic bf16 states; the oracle on three heads
    w = WORKLOADS[name]
    print("case chunk_dq_full", name, flush=True)
    hck, do = _synthetic(w.B, w.T, w.H, w.K, w.V, w.chunk, "bf16", seed=w.seed)
    dq = gdn.chunk_dq(do.to(_dev()), hck.to(_dev()), w.chunk)
    torch.cuda.synchronize()
    pairs = w.B * w.H
    for bh in sorted(set([0, (7 * pairs) // 11, pairs - 1])):
        b, h = bh // w.H, bh % w.H
        ref = oracle.rescan_dq(hck[b:b + 1, :, h:h + 1].double().numpy(),
                               do[b:b + 1, :, h:h + 1].double().numpy(), w.chunk)
        rel = oracle.rel_err(_np(dq[b:b + 1, :, h:h + 1]), ref)
        print("  head", bh, "dq rel %.3e" % rel, flush=True)
        assert rel <= TOL
