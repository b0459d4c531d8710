"""GPU parity of gdn_rescan_dq (the backward's forward re-scan, through the C
ABI) against the fp64 oracle, for the scalar gate and the per-key gate.

dq's chunk-start-state term dq[t] = h_c dO_t, the chunk-start states and v'
are held to the forward's bar: max |x - x_ref| / rms(x_ref) <= 2e-2 with bf16
inputs for fp32 outputs (dq is always fp32).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs, WORKLOADS

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _np(t):
    return t.detach().float().cpu().numpy()


def _dout(B, T, H, V, seed):
    gen = torch.Generator().manual_seed(int(seed))
    return torch.randn(B, T, H, V, generator=gen).to(torch.bfloat16).contiguous()


def run_rescan(case, B, T, H, K, V, C, h0, seed, heads=None, gate="head", bias=2.0):
    inp = make_inputs(B, T, H, K, V, io="bf16", gate=gate, gate_bias=bias, h0=h0, seed=seed)
    do = _dout(B, T, H, V, seed + 1)
    d = {n: (None if t is None else t.to(_dev())) for n, t in inp.items()}
    print("case", case, [B, T, H, K, V, C], gate, flush=True)
    hT, hck, vnew, dq = gdn.rescan_dq(d["q"], d["k"], d["v"], d["beta"], d["g"], do.to(_dev()),
                                      C, d["h0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    _, h_ref, ck_ref, vn_ref = oracle.token_states(
        inp["q"].float().numpy(), inp["k"].float().numpy(), inp["v"].float().numpy(),
        inp["beta"].numpy(), inp["g"].numpy(), C,
        None if inp["h0"] is None else inp["h0"].numpy(), heads=heads)
    if heads is None:
        dq_ref = oracle.rescan_dq(ck_ref, do.float().numpy(), C)
        got = dict(dq=_np(dq), hT=_np(hT), hck=_np(hck), vnew=_np(vnew))
    else:
        # head-major references: [n,NT,K,V] states, dO of the same heads
        dsel = np.stack([do[bh // H, :, bh % H].float().numpy() for bh in heads])  # [n,T,V]
        dq_ref = oracle.rescan_dq(ck_ref[:, :, None], dsel[:, :, None], C)[:, :, 0]
        got = dict(dq=np.stack([_np(dq[bh // H, :, bh % H]) for bh in heads]),
                   hT=np.stack([_np(hT[bh // H, bh % H]) for bh in heads]),
                   hck=np.stack([_np(hck[bh // H, :, bh % H]) for bh in heads]),
                   vnew=np.stack([_np(vnew[bh // H, :, bh % H]) for bh in heads]))
    for name, ref in (("dq", dq_ref), ("hT", h_ref), ("hck", ck_ref), ("vnew", vn_ref)):
        rel = oracle.rel_err(got[name], ref)
        print("  %s rel %.3e" % (name, rel), flush=True)
        assert rel <= TOL, "%s %s rel err %.3e" % (case, name, rel)
    return d, do, dq


CASES = [
    # B, T, H, K, V, chunk, h0, gate
    (2, 333, 2, 128, 128, 64, True, "head"),
    (1, 200, 3, 64, 64, 32, False, "head"),
    (1, 130, 2, 128, 64, 64, True, "head"),       # one V tile
    (1, 97, 2, 64, 128, 32, True, "head"),        # dk != dv
    (1, 1, 1, 128, 128, 64, True, "head"),        # a single token
    (2, 300, 2, 128, 128, 64, True, "key"),
    (1, 200, 3, 64, 64, 64, False, "key"),
    (1, 130, 2, 128, 64, 64, True, "key"),        # one V tile, ragged tail
    (1, 97, 2, 64, 128, 64, True, "key"),         # dk != dv
    (1, 1, 1, 128, 128, 64, True, "key"),         # a single token
    (2, 200, 2, 128, 128, 32, True, "key"),       # chunk 32: the state staged on its own
    (1, 111, 3, 64, 128, 32, False, "key"),
    (1, 77, 2, 128, 64, 32, True, "key"),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "B%dT%dH%dK%dV%dC%d_%s" % (c[:6] + c[7:]))
def test_rescan_dq_small(cfg):
    B, T, H, K, V, C, h0, gate = cfg
    run_rescan("rescan_small", B, T, H, K, V, C, h0, seed=T + K + 3, gate=gate,
               bias=3.0 if gate == "key" else 2.0)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_rescan_dq_accumulates_and_is_deterministic(gate):
    d, do, dq = run_rescan("rescan_acc", 1, 256, 2, 128, 128, 64, True, seed=77, gate=gate,
                           bias=3.0)
    do = do.to(_dev())
    base = torch.full_like(dq, 0.25)
    _, _, _, dq2 = gdn.rescan_dq(d["q"], d["k"], d["v"], d["beta"], d["g"], do, 64, d["h0"],
                                 o_dtype=torch.float32, dq=base)
    _, _, _, dq3 = gdn.rescan_dq(d["q"], d["k"], d["v"], d["beta"], d["g"], do, 64, d["h0"],
                                 o_dtype=torch.float32)
    torch.cuda.synchronize()
    # the two V tiles add into dq in either order: the same bits every run
    assert torch.equal(dq3, dq)
    assert torch.allclose(dq2 - 0.25, dq, rtol=0, atol=1e-5)


@pytest.mark.parametrize("name", ["gdn_t4k", "gdn_c32_d64", "kda_t8k"])
def test_rescan_dq_full_size_sampled(name):
    w = WORKLOADS[name]
    pairs = w.B * w.H
    run_rescan("rescan_full_" + name, w.B, w.T, w.H, w.K, w.V, w.chunk, w.h0, w.seed,
               heads=[0, (7 * pairs) // 11, pairs - 1], gate=w.gate, bias=w.gate_bias)
