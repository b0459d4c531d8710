"""GPU parity of gdn_forward_states (through the C ABI) against the fp64 oracle.

The saved states are the chunk-start states hck [B,NT,H,K,V] and the
per-token deltas vnew [B,T,H,V] that a backward pass re-reads.  They are
held to the same bar as o and the final state: max |x - x_ref| / rms(x_ref)
<= 2e-2 with bf16 inputs, <= 1e-4 with fp32 inputs, for fp32 outputs; bf16
outputs element by element within 2e-2 rms(x_ref) + half a bf16 ulp.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs, WORKLOADS

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}
TDT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _np(t):
    return t.detach().float().cpu().numpy()


def _half_ulp_bf16(x):
    a = np.abs(np.asarray(x, np.float64))
    return np.exp2(np.floor(np.log2(np.maximum(a, 1e-38))) - 8)


def _check(name, got, ref, io, out_dtype, case):
    rel = oracle.rel_err(got, ref)
    if out_dtype == "bf16":
        rms = math.sqrt(float(np.mean(ref ** 2))) if ref.size else 0.0
        slack = TOL[io] * rms + _half_ulp_bf16(np.maximum(np.abs(ref), np.abs(got)))
        bad = np.abs(got - ref) > slack
        assert not bad.any(), "%s %s: %d bf16 elements outside the bound (rel %.3e)" % (
            case, name, int(bad.sum()), rel)
    else:
        assert rel <= TOL[io], "%s %s: rel err %.3e > %.1e" % (case, name, rel, TOL[io])
    print(case, name, out_dtype, "rel %.3e" % rel, flush=True)
    return rel


def run_states(case, B, T, H, K, V, chunk, io, gate, bias, h0, seed, o_dtypes, heads=None):
    inp = make_inputs(B, T, H, K, V, io=io, gate=gate, gate_bias=bias, h0=h0, seed=seed)
    d = {k: (None if v is None else v.to(_dev())) for k, v in inp.items()}
    o_ref, h_ref, ck_ref, vn_ref = oracle.token_states(
        inp["q"].float().numpy(), inp["k"].float().numpy(), inp["v"].float().numpy(),
        inp["beta"].numpy(), inp["g"].numpy(), chunk,
        None if inp["h0"] is None else inp["h0"].numpy(), heads=heads)
    NT = (T + chunk - 1) // chunk
    for od in o_dtypes:
        print("case", case, [B, T, H, K, V, chunk], io, gate, od, flush=True)
        o, hT, hck, vnew = gdn.forward_states(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                              chunk, d["h0"], o_dtype=TDT[od])
        o2, h2 = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], chunk, d["h0"],
                             o_dtype=TDT[od])
        torch.cuda.synchronize()
        assert tuple(hck.shape) == (B, NT, H, K, V)
        # the states instance computes o and hT with the plain forward's
        # arithmetic in the same order (it only adds the checkpoint and v'
        # stores), so the two agree bit for bit; each is also checked against
        # the oracle below
        assert torch.equal(o, o2), (case, (o.float() - o2.float()).abs().max().item())
        assert torch.equal(hT, h2), (case, (hT - h2).abs().max().item())
        if heads is not None:
            og = np.stack([_np(o[bh // H, :, bh % H]) for bh in heads])
            hg = np.stack([_np(hT[bh // H, bh % H]) for bh in heads])
            cg = np.stack([_np(hck[bh // H, :, bh % H]) for bh in heads])
            vg = np.stack([_np(vnew[bh // H, :, bh % H]) for bh in heads])
        else:
            og, hg, cg, vg = _np(o), _np(hT), _np(hck), _np(vnew)
        _check("o", og, o_ref, io, od, case)
        _check("hT", hg, h_ref, io, "fp32", case)
        _check("hck", cg, ck_ref, io, od, case)
        _check("vnew", vg, vn_ref, io, od, case)
        # checkpoint 0 is the initial state itself (rounded to the o dtype)
        h0_t = d["h0"] if d["h0"] is not None else torch.zeros(B, H, K, V, device=_dev())
        assert torch.equal(hck[:, 0], h0_t.to(TDT[od])), case
        del o, hT, hck, vnew, o2, h2


STATE_CASES = [
    # B, T, H, K, V, chunk, io, gate, bias, h0
    (1, 128, 1, 64, 64, 64, "fp32", "head", 2.0, False),
    (2, 150, 2, 64, 64, 32, "fp32", "key", 3.0, True),
    (1, 97, 3, 128, 128, 32, "fp32", "head", 2.0, True),
    (2, 333, 4, 128, 128, 64, "bf16", "head", 2.0, True),
    (2, 256, 4, 64, 64, 32, "bf16", "head", 4.0, False),
    (1, 160, 2, 128, 128, 32, "bf16", "head", 2.0, True),
    (1, 300, 4, 128, 128, 64, "bf16", "key", 3.0, False),
    (1, 130, 2, 128, 64, 64, "bf16", "head", 2.0, True),      # dk != dv
    (1, 130, 2, 64, 128, 32, "bf16", "key", 3.0, True),       # dk != dv
    (1, 1, 1, 64, 64, 64, "bf16", "head", 2.0, True),         # a single token
    (4, 64, 2, 128, 128, 64, "bf16", "head", 2.0, True),      # B*H = 8: XCD swizzle
]


@pytest.mark.parametrize("cfg", STATE_CASES, ids=lambda c: "B%dT%dH%dK%dV%dC%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7]))
def test_forward_states_small(cfg):
    B, T, H, K, V, C, io, gate, bias, h0 = cfg
    run_states("states_small", B, T, H, K, V, C, io, gate, bias, h0,
               seed=B * 1000 + T + K + 7,
               o_dtypes=[io] if io == "fp32" else ["fp32", "bf16"])


def test_forward_states_empty_sequence():
    d = _dev()
    B, H, K, V = 1, 2, 64, 64
    q = torch.empty(B, 0, H, K, device=d, dtype=torch.bfloat16)
    v = torch.empty(B, 0, H, V, device=d, dtype=torch.bfloat16)
    beta = torch.empty(B, 0, H, device=d)
    g = torch.empty(B, 0, H, device=d)
    h0 = torch.randn(B, H, K, V, device=d)
    o, hT, hck, vnew = gdn.forward_states(q, q, v, beta, g, 64, h0)
    torch.cuda.synchronize()
    assert hck.shape[1] == 0 and vnew.numel() == 0
    assert torch.equal(hT, h0)


@pytest.mark.parametrize("name", ["gdn_t4k", "gdn_c32_d64", "kda_t8k"])
def test_forward_states_full_size_sampled(name):
    w = WORKLOADS[name]
    pairs = w.B * w.H
    heads = sorted(set([0, pairs - 1, (7 * pairs) // 11]))
    run_states("states_full_" + name, w.B, w.T, w.H, w.K, w.V, w.chunk, w.io, w.gate,
               w.gate_bias, w.h0, w.seed, o_dtypes=["fp32", "bf16"], heads=heads)
