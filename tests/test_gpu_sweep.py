"""GPU parity sweep: seeded random shapes through every forward entry point,
against the fp64 oracle, at the forward's bar (max |x - x_ref| / rms(x_ref)
<= 2e-2 with bf16 inputs, 1e-4 with fp32 inputs, fp32 outputs).

Each case draws B, T (ragged, 1 .. 300), H, K, V, the chunk, the gate kind,
its bias and whether h0 is given from a generator seeded by the case index,
so the sweep is the same on every run.  gdn_forward, gdn_forward_states
(o, the final state, the saved states and v') and, with bf16 inputs,
gdn_chunk_dq on those states are checked in each case.
"""
import random

import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}
N_CASES = 24


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _np(t):
    return t.detach().float().cpu().numpy()


def _draw(i):
    r = random.Random(1000 + i)
    io = "fp32" if i % 6 == 5 else "bf16"
    return dict(B=r.choice([1, 2, 3]), T=r.randint(1, 300), H=r.choice([1, 2, 3]),
                K=r.choice([64, 128]), V=r.choice([64, 128]), C=r.choice([32, 64]),
                gate=r.choice(["head", "key"]), bias=r.choice([1.0, 2.0, 3.0, 4.0]),
                h0=r.random() < 0.6, io=io)


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_case(i):
    c = _draw(i)
    print("case sweep", i, c, flush=True)
    B, T, H, K, V, C, io = c["B"], c["T"], c["H"], c["K"], c["V"], c["C"], c["io"]
    inp = make_inputs(B, T, H, K, V, io=io, gate=c["gate"], gate_bias=c["bias"], h0=c["h0"],
                      seed=7000 + i)
    d = {n: (None if t is None else t.to(_dev())) for n, t in inp.items()}
    o_ref, h_ref, ck_ref, vn_ref = oracle.token_states(
        inp["q"].float().numpy(), inp["k"].float().numpy(), inp["v"].float().numpy(),
        inp["beta"].numpy(), inp["g"].numpy(), C,
        None if inp["h0"] is None else inp["h0"].numpy())
    tol = TOL[io]
    o, hT = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"],
                        o_dtype=torch.float32)
    o2, hT2, hck, vnew = gdn.forward_states(d["q"], d["k"], d["v"], d["beta"], d["g"], C,
                                            d["h0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    for name, got, ref in (("o", o, o_ref), ("hT", hT, h_ref), ("states o", o2, o_ref),
                           ("states hT", hT2, h_ref), ("hck", hck, ck_ref), ("vnew", vnew, vn_ref)):
        rel = oracle.rel_err(_np(got), ref)
        print("  %s rel %.3e" % (name, rel), flush=True)
        assert rel <= tol, "case %d %s rel %.3e" % (i, name, rel)

    if io == "bf16":
        gen = torch.Generator().manual_seed(8000 + i)
        do = torch.randn(B, T, H, V, generator=gen).to(torch.bfloat16)
        dq = gdn.chunk_dq(do.to(_dev()), hck, C)
        torch.cuda.synchronize()
        # end to end: saved states, then the product, against the oracle's
        # dq from its own states (the states' error is in it: the same bar)
        ref = oracle.rescan_dq(ck_ref, do.double().numpy(), C)
        rel = oracle.rel_err(_np(dq), ref)
        print("  chunk_dq rel %.3e" % rel, flush=True)
        assert rel <= tol, "case %d chunk_dq rel %.3e" % (i, rel)
