"""GPU parity of gdn_forward_varlen (packed sequences, through the C ABI)
against the fp64 oracle run on each sequence separately.

Same bar as the fixed-length forward: max |x - x_ref| / rms(x_ref) <= 2e-2
with bf16 inputs and <= 1e-4 with fp32 inputs, for fp32 o and for every
sequence's final state.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _np(t):
    return t.detach().float().cpu().numpy()


def _inputs(lens, H, K, V, io, gate, bias, h0, seed):
    T = int(sum(lens))
    inp = make_inputs(1, T, H, K, V, io=io, gate=gate, gate_bias=bias, h0=False, seed=seed)
    # one initial state per sequence, from a generator of its own
    inp["h0"] = make_inputs(len(lens), 1, H, K, V, h0=True, seed=seed + 1)["h0"] if h0 else None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return inp, cu


def _oracle(inp, cu):
    """The token recurrence on each sequence on its own."""
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    beta, g = inp["beta"].numpy(), inp["g"].numpy()
    N = len(cu) - 1
    H, K, V = q.shape[2], q.shape[3], v.shape[3]
    o = np.zeros(v.shape, np.float64)
    hT = np.zeros((N, H, K, V), np.float64)
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        h0 = None if inp["h0"] is None else inp["h0"][n:n + 1].numpy()
        on, hn = oracle.token_recurrence(q[:, a:b], k[:, a:b], v[:, a:b], beta[:, a:b],
                                         g[:, a:b], h0)
        o[:, a:b] = on
        hT[n] = hn[0]
    return o, hT


CASES = [
    # lengths, H, K, V, chunk, io, gate, bias, h0
    ([0, 1, 63, 64, 65, 200, 129], 2, 128, 128, 64, "bf16", "head", 2.0, True),
    ([31, 32, 33, 100, 0, 7], 3, 64, 64, 32, "bf16", "head", 4.0, False),
    ([70, 5, 128], 2, 128, 128, 32, "bf16", "head", 2.0, True),
    ([90, 1, 64, 130], 2, 128, 128, 64, "bf16", "key", 3.0, True),
    ([33, 0, 96], 2, 64, 128, 32, "bf16", "key", 3.0, False),
    ([50, 77, 1], 2, 64, 64, 64, "fp32", "head", 2.0, True),
    ([40, 64, 9], 1, 128, 128, 32, "fp32", "key", 3.0, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "N%dK%dV%dC%d_%s_%s" % (
    len(c[0]), c[2], c[3], c[4], c[5], c[6]))
def test_forward_varlen_matches_per_sequence_oracle(case):
    lens, H, K, V, C, io, gate, bias, h0 = case
    inp, cu = _inputs(lens, H, K, V, io, gate, bias, h0, seed=sum(lens) + 11 * K + C)
    print("case varlen", lens, H, K, V, C, io, gate, flush=True)
    d = {n: (None if t is None else t.to(_dev())) for n, t in inp.items()}
    cu_d = torch.from_numpy(cu).to(_dev())
    o_ref, h_ref = _oracle(inp, cu)
    for od in (["fp32"] if io == "fp32" else ["fp32", "bf16"]):
        tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[od]
        o, hT = gdn.forward_varlen(d["q"], d["k"], d["v"], d["beta"], d["g"], cu_d, C, d["h0"],
                                   o_dtype=tdt)
        torch.cuda.synchronize()
        ro, rh = oracle.rel_err(_np(o), o_ref), oracle.rel_err(_np(hT), h_ref)
        print("  o_dtype %s: o rel %.3e, hT rel %.3e" % (od, ro, rh), flush=True)
        assert rh <= TOL[io], "hT rel err %.3e" % rh
        if od == "fp32":
            assert ro <= TOL[io], "o rel err %.3e" % ro
        else:
            # bf16 o: the fp32 bound plus half a bf16 ulp, element by element
            rms = float(np.sqrt(np.mean(o_ref ** 2)))
            a = np.maximum(np.abs(o_ref), np.abs(_np(o)))
            slack = TOL[io] * rms + np.exp2(np.floor(np.log2(np.maximum(a, 1e-38))) - 8)
            assert not (np.abs(_np(o) - o_ref) > slack).any()


@pytest.mark.parametrize("gate,io,C", [("head", "bf16", 64), ("head", "bf16", 32),
                                       ("key", "bf16", 64), ("head", "fp32", 64)])
def test_forward_varlen_equal_lengths_is_the_batched_forward(gate, io, C):
    # packed sequences of one length L are the [N, L, H, .] batch laid end to
    # end: the same streams, so the same bits
    N, L, H, K, V = 3, 150, 2, 128, 128
    inp = make_inputs(N, L, H, K, V, io=io, gate=gate, gate_bias=3.0, h0=True, seed=5)
    d = {n: t.to(_dev()) for n, t in inp.items()}
    o_b, h_b = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"])
    flat = {n: d[n].reshape(1, N * L, *d[n].shape[2:]) for n in ("q", "k", "v", "beta", "g")}
    cu = torch.arange(0, N * L + 1, L, dtype=torch.int32, device=_dev())
    o_v, h_v = gdn.forward_varlen(flat["q"], flat["k"], flat["v"], flat["beta"], flat["g"], cu,
                                  C, d["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o_v.reshape(N, L, H, V), o_b)
    assert torch.equal(h_v, h_b)


def test_forward_varlen_mixed_lengths_larger():
    # 8 sequences from 1 to 4000 tokens over 16 heads of 128 x 128
    lens = [4000, 1, 777, 64, 2500, 130, 1999, 33]
    inp, cu = _inputs(lens, 16, 128, 128, "bf16", "head", 2.0, True, seed=99)
    d = {n: (None if t is None else t.to(_dev())) for n, t in inp.items()}
    o, hT = gdn.forward_varlen(d["q"], d["k"], d["v"], d["beta"], d["g"],
                               torch.from_numpy(cu).to(_dev()), 64, d["h0"],
                               o_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = _oracle(inp, cu)
    ro, rh = oracle.rel_err(_np(o), o_ref), oracle.rel_err(_np(hT), h_ref)
    print("varlen larger: o rel %.3e, hT rel %.3e" % (ro, rh), flush=True)
    assert ro <= TOL["bf16"] and rh <= TOL["bf16"]
