"""gdn_forward_noalloc against gdn_forward, through the C ABI.

The no-alloc entry point runs the same kernels as gdn_forward with the
per-key gate's Gram workspace taken from the library's static device array
instead of caller memory, so on the same inputs its outputs must equal
gdn_forward's bit for bit.  Two calls in a row, the second on a smaller
problem, check that a call does not depend on what the previous one left in
the shared array; both are also held to the oracle's bar on the smaller case.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def _run_pair(B, T, H, K, V, C, io, gate, seed):
    dev = torch.device("cuda:0")
    inp = make_inputs(B, T, H, K, V, io=io, gate=gate, gate_bias=3.0, h0=True, seed=seed)
    d = {n: (None if x is None else x.to(dev)) for n, x in inp.items()}
    od = torch.float32
    o_ref, h_ref = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"], o_dtype=od)
    o = torch.full((B, T, H, V), float("nan"), device=dev, dtype=od)
    hT = torch.full((B, H, K, V), float("nan"), device=dev, dtype=torch.float32)
    print("no-alloc case", dict(B=B, T=T, H=H, K=K, V=V, C=C, io=io, gate=gate), flush=True)
    gdn.forward_noalloc(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"], o=o, hT=hT)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "o differs from gdn_forward's"
    assert torch.equal(hT, h_ref), "hT differs from gdn_forward's"
    return inp, o, hT


@pytest.mark.parametrize("io,C,K", [("bf16", 64, 128), ("bf16", 32, 64), ("fp32", 64, 128)])
def test_noalloc_matches_forward_twice(io, C, K):
    # first call: a scratch need close to the array's size
    need_per_chunk_head = 2 * C * C * 4 if io == "fp32" else 2 * C * C * 2 + 3 * C * K * 2 + K * 4
    nt = (gdn.NOALLOC_SCRATCH_BYTES // need_per_chunk_head) // 8 - 3   # H = 8, B = 1
    _run_pair(1, nt * C - 5, 8, K, K, C, io, "key", seed=90)
    # second call, smaller, also against the oracle
    inp, o, hT = _run_pair(1, 3 * C + 11, 2, K, K, C, io, "key", seed=91)
    f = lambda x: x.float().numpy()
    o_r, h_r = oracle.token_recurrence(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"]),
                                       f(inp["g"]), f(inp["h0"]))
    assert oracle.rel_err(o.cpu().numpy(), o_r) <= TOL[io]
    assert oracle.rel_err(hT.cpu().numpy(), h_r) <= TOL[io]


def test_noalloc_scalar_gate_needs_no_scratch():
    _run_pair(2, 300, 4, 128, 128, 64, "bf16", "head", seed=92)


def test_noalloc_refuses_oversize_before_launch():
    dev = torch.device("cuda:0")
    C, K = 64, 128
    nt = gdn.NOALLOC_SCRATCH_BYTES // (2 * C * C * 2 + 3 * C * K * 2 + K * 4) + 1   # one too many
    B, T, H = 1, nt * C, 1
    inp = make_inputs(B, T, H, K, K, io="bf16", gate="key", gate_bias=3.0, h0=False, seed=93)
    d = {n: (None if x is None else x.to(dev)) for n, x in inp.items()}
    o = torch.zeros(B, T, H, K, device=dev, dtype=torch.bfloat16)
    with pytest.raises(gdn.GdnError) as e:
        gdn.forward_noalloc(d["q"], d["k"], d["v"], d["beta"], d["g"], C, None, o=o)
    assert e.value.status == 6                                        # GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0
