"""gdn_forward_split (the scalar-gate forward with each stream cut in two
segments that run at the same time) against the fp64 token recurrence (the
oracle), through the C ABI.

The second segment's outputs and the final state are assembled from its
zero-start and identity-start passes and the first segment's end state
(o_t = o0_t + h_in^T oI_t, hT = N + M h_in), so they differ from
gdn_forward's in rounding only: the same bar as every forward, max|x - ref| /
rms(ref) <= 2e-2 with fp32 o and for hT, and with bf16 o element by element
within 2e-2 rms + half a bf16 ulp.  Cases cover ragged T, K != V, B H not a
multiple of 8 (no XCD swizzle), cuts near either end and strong decays.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs
from test_decay_model import strong_inputs
from test_gpu_parity import TOL, check_o, _np, _record

pytestmark = pytest.mark.gpu

CASES = [
    # B, T, H, K, V, t_split, h0, gate bias or recipe
    (1, 700, 8, 128, 128, 448, True, 2.0),
    (2, 512, 4, 64, 64, 320, False, 4.0),
    (1, 1000, 3, 128, 64, 640, True, 2.0),
    (4, 256, 2, 64, 128, 64, True, 3.0),
    (1, 300, 8, 128, 128, 256, True, 1.0),
    (2, 640, 8, 128, 128, 384, True, "m8"),
    (1, 513, 8, 128, 128, 448, True, "reset"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_split_forward_matches_oracle(case):
    B, T, H, K, V, ts, h0, bias = CASES[case]
    print("split case", CASES[case], flush=True)
    if isinstance(bias, str):
        inp = strong_inputs(B, T, H, K, V, "head", bias, seed=300 + case, io="bf16", h0=h0)
    else:
        inp = make_inputs(B, T, H, K, V, io="bf16", gate="head", gate_bias=bias, h0=h0, seed=300 + case)
    d = {n: (None if x is None else x.cuda()) for n, x in inp.items()}
    f = lambda x: None if x is None else x.float().numpy()
    o_ref, h_ref = oracle.token_recurrence(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"]),
                                           f(inp["g"]), f(inp["h0"]))
    for od in ("fp32", "bf16"):
        tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[od]
        o, hT = gdn.forward_split(d["q"], d["k"], d["v"], d["beta"], d["g"], 64, ts, d["h0"],
                                  o_dtype=tdt)
        torch.cuda.synchronize()
        og, hg = _np(o), _np(hT)
        assert np.isfinite(og).all() and np.isfinite(hg).all()
        ro = check_o(og, o_ref, "bf16", "split%d" % case, od)
        rh = oracle.rel_err(hg, h_ref)
        _record("split%d" % case, o_dtype=od, o_rel=ro, hT_rel=rh)
        assert rh <= TOL["bf16"], (od, rh)
        # the first segment is the plain kernel's work: equal to gdn_forward there
        o1, _ = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], 64, d["h0"], o_dtype=tdt)
        torch.cuda.synchronize()
        assert torch.equal(o[:, :ts], o1[:, :ts])


def test_split_forward_without_final_state():
    B, T, H, K, V, ts = 1, 400, 8, 64, 64, 192
    inp = make_inputs(B, T, H, K, V, io="bf16", gate="head", gate_bias=2.0, h0=True, seed=333)
    d = {n: (None if x is None else x.cuda()) for n, x in inp.items()}
    o, hT = gdn.forward_split(d["q"], d["k"], d["v"], d["beta"], d["g"], 64, ts, d["h0"],
                              o_dtype=torch.float32, output_final_state=False)
    torch.cuda.synchronize()
    assert hT is None
    f = lambda x: x.float().numpy()
    o_ref, _ = oracle.token_recurrence(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"]),
                                       f(inp["g"]), f(inp["h0"]))
    assert oracle.rel_err(_np(o), o_ref) <= TOL["bf16"]


def test_split_refuses_the_per_key_gate():
    inp = make_inputs(1, 256, 2, 64, 64, io="bf16", gate="key", gate_bias=3.0, h0=False, seed=334)
    d = {n: (None if x is None else x.cuda()) for n, x in inp.items()}
    with pytest.raises(gdn.GdnError) as e:
        gdn.forward_split(d["q"], d["k"], d["v"], d["beta"], d["g"], 64, 128)
    assert e.value.status == 3


# ---------------------------------------------------------------------------
# gdn_forward's own split: at gdn_forward_split_point when the workspace is
# there, the single pass otherwise
# ---------------------------------------------------------------------------

def test_forward_splits_long_streams_on_an_idle_device(monkeypatch):
    """B H = 4 streams of 8229 tokens (129 chunks, a ragged last one) keep 8
    of 256 compute units busy: gdn_forward cuts them at 4096 (one round of
    the 16 second-segment streams).  Its outputs meet the oracle's bar, hT
    may alias h0, and they agree with the single pass (GDN_FORWARD_NO_SPLIT)
    to rounding; without a workspace gdn_forward runs exactly that single
    pass."""
    monkeypatch.delenv("GDN_FORWARD_NO_SPLIT", raising=False)
    B, T, H, K, V, C = 1, 8229, 4, 128, 128, 64
    assert gdn.forward_split_point(B, T, H, K, V, C, torch.bfloat16) == 4096
    inp = make_inputs(B, T, H, K, V, io="bf16", gate="head", gate_bias=2.0, h0=True, seed=331)
    d = {n: (None if x is None else x.cuda()) for n, x in inp.items()}
    f = lambda x: x.float().numpy()
    o_ref, h_ref = oracle.token_recurrence(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"]),
                                           f(inp["g"]), f(inp["h0"]))
    outs = {}
    for od in ("fp32", "bf16"):
        tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[od]
        hT = d["h0"].clone()            # hT aliasing h0
        o, _ = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, hT, o_dtype=tdt, hT=hT)
        torch.cuda.synchronize()
        og, hg = _np(o), _np(hT)
        assert np.isfinite(og).all() and np.isfinite(hg).all()
        ro = check_o(og, o_ref, "bf16", "auto_split", od)
        rh = oracle.rel_err(hg, h_ref)
        _record("auto_split", o_dtype=od, o_rel=ro, hT_rel=rh)
        assert rh <= TOL["bf16"], (od, rh)
        outs[od] = (o, hT)
    # the single pass, by switch and for want of a workspace
    monkeypatch.setenv("GDN_FORWARD_NO_SPLIT", "1")
    o1, h1 = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"], o_dtype=torch.float32)
    monkeypatch.delenv("GDN_FORWARD_NO_SPLIT")
    lib = gdn.load_library()
    pr = gdn.Problem(B, T, H, K, V, C, gdn.GDN_BF16, gdn.GDN_F32, gdn.GDN_GATE_HEAD)
    o2 = torch.empty_like(o1)
    h2 = torch.empty_like(h1)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    assert lib.gdn_forward(ctypes.byref(pr), P(d["q"]), P(d["k"]), P(d["v"]), P(d["beta"]), P(d["g"]),
                           P(d["h0"]), P(o2), P(h2), None, ctypes.c_size_t(0), None) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    # split against single pass: rounding apart
    assert oracle.rel_err(_np(outs["fp32"][0]), _np(o1)) < 5e-3
    assert oracle.rel_err(_np(outs["fp32"][1]), _np(h1)) < 5e-3
