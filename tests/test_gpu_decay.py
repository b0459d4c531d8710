"""GPU parity at ordinary and strong gates, through the C ABI, against the
fp64 token recurrence (the oracle).

The workloads draw g = logsigmoid(N(0,1) + bias) with bias 2..4; these cases
go well below that: a scalar gate near -8 per token, sparse hard resets
(g = -60 or -100 on a few tokens), and for the per-key gate biases +1, 0 and
-2, four key channels pinned at g = -20, and per-channel resets.  Every
decay inside the kernels' products must then stay a decay (see
tests/test_decay_model.py); a growth factor shows up here as inf/NaN or as
an error far above the bar.  Bar as in test_gpu_parity: max|x - ref| /
rms(ref) <= 2e-2 (bf16 io, fp32 o and hT) or 1e-4 (fp32 io); a bf16 o
element by element within 2e-2 rms + half a bf16 ulp.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from test_decay_model import strong_inputs
from test_gpu_parity import TOL, check_o, _record, _np

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _ref(inp):
    f = lambda x: None if x is None else x.float().numpy()
    return oracle.token_recurrence(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"]),
                                   f(inp["g"]), f(inp["h0"]))


def _forward_case(case, B, T, H, K, V, C, io, gate, recipe, seed, o_dtypes):
    inp = strong_inputs(B, T, H, K, V, gate, recipe, seed, io=io, h0=True)
    o_ref, h_ref = _ref(inp)
    d = {n: (None if x is None else x.to(_dev())) for n, x in inp.items()}
    for od in o_dtypes:
        tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[od]
        o, hT = gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"], o_dtype=tdt)
        torch.cuda.synchronize()
        og, hg = _np(o), _np(hT)
        assert np.isfinite(og).all() and np.isfinite(hg).all(), "%s: non-finite output" % case
        ro = check_o(og, o_ref, io, case, od)
        rh = oracle.rel_err(hg, h_ref)
        _record(case, shape=[B, T, H, K, V, C], io=io, gate=gate, recipe=recipe, o_dtype=od,
                o_rel=ro, hT_rel=rh)
        assert rh <= TOL[io], "%s: hT rel err %.3e" % (case, rh)


HEAD_CASES = [
    # K, V, C, io, recipe
    (128, 128, 64, "bf16", "m8"),
    (64, 64, 32, "bf16", "m8"),
    (128, 64, 32, "bf16", "m8"),
    (128, 128, 64, "bf16", "reset"),
    (64, 64, 32, "bf16", "reset"),
    (64, 64, 64, "fp32", "m8"),
    (128, 128, 32, "fp32", "reset"),
]


@pytest.mark.parametrize("K,V,C,io,recipe", HEAD_CASES,
                         ids=lambda c: str(c))
def test_scalar_gate_strong_decay(K, V, C, io, recipe):
    _forward_case("decay_head_%s" % recipe, 2, 3 * C + 17, 2, K, V, C, io, "head", recipe,
                  seed=41 + K + C, o_dtypes=["fp32"] if io == "fp32" else ["fp32", "bf16"])


@pytest.mark.parametrize("recipe", ["m8", "reset"])
@pytest.mark.parametrize("C", [32, 64])
def test_scalar_gate_strong_decay_prepare_scan(recipe, C):
    """The two-stage path: gdn_prepare's w, u against the fp64 chunk form,
    then gdn_scan on them against the token recurrence."""
    B, T, H, K, V = 1, 2 * C + 9, 2, 64, 64
    inp = strong_inputs(B, T, H, K, V, "head", recipe, seed=43 + C, io="bf16", h0=True)
    d = {n: (None if x is None else x.to(_dev())) for n, x in inp.items()}
    w, u, gc = gdn.prepare(d["k"], d["v"], d["beta"], d["g"], C)
    o, hT = gdn.scan(d["q"], d["k"], w, u, gc, C, d["h0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    gr, wr, ur = oracle.chunk_prepare(inp["k"].float().numpy(), inp["v"].float().numpy(),
                                      inp["beta"].numpy(), inp["g"].numpy(), C)
    o_ref, h_ref = _ref(inp)
    for name, x, ref in (("w", w, wr), ("u", u, ur), ("o", o, o_ref), ("hT", hT, h_ref)):
        xv = _np(x)
        assert np.isfinite(xv).all(), "%s not finite" % name
        assert oracle.rel_err(xv, ref) <= TOL["bf16"], name


KEY_CASES = [
    # K, V, C, io, recipe
    (128, 128, 64, "bf16", "b1"),
    (128, 128, 64, "bf16", "b0"),
    (128, 128, 64, "bf16", "bm2"),
    (128, 128, 64, "bf16", "pin20"),
    (128, 128, 64, "bf16", "reset"),
    (128, 128, 32, "bf16", "b0"),
    (128, 64, 32, "bf16", "pin20"),
    (64, 64, 32, "bf16", "bm2"),
    (64, 128, 64, "bf16", "reset"),
    (128, 128, 64, "fp32", "bm2"),
    (128, 128, 64, "fp32", "pin20"),
    (64, 64, 32, "fp32", "reset"),
    (64, 64, 64, "fp32", "b0"),
]


@pytest.mark.parametrize("K,V,C,io,recipe", KEY_CASES, ids=lambda c: str(c))
def test_key_gate_strong_decay(K, V, C, io, recipe):
    _forward_case("decay_key_%s" % recipe, 2, 2 * C + 21, 2, K, V, C, io, "key", recipe,
                  seed=61 + K + C, o_dtypes=["fp32"] if io == "fp32" else ["fp32", "bf16"])


@pytest.mark.parametrize("recipe", ["bm2", "pin20"])
@pytest.mark.parametrize("C", [32, 64])
def test_key_gate_strong_decay_prepare_scan(recipe, C):
    """The two-stage path with the per-key gate: gdn_prepare's w, u against
    the fp64 chunk form, gdn_scan on them against the token recurrence."""
    B, T, H, K, V = 1, 2 * C + 9, 2, 64, 64
    inp = strong_inputs(B, T, H, K, V, "key", recipe, seed=63 + C, io="bf16", h0=True)
    d = {n: (None if x is None else x.to(_dev())) for n, x in inp.items()}
    w, u, gc = gdn.prepare(d["k"], d["v"], d["beta"], d["g"], C)
    o, hT = gdn.scan(d["q"], d["k"], w, u, gc, C, d["h0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    gr, wr, ur = oracle.chunk_prepare(inp["k"].float().numpy(), inp["v"].float().numpy(),
                                      inp["beta"].numpy(), inp["g"].numpy(), C)
    o_ref, h_ref = _ref(inp)
    for name, x, ref in (("gcum", gc, gr), ("w", w, wr), ("u", u, ur), ("o", o, o_ref),
                         ("hT", hT, h_ref)):
        xv = _np(x)
        assert np.isfinite(xv).all(), "%s not finite" % name
        err = oracle.rel_err(xv, ref)
        _record("decay_key_prepare_scan_%s" % recipe, C=C, name=name, rel=err)
        assert err <= (1e-5 if name == "gcum" else TOL["bf16"]), (name, err)


@pytest.mark.parametrize("recipe", ["b0", "pin20"])
def test_key_gate_strong_decay_states_and_varlen(recipe):
    """The per-key gate's other forward entry points at strong gates: saved
    states against the oracle's, packed sequences against per-sequence runs
    of the oracle."""
    B, T, H, K, V, C = 1, 150, 2, 128, 128, 64
    inp = strong_inputs(B, T, H, K, V, "key", recipe, seed=71, io="bf16", h0=True)
    d = {n: (None if x is None else x.to(_dev())) for n, x in inp.items()}
    f = lambda x: None if x is None else x.float().numpy()
    o, hT, hck, vnew = gdn.forward_states(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"],
                                          o_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref, hck_ref, vn_ref = oracle.token_states(
        f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"]), f(inp["g"]), C, f(inp["h0"]))
    for name, x, ref in (("o", o, o_ref), ("hT", hT, h_ref), ("hck", hck, hck_ref),
                         ("vnew", vnew, vn_ref)):
        xv = _np(x)
        assert np.isfinite(xv).all(), name
        assert oracle.rel_err(xv, ref) <= TOL["bf16"], (name, oracle.rel_err(xv, ref))
    # packed: the stream cut into sequences of 70 and 80 tokens, own states
    lens = [70, 80]
    cu = torch.tensor([0, 70, 150], dtype=torch.int32, device=_dev())
    h0v = 0.1 * torch.randn(2, H, K, V, generator=torch.Generator().manual_seed(5))
    ov, hTv = gdn.forward_varlen(d["q"], d["k"], d["v"], d["beta"], d["g"], cu, C, h0v.to(_dev()),
                                 o_dtype=torch.float32)
    torch.cuda.synchronize()
    s0 = 0
    for n, L in enumerate(lens):
        sl = lambda x: f(x)[:, s0:s0 + L]
        o_r, h_r = oracle.token_recurrence(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]),
                                           sl(inp["beta"]), sl(inp["g"]), f(h0v)[n:n + 1])
        assert oracle.rel_err(_np(ov)[:, s0:s0 + L], o_r) <= TOL["bf16"]
        assert oracle.rel_err(_np(hTv)[n:n + 1], h_r) <= TOL["bf16"]
        s0 += L
