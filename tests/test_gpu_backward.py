"""GPU parity of gdn_backward (the scalar gate's gradients, through the C ABI)
against the fp64 oracle.

Both gates: one gate per head (Gated DeltaNet) and one per key dimension
(KDA), the latter with the decay-weighted sums of its own kernels.

gdn_backward takes the forward's saved chunk-start states and deltas (hck,
vnew) in bf16, as inputs.  Their rounding alone moves dq and dk by 1-3e-2
(max |x - ref| / rms(ref)) against the exact gradients, which the oracle
shows by computing the gradients from rounded states.  So parity is taken
the way the forward's is, on identical inputs: the states are the oracle's
(token_states), rounded to bf16, and both the GPU and ``chunk_backward`` get
those same bf16 values; bar 2e-2 for every gradient, the forward's bar for
bf16 inputs.  The workspace's intermediates (v's gradient before the beta
factor, each chunk's end-state gradient) are held to the same bar.

End to end (the GPU forward's saved states, then the GPU backward, against
``token_backward``'s exact gradients) the bar is 2e-2 plus the oracle's own
error from bf16-rounded states in that case.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _np(t):
    return t.detach().float().cpu().numpy()


def _grads_inputs(B, T, H, K, V, h0, dhT, seed, bias=2.0, gate="head", recipe=None):
    if recipe is not None:
        from test_decay_model import strong_inputs
        inp = strong_inputs(B, T, H, K, V, gate, recipe, seed, io="bf16", h0=h0)
    else:
        inp = make_inputs(B, T, H, K, V, io="bf16", gate=gate, gate_bias=bias, h0=h0, seed=seed)
    gen = torch.Generator().manual_seed(seed + 7)
    do = torch.randn(B, T, H, V, generator=gen).to(torch.bfloat16).contiguous()
    dh = torch.randn(B, H, K, V, generator=gen).contiguous() if dhT else None
    return inp, do, dh


def _f(x):
    return None if x is None else x.float().numpy()


def _oracle_states(inp, C):
    """The chunk-start states and deltas from the oracle's token recurrence,
    rounded to bf16 (torch, round to nearest even)."""
    _, _, hck, vnew = oracle.token_states(_f(inp["q"]), _f(inp["k"]), _f(inp["v"]), _f(inp["beta"]),
                                          _f(inp["g"]), C, _f(inp["h0"]))
    return (torch.from_numpy(hck).to(torch.bfloat16).contiguous(),
            torch.from_numpy(vnew).to(torch.bfloat16).contiguous())


def _gpu_backward(inp, do, dh, C, hck, vnew, workspace=None, want_dh0=True):
    d = {n: (None if t is None else t.to(_dev())) for n, t in inp.items()}
    out = gdn.backward(d["q"], d["k"], d["v"], d["beta"], d["g"], do.to(_dev()), C, hck.to(_dev()),
                       vnew.to(_dev()), None if dh is None else dh.to(_dev()), want_dh0=want_dh0,
                       workspace=workspace)
    torch.cuda.synchronize()
    return out


def _gpu_forward_states(inp, C):
    d = {n: (None if t is None else t.to(_dev())) for n, t in inp.items()}
    _, _, hck, vnew = gdn.forward_states(d["q"], d["k"], d["v"], d["beta"], d["g"], C, d["h0"],
                                         o_dtype=torch.bfloat16)
    return hck, vnew


def _oracle_grads(inp, do, dh, C, hck, vnew):
    B, T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    h0 = _f(inp["h0"]) if inp["h0"] is not None else np.zeros((B, H, K, V))
    return oracle.chunk_backward(_f(inp["q"]), _f(inp["k"]), _f(inp["v"]), _f(inp["beta"]),
                                 _f(inp["g"]), _f(do), C, h0, _f(dh),
                                 hck=None if hck is None else _f(hck),
                                 vnew=None if vnew is None else _f(vnew))


CASES = [
    # B, T, H, K, V, C, h0, dhT
    (1, 150, 2, 64, 64, 64, True, True),
    (2, 100, 2, 64, 64, 32, False, True),
    (1, 130, 2, 128, 128, 64, True, True),
    (1, 97, 3, 128, 64, 32, True, False),
    (1, 128, 2, 64, 128, 64, False, False),
    (1, 64, 1, 128, 128, 64, True, True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_matches_oracle(case):
    B, T, H, K, V, C, h0, dhT = CASES[case]
    print("backward case", CASES[case], flush=True)
    inp, do, dh = _grads_inputs(B, T, H, K, V, h0, dhT, seed=900 + case)
    hck, vnew = _oracle_states(inp, C)
    got = _gpu_backward(inp, do, dh, C, hck, vnew)
    ref = _oracle_grads(inp, do, dh, C, hck, vnew)
    for name, x, r in zip(NAMES, got, ref[:6]):
        xv = _np(x)
        assert np.isfinite(xv).all(), name
        err = oracle.rel_err(xv, r)
        print("  %s rel err %.3e" % (name, err), flush=True)
        assert err <= TOL, (name, err)


@pytest.mark.parametrize("case", [0, 2, 3])
def test_backward_end_to_end(case):
    """gdn_forward_states then gdn_backward on the GPU, against the exact
    gradients (token_backward)."""
    B, T, H, K, V, C, h0, dhT = CASES[case]
    inp, do, dh = _grads_inputs(B, T, H, K, V, h0, dhT, seed=920 + case)
    hck, vnew = _gpu_forward_states(inp, C)
    got = _gpu_backward(inp, do, dh, C, hck, vnew)
    exact = oracle.token_backward(_f(inp["q"]), _f(inp["k"]), _f(inp["v"]), _f(inp["beta"]),
                                  _f(inp["g"]), _f(do), _f(inp["h0"]), _f(dh))
    exact = list(exact)
    if exact[5] is None:
        exact[5] = _oracle_grads(inp, do, dh, C, None, None)[5]
    rounded = _oracle_grads(inp, do, dh, C, *_oracle_states(inp, C))
    for name, x, r, o in zip(NAMES, got, exact, rounded[:6]):
        bar = TOL + oracle.rel_err(o, r)
        err = oracle.rel_err(_np(x), r)
        print("  %s rel err %.3e (bar %.3e)" % (name, err, bar), flush=True)
        assert err <= bar, (name, err, bar)


def test_backward_workspace_holds_the_scan_intermediates():
    """v's gradient before the beta factor and every chunk's end-state
    gradient, as the reverse scan leaves them, against chunk_backward's."""
    import ctypes
    B, T, H, K, V, C = 1, 200, 2, 128, 128, 64
    inp, do, dh = _grads_inputs(B, T, H, K, V, True, True, seed=931)
    pr = gdn.Problem(B, T, H, K, V, C, gdn.GDN_BF16, gdn.GDN_BF16, gdn.GDN_GATE_HEAD)
    need = int(gdn.load_library().gdn_workspace_bytes_backward(ctypes.byref(pr)))
    ws = torch.empty(need, device=_dev(), dtype=torch.uint8)
    hck, vnew = _oracle_states(inp, C)
    _gpu_backward(inp, do, dh, C, hck, vnew, workspace=ws)
    nt = (T + C - 1) // C
    wsf = ws.view(torch.float32)
    dR = _np(wsf[:B * T * H * V].view(B, T, H, V))
    dhe = _np(wsf[B * T * H * V:B * T * H * V + B * nt * H * K * V].view(B, nt, H, K, V))
    ref = _oracle_grads(inp, do, dh, C, hck, vnew)[6]
    assert oracle.rel_err(dR, ref["dR"]) <= TOL
    assert oracle.rel_err(dhe, ref["dhe"]) <= TOL
    # the last chunk's end gradient is dhT itself
    np.testing.assert_array_equal(dhe[:, -1], _np(dh))


def test_backward_without_dh0_and_empty_sequence():
    B, T, H, K, V, C = 1, 70, 2, 64, 64, 64
    inp, do, dh = _grads_inputs(B, T, H, K, V, True, True, seed=941)
    hck, vnew = _oracle_states(inp, C)
    full = _gpu_backward(inp, do, dh, C, hck, vnew)
    part = _gpu_backward(inp, do, dh, C, hck, vnew, want_dh0=False)
    assert part[5] is None
    for a, b in zip(full[:5], part[:5]):
        assert torch.equal(a, b)            # deterministic, and dh0 changes nothing else
    # T = 0: dh0 = dhT
    z = torch.empty(1, 0, H, K, device=_dev(), dtype=torch.bfloat16)
    zv = torch.empty(1, 0, H, V, device=_dev(), dtype=torch.bfloat16)
    zb = torch.empty(1, 0, H, device=_dev(), dtype=torch.float32)
    hz = torch.empty(1, 0, H, K, V, device=_dev(), dtype=torch.bfloat16)
    out = gdn.backward(z, z, zv, zb, zb, zv, C, hz, zv, dh.to(_dev()))
    torch.cuda.synchronize()
    assert torch.equal(out[5].cpu(), dh)


FULL = {
    # name: (B, T, H, K, V, C, h0, gate bias), heads sampled
    "gdn_t4k": ((4, 4096, 16, 128, 128, 64, True, 2.0), [(0, 0), (3, 15)]),
    "gdn_c32_d64": ((8, 2048, 32, 64, 64, 32, False, 4.0), [(5, 17)]),
}


@pytest.mark.parametrize("name", sorted(FULL))
def test_backward_full_size_sampled_heads(name):
    """The full problem on the GPU (states from the oracle for every head),
    sampled heads against chunk_backward on the same states."""
    (B, T, H, K, V, C, h0, bias), heads = FULL[name]
    print("backward full size", name, flush=True)
    inp, do, dh = _grads_inputs(B, T, H, K, V, h0, True, seed=951, bias=bias)
    hck, vnew = _oracle_states(inp, C)
    got = [_np(x) for x in _gpu_backward(inp, do, dh, C, hck, vnew)]
    for b, h in heads:
        one = {n: (None if t is None else (t[b:b + 1, h:h + 1] if n == "h0" else t[b:b + 1, :, h:h + 1]))
               for n, t in inp.items()}
        ref = _oracle_grads(one, do[b:b + 1, :, h:h + 1], dh[b:b + 1, h:h + 1], C,
                            hck[b:b + 1, :, h:h + 1], vnew[b:b + 1, :, h:h + 1])
        for nm, x, r in zip(NAMES, got, ref[:6]):
            xs = x[b:b + 1, h:h + 1] if nm == "dh0" else x[b:b + 1, :, h:h + 1]
            err = oracle.rel_err(xs, r)
            print("  head (%d, %d) %s rel err %.3e" % (b, h, nm, err), flush=True)
            assert err <= TOL, (nm, b, h, err)


KEY_CASES = [
    # B, T, H, K, V, C, h0, dhT, recipe (None: logsigmoid(N(0,1) + 3))
    (1, 150, 2, 64, 64, 64, True, True, None),
    (1, 97, 2, 128, 128, 64, True, True, None),
    (2, 100, 2, 128, 64, 32, False, True, None),
    (1, 128, 2, 64, 128, 32, True, False, None),
    (1, 130, 2, 128, 128, 64, True, True, "pin20"),
    (1, 100, 2, 64, 64, 32, True, True, "bm2"),
]


@pytest.mark.parametrize("case", range(len(KEY_CASES)))
def test_backward_key_gate_matches_oracle(case):
    B, T, H, K, V, C, h0, dhT, recipe = KEY_CASES[case]
    print("backward key case", KEY_CASES[case], flush=True)
    inp, do, dh = _grads_inputs(B, T, H, K, V, h0, dhT, seed=960 + case, bias=3.0, gate="key", recipe=recipe)
    hck, vnew = _oracle_states(inp, C)
    got = _gpu_backward(inp, do, dh, C, hck, vnew)
    ref = _oracle_grads(inp, do, dh, C, hck, vnew)
    for name, x, r in zip(NAMES, got, ref[:6]):
        xv = _np(x)
        assert np.isfinite(xv).all(), name
        err = oracle.rel_err(xv, r)
        print("  %s rel err %.3e" % (name, err), flush=True)
        assert err <= TOL, (name, err)


def test_backward_key_gate_intermediates_and_end_to_end():
    import ctypes
    B, T, H, K, V, C = 1, 200, 2, 128, 128, 64
    inp, do, dh = _grads_inputs(B, T, H, K, V, True, True, seed=981, bias=3.0, gate="key")
    pr = gdn.Problem(B, T, H, K, V, C, gdn.GDN_BF16, gdn.GDN_BF16, gdn.GDN_GATE_KEY)
    need = int(gdn.load_library().gdn_workspace_bytes_backward(ctypes.byref(pr)))
    ws = torch.empty(need, device=_dev(), dtype=torch.uint8)
    hck, vnew = _oracle_states(inp, C)
    _gpu_backward(inp, do, dh, C, hck, vnew, workspace=ws)
    nt = (T + C - 1) // C
    wsf = ws.view(torch.float32)
    dR = _np(wsf[:B * T * H * V].view(B, T, H, V))
    dhe = _np(wsf[B * T * H * V:B * T * H * V + B * nt * H * K * V].view(B, nt, H, K, V))
    ref = _oracle_grads(inp, do, dh, C, hck, vnew)[6]
    assert oracle.rel_err(dR, ref["dR"]) <= TOL
    assert oracle.rel_err(dhe, ref["dhe"]) <= TOL
    # end to end: the GPU forward's states, against the exact gradients
    hg, vg = _gpu_forward_states(inp, C)
    got = _gpu_backward(inp, do, dh, C, hg, vg)
    exact = oracle.token_backward(_f(inp["q"]), _f(inp["k"]), _f(inp["v"]), _f(inp["beta"]),
                                  _f(inp["g"]), _f(do), _f(inp["h0"]), _f(dh))
    rounded = _oracle_grads(inp, do, dh, C, hck, vnew)
    for name, x, r, o in zip(NAMES, got, exact, rounded[:6]):
        bar = TOL + oracle.rel_err(o, r)
        err = oracle.rel_err(_np(x), r)
        print("  end to end %s rel err %.3e (bar %.3e)" % (name, err, bar), flush=True)
        assert err <= bar, (name, err, bar)


def test_backward_key_gate_full_size_sampled_heads():
    """kda_t8k's shape (2 x 8192 tokens, 32 heads, per-key gate), states from
    the oracle for every head, two heads against chunk_backward."""
    B, T, H, K, V, C = 2, 8192, 32, 128, 128, 64
    print("backward key full size", flush=True)
    inp, do, dh = _grads_inputs(B, T, H, K, V, False, True, seed=991, bias=3.0, gate="key")
    hck, vnew = _oracle_states(inp, C)
    got = [_np(x) for x in _gpu_backward(inp, do, dh, C, hck, vnew)]
    for b, h in [(0, 5), (1, 30)]:
        one = {n: (None if t is None else t[b:b + 1, :, h:h + 1]) for n, t in inp.items()}
        ref = _oracle_grads(one, do[b:b + 1, :, h:h + 1], dh[b:b + 1, h:h + 1], C,
                            hck[b:b + 1, :, h:h + 1], vnew[b:b + 1, :, h:h + 1])
        for nm, x, r in zip(NAMES, got, ref[:6]):
            xs = x[b:b + 1, h:h + 1] if nm == "dh0" else x[b:b + 1, :, h:h + 1]
            err = oracle.rel_err(xs, r)
            print("  head (%d, %d) %s rel err %.3e" % (b, h, nm, err), flush=True)
            assert err <= TOL, (nm, b, h, err)
