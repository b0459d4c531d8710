"""The bounded LDS waits inside the bf16-io kernels report when they give up.

A normal launch must leave the device's give-up count at zero.  With
GDN_WAIT_FORCE_TIMEOUT=1 the host adds a bias to every wait target that no
counter reaches and limits the polls to a few, so every bounded wait gives up
(the kernels still run to their end; their results are garbage): the count
must then grow, for both gates and for the re-scan's chain-side waits.
"""
import os

import pytest

torch = pytest.importorskip("torch")

import chunked_gated_delta_prepare_amd as gdn
from chunked_gated_delta_prepare_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def _inputs(gate, C, T=200):
    d = torch.device("cuda:0")
    inp = make_inputs(1, T, 2, 128, 128, io="bf16", gate=gate, gate_bias=3.0, h0=True, seed=51)
    return {n: (None if x is None else x.to(d)) for n, x in inp.items()}


def _forward(inp, C):
    gdn.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], C, inp["h0"],
                o_dtype=torch.float32)
    torch.cuda.synchronize()


@pytest.fixture
def forced_timeouts():
    os.environ["GDN_WAIT_FORCE_TIMEOUT"] = "1"
    try:
        yield
    finally:
        del os.environ["GDN_WAIT_FORCE_TIMEOUT"]
        gdn.wait_timeouts(reset=True)


def test_normal_launches_do_not_time_out():
    gdn.wait_timeouts(reset=True)
    for gate in ("head", "key"):
        for C in (32, 64):
            _forward(_inputs(gate, C), C)
    assert gdn.wait_timeouts() == 0


@pytest.mark.parametrize("C", [32, 64])
def test_forced_timeouts_are_counted(C, forced_timeouts):
    inp = _inputs("head", C)
    gdn.wait_timeouts(reset=True)
    _forward(inp, C)
    # four prepare waves per workgroup wait at least once per prepared chunk
    nt = (200 + C - 1) // C
    assert gdn.wait_timeouts() >= 4 * nt * 4


@pytest.mark.parametrize("C", [32, 64])
def test_key_gate_forward_has_no_bounded_waits(C, forced_timeouts):
    """The per-key forward's prepare waves only copy what the Gram kernel
    left in the workspace, and hand it over at workgroup barriers: nothing
    to give up on, so even a forced timeout leaves the count at zero."""
    inp = _inputs("key", C)
    gdn.wait_timeouts(reset=True)
    _forward(inp, C)
    assert gdn.wait_timeouts() == 0


@pytest.mark.parametrize("gate", ["head", "key"])
def test_forced_timeouts_in_the_rescan(gate, forced_timeouts):
    # the re-scan's chain waves wait on each other around the dq staging
    inp = _inputs(gate, 64)
    dout = torch.randn(1, 200, 2, 128, device="cuda:0").to(torch.bfloat16)
    gdn.wait_timeouts(reset=True)
    gdn.rescan_dq(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], dout, 64, inp["h0"],
                  o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert gdn.wait_timeouts() > 0


def test_count_resets():
    gdn.wait_timeouts(reset=True)
    assert gdn.wait_timeouts() == 0
