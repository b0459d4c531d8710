"""CPU checks of the seeded input generators shared by the tests, the smoke
check and the benchmark: the recipe's invariants and determinism."""
import pytest

torch = pytest.importorskip("torch")

from chunked_gated_delta_prepare_amd.inputs import (make_inputs, varlen_lengths, VARLEN_MIX,
                                                    WORKLOADS)


def test_make_inputs_is_deterministic_and_follows_the_recipe():
    a = make_inputs(2, 40, 3, 64, 32, io="bf16", gate="key", gate_bias=3.0, h0=True, seed=7)
    b = make_inputs(2, 40, 3, 64, 32, io="bf16", gate="key", gate_bias=3.0, h0=True, seed=7)
    for n in a:
        assert torch.equal(a[n], b[n]), n
    assert a["q"].dtype == torch.bfloat16 and a["beta"].dtype == torch.float32
    assert a["g"].shape == (2, 40, 3, 64) and a["h0"].shape == (2, 3, 64, 32)
    # q and k are L2-normalised per token before the cast; beta in (0, 1); g = logsigmoid < 0
    nq = a["q"].float().norm(dim=-1)
    assert torch.allclose(nq, torch.ones_like(nq), atol=2e-2)
    assert (a["beta"] > 0).all() and (a["beta"] < 1).all()
    assert (a["g"] < 0).all()
    c = make_inputs(2, 40, 3, 64, 32, io="bf16", gate="key", gate_bias=3.0, h0=True, seed=8)
    assert not torch.equal(a["q"], c["q"])


@pytest.mark.parametrize("total", [16384, 65536, 16384 * 3 + 5, 8])
def test_varlen_lengths_split_the_total(total):
    lens = varlen_lengths(total)
    assert len(lens) == len(VARLEN_MIX)
    assert sum(lens) == total and min(lens) >= 0
    if total == sum(VARLEN_MIX):
        assert lens == list(VARLEN_MIX)


def test_workloads_have_the_stated_shapes():
    w = WORKLOADS["gdn_t4k"]
    assert (w.B, w.H, w.T, w.K, w.V, w.chunk, w.gate) == (4, 16, 4096, 128, 128, 64, "head")
    w = WORKLOADS["kda_t8k"]
    assert (w.B, w.H, w.T, w.K, w.V, w.chunk, w.gate) == (2, 32, 8192, 128, 128, 64, "key")
