"""Seeded synthetic inputs for the gated delta rule forward pass.

This module draws random inputs and nothing else: it holds none of the
method's arithmetic, so both the HIP path's tests/benchmark and the oracle
consume the same tensors from here.

Recipe (torch CPU generator, ``manual_seed(seed)``, fp32 draws in this order):
  1. q = randn(B,T,H,K)        2. k = randn(B,T,H,K)      3. v = randn(B,T,H,V)
  4. beta = sigmoid(randn(B,T,H))
  5. g = logsigmoid(randn(B,T,H[,K]) + bias)   (stable form: -softplus(-x))
  6. h0 = 0.1 * randn(B,H,K,V)                  (only when the workload has one)
then q and k are L2-normalised per token in fp32 (no epsilon) and q, k, v are
rounded to the io dtype (round to nearest even).  beta, g and h0 stay fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    K: int
    V: int
    chunk: int
    io: str             # "fp32" or "bf16"
    gate: str           # "head" (one gate per head) or "key" (per key dim)
    gate_bias: float
    h0: bool
    seed: int

    def tokens(self) -> int:
        return self.B * self.T

    def as_dict(self):
        return asdict(self)


# The five workloads the pages' kernels are shaped for: chunk 32/64, head dims
# 64/128, V tiles of 64, GDN (scalar gate) and KDA (per-key gate).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 128, 64, 64, 64, "fp32", "head", 2.0, False, 0),
    "gdn_t4k": Workload("gdn_t4k", 4, 16, 4096, 128, 128, 64, "bf16", "head", 2.0, True, 1),
    "gdn_c32_d64": Workload("gdn_c32_d64", 8, 32, 2048, 64, 64, 32, "bf16", "head", 4.0, False, 2),
    "kda_t8k": Workload("kda_t8k", 2, 32, 8192, 128, 128, 64, "bf16", "key", 3.0, False, 3),
    "gdn_t64k": Workload("gdn_t64k", 1, 64, 65536, 128, 128, 64, "bf16", "head", 2.0, True, 4),
}
WORKLOAD_ORDER = ["tiny_fp32", "gdn_t4k", "gdn_c32_d64", "kda_t8k", "gdn_t64k"]


def _dtype(io: str):
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[io]


def make_inputs(B, T, H, K, V, *, io="bf16", gate="head", gate_bias=2.0,
                h0=False, seed=0):
    """Return a dict of CPU tensors: q, k, v (io dtype), beta, g, h0 (fp32)."""
    gen = torch.Generator().manual_seed(int(seed))
    f32 = torch.float32
    q = torch.randn(B, T, H, K, generator=gen, dtype=f32)
    k = torch.randn(B, T, H, K, generator=gen, dtype=f32)
    v = torch.randn(B, T, H, V, generator=gen, dtype=f32)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=gen, dtype=f32))
    gshape = (B, T, H, K) if gate == "key" else (B, T, H)
    x = torch.randn(*gshape, generator=gen, dtype=f32) + gate_bias
    g = torch.nn.functional.logsigmoid(x)
    hz = (0.1 * torch.randn(B, H, K, V, generator=gen, dtype=f32)) if h0 else None
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    dt = _dtype(io)
    return {"q": q.to(dt).contiguous(), "k": k.to(dt).contiguous(),
            "v": v.to(dt).contiguous(), "beta": beta.contiguous(),
            "g": g.contiguous(), "h0": hz}


# Length mix for packed sequences: eight sequences whose lengths are these
# shares of the total token count (at 16384 tokens exactly these lengths,
# the longest 4096).
VARLEN_MIX = (4096, 3000, 2500, 2000, 1596, 1200, 1000, 992)


def varlen_lengths(total: int):
    """Sequence lengths of the packed-sequence mix for `total` tokens."""
    base = sum(VARLEN_MIX)
    lens = [total * x // base for x in VARLEN_MIX]
    lens[-1] += total - sum(lens)
    return lens


def workload_inputs(w: Workload, *, T=None, B=None, H=None):
    """Inputs for a named workload; T/B/H may be overridden to shrink it."""
    return make_inputs(B or w.B, T or w.T, H or w.H, w.K, w.V, io=w.io,
                       gate=w.gate, gate_bias=w.gate_bias, h0=w.h0, seed=w.seed)
