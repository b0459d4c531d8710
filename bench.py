#!/usr/bin/env python3
"""Throughput of the chunked gated delta rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one gdn_forward call over one batch of synthetic input already in
HBM (q, k, v, beta, g, h0 -> o, hT).  Prints one JSON line: tokens/s, the
roofline of the dominant kernel (algorithmic bytes or flops per launch over
its average HIP-event-timed duration), and the fp64 CPU oracle timed on the
host's cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/sec of chunked GDN forward at 1 MI355X; % of bf16 MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
DEFAULT_WORKLOAD = "gdn_t4k"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--o-dtype", default=None, choices=[None, "bf16", "fp32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of known size (counter scale)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (counted once: inputs read, outputs written, no
# intermediates; triangular products at half, the inverse at C^3/6)
# ---------------------------------------------------------------------------

def io_bytes(dt):
    return {"bf16": 2, "fp32": 4}[dt]


def forward_bytes(w, o_dtype):
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    per_tok = (io_bytes(w.io) * 2 * K + io_bytes(w.io) * V + io_bytes(o_dtype) * V
               + 4 + 4 * (K if w.gate == "key" else 1))
    state = 4 * K * V * B * H * (2 if w.h0 else 1)
    return B * T * H * per_tok + state


def forward_flops(w):
    C, K, V = w.chunk, w.K, w.V
    mac = 1.5 * C * K + C * V + C * C / 6.0 + 3 * K * V
    return 2.0 * mac * w.B * w.T * w.H


def scan_bytes(w, o_dtype):
    """gdn_scan kernel: reads q, k (io), w, u, gcum (fp32), h0; writes o, hT."""
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    per_tok = (io_bytes(w.io) * 2 * K + 4 * K + 4 * V + 4 * (K if w.gate == "key" else 1)
               + io_bytes(o_dtype) * V)
    return B * T * H * per_tok + 4 * K * V * B * H * (2 if w.h0 else 1)


def prepare_bytes(w):
    """gdn_prepare kernel: reads k, v (io), beta, g; writes w, u, gcum (fp32)."""
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    g = 4 * (K if w.gate == "key" else 1)
    return B * T * H * (io_bytes(w.io) * (K + V) + 4 + g + 4 * K + 4 * V + g)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(batch/head and sequence sharding across GPUs is a design note, not built)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import chunked_gated_delta_prepare_amd as gdn
    from chunked_gated_delta_prepare_amd.inputs import WORKLOADS, workload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe:
        n = 256 << 20
        x = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                          "launches": 5}))
        return

    w = WORKLOADS[args.workload]
    o_dtype = args.o_dtype or w.io
    inp = workload_inputs(w)
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[o_dtype]
    o = torch.empty(w.B, w.T, w.H, w.V, device=dev, dtype=tdt)
    hT = torch.empty(w.B, w.H, w.K, w.V, device=dev, dtype=torch.float32)
    ws_bytes = gdn.workspace_bytes(w.B, w.T, w.H, w.K, w.V, w.chunk,
                                   {"bf16": torch.bfloat16, "fp32": torch.float32}[w.io],
                                   w.gate == "key", tdt)
    ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)

    def step():
        gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], w.chunk, d["h0"],
                    o_dtype=tdt, o=o, hT=hT, workspace=ws)

    print("bench: workload %s warmup %d" % (w.name, args.warmup), file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- the timed region: exactly K steps, synchronised on both sides
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    tokens = w.B * w.T
    value = tokens / (ms_step * 1e-3)
    print("bench: %d steps, %.4f ms/step (wall %.4f ms/step)"
          % (args.steps, ms_step, wall * 1e3 / args.steps), file=sys.stderr, flush=True)

    # ---- per-kernel durations with events on the same stream: the forward
    # runs gdn_prepare then gdn_scan; time each entry point alone
    wbuf = torch.empty(w.B, w.T, w.H, w.K, device=dev, dtype=torch.float32)
    ubuf = torch.empty(w.B, w.T, w.H, w.V, device=dev, dtype=torch.float32)
    gbuf = torch.empty_like(d["g"])
    gdn.prepare(d["k"], d["v"], d["beta"], d["g"], w.chunk, w=wbuf, u=ubuf, gcum=gbuf)
    torch.cuda.synchronize()

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    n_k = max(5, args.steps // 2)
    ms_prep = timed(lambda: gdn.prepare(d["k"], d["v"], d["beta"], d["g"], w.chunk,
                                        w=wbuf, u=ubuf, gcum=gbuf), n_k)
    ms_scan = timed(lambda: gdn.scan(d["q"], d["k"], wbuf, ubuf, gbuf, w.chunk, d["h0"],
                                     o_dtype=tdt, o=o, hT=hT), n_k)
    kernels = {
        "prepare_kernel": {"ms": ms_prep, "bytes": prepare_bytes(w)},
        "scan_kernel": {"ms": ms_scan, "bytes": scan_bytes(w, o_dtype)},
    }
    dom_name = max(kernels, key=lambda k: kernels[k]["ms"])
    dom = kernels[dom_name]
    achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
    roofline = {"kernel": dom_name, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None, "ms_per_launch": round(dom["ms"], 5),
                "algorithmic_bytes_per_launch": dom["bytes"]}

    fbytes, fflops = forward_bytes(w, o_dtype), forward_flops(w)
    forward_frac = {
        "hbm": round(fbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_bf16": round(fflops / (ms_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
        "algorithmic_bytes": fbytes, "algorithmic_flops": fflops,
    }

    # ---- the oracle on the host's cores, on a bounded sample of the workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.io == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "K": w.K, "V": w.V,
                   "chunk": w.chunk, "io": w.io, "o_dtype": o_dtype, "gate": w.gate,
                   "h0": w.h0, "parallelism": "single-gpu"},
        "roofline": roofline,
        "forward_roofline_frac": forward_frac,
        "kernels_ms": {k: round(v["ms"], 5) for k, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, inp, target_s):
    """Time the fp64 oracle on whole heads of the same workload, growing the
    sample until it takes about target_s seconds (or covers every head)."""
    import numpy as np
    import oracle

    nthreads = min(os.cpu_count() or 1, 16)
    q = inp["q"].float().numpy()
    k = inp["k"].float().numpy()
    v = inp["v"].float().numpy()
    beta, g = inp["beta"].numpy(), inp["g"].numpy()
    h0 = None if inp["h0"] is None else inp["h0"].numpy()
    pairs = w.B * w.H
    n = min(pairs, nthreads)
    spent = 0.0
    while True:
        heads = list(range(n))
        t0 = time.perf_counter()
        oracle.token_recurrence(q, k, v, beta, g, h0, heads=heads, nthreads=nthreads,
                                want_hT=False)
        spent = time.perf_counter() - t0
        if spent >= target_s / 4 or n >= pairs:
            break
        n = min(pairs, max(n + 1, int(n * min(8.0, target_s / max(spent, 1e-3)))))
    token_heads_per_s = n * w.T / spent
    return {"value": round(token_heads_per_s / w.H, 1), "unit": "tokens/s",
            "cores": min(nthreads, n), "kind": "oracle",
            "sample": "%d of %d (batch, head) sequences of %d tokens, fp64 token recurrence "
                      "in C; tokens/s = token-heads/s / H" % (n, pairs, w.T),
            "seconds": round(spent, 3)}


if __name__ == "__main__":
    main()
