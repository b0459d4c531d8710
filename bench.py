#!/usr/bin/env python3
"""Throughput of the chunked gated delta rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one gdn_forward call over one batch of synthetic input already in
HBM (q, k, v, beta, g, h0 -> o, hT), with the workspace gdn_workspace_bytes
asks for (there gdn_forward cuts long streams in two where that fills idle
compute units: gdn_forward_split_point); by default the long-context workload
gdn_t64k (1 x 65536 tokens, 64 heads, dk = dv = 128), the largest that the
five workloads put on one GPU.  Each timed step is bracketed by its own HIP
events on the library's stream; between steps (outside those brackets) a
1 GiB buffer is written so that no input is still in the 256 MB Infinity
Cache.  Prints one JSON line: tokens/s from the mean step time (with the
median and minimum beside it), the roofline of the dominant kernel
(algorithmic bytes per launch over its mean event-timed duration), a plain
device copy's bandwidth measured in the same run, and the fp64 CPU oracle
timed on the host's cores on a bounded sample of the same workload.
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
DEFAULT_WORKLOAD = "gdn_t64k"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB written between timed steps to evict the Infinity Cache (0: none)")
    ap.add_argument("--chunk", type=int, default=None,
                    help="override the workload's chunk size (32 or 64)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--o-dtype", default=None, choices=[None, "bf16", "fp32"])
    ap.add_argument("--states", action="store_true",
                    help="time gdn_forward_states (also saves chunk-start states and v')")
    ap.add_argument("--rescan", action="store_true",
                    help="time gdn_rescan_dq (the backward's re-scan: states, v', dq; no o)")
    ap.add_argument("--varlen", action="store_true",
                    help="time gdn_forward_varlen on the workload's tokens packed as eight "
                         "sequences of mixed lengths")
    ap.add_argument("--chunk-dq", action="store_true",
                    help="time gdn_chunk_dq (dq's state term from saved states, on its own)")
    ap.add_argument("--split", type=float, default=None,
                    help="run gdn_forward_split with the cut at this fraction of T (rounded to "
                         "whole chunks): the scalar gate's two-segment forward")
    ap.add_argument("--no-split", action="store_true",
                    help="make gdn_forward run its single pass where it would split the "
                         "sequence (GDN_FORWARD_NO_SPLIT=1)")
    ap.add_argument("--backward", action="store_true",
                    help="time gdn_backward (the scalar gate's gradients from saved bf16 states; "
                         "the states come from one untimed gdn_forward_states call)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
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


def forward_bytes(w, o_dtype, states=False, rescan=False):
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    per_tok = (io_bytes(w.io) * 2 * K + io_bytes(w.io) * V + io_bytes(o_dtype) * V
               + 4 + 4 * (K if w.gate == "key" else 1))
    if rescan:
        # no o; dO read (io dtype), dq accumulated (fp32, read and written)
        per_tok += io_bytes(w.io) * V - io_bytes(o_dtype) * V + 8 * K
        states = True
    state = 4 * K * V * B * H * (2 if w.h0 else 1)
    saved = 0
    if states:
        # chunk-start states [B,NT,H,K,V] and v' [B,T,H,V], in the o dtype
        nt = (T + w.chunk - 1) // w.chunk
        saved = io_bytes(o_dtype) * (B * nt * H * K * V + B * T * H * V)
    return B * T * H * per_tok + state + saved


def chunk_dq_bytes(w, o_dtype):
    """dO read (io dtype), the saved states read (o dtype), dq written (fp32)."""
    nt = (w.T + w.chunk - 1) // w.chunk
    return (w.B * w.T * w.H * (io_bytes(w.io) * w.V + 4 * w.K)
            + io_bytes(o_dtype) * w.B * nt * w.H * w.K * w.V)


def backward_bytes(w):
    """Inputs q, k, v, dO (io dtype), beta, g, dhT and the saved bf16 states
    (hck, vnew) read once; dq, dk, dv, dbeta, dg, dh0 (fp32) written once
    (g and dg per key for the per-key gate)."""
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    nt = (T + w.chunk - 1) // w.chunk
    gd = K if w.gate == "key" else 1
    per_tok = io_bytes(w.io) * (2 * K + 2 * V) + 4 + 4 * gd + 2 * V + 4 * (2 * K + V) + 4 + 4 * gd
    return B * T * H * per_tok + 2 * B * nt * H * K * V + 8 * B * H * K * V


def backward_flops(w):
    """Per token-head: the reverse scan's Gram halves, inverse, P^T dO, the
    state products and T^T dD (C K + C V + C^2/6 + 3 K V multiply-adds), the
    gradient stage's Gram halves again, dO D^T and dR D^T halves, the three
    state products and F K, F^T Q, G K halves (1.5 C K + C V + 3 K V)."""
    C, K, V = w.chunk, w.K, w.V
    mac = 2.5 * C * K + 2 * C * V + C * C / 6.0 + 6 * K * V
    return 2.0 * mac * w.B * w.T * w.H


def forward_flops(w):
    C, K, V = w.chunk, w.K, w.V
    mac = 1.5 * C * K + C * V + C * C / 6.0 + 3 * K * V
    return 2.0 * mac * w.B * w.T * w.H


def kernel_name(w, o_dtype, states=False, rescan=False):
    """Template instance of the kernel that gdn_forward (or, with states,
    gdn_forward_states) launches: with bf16 io the pipelined kernel of the
    scalar or the per-key gate, with fp32 io the four-wave one."""
    io = {"bf16": "bf16_t", "fp32": "float"}
    st = ", true, false, true" if rescan else (", true" if states else "")
    if w.io == "bf16":
        name = "forward_pipe_kernel" if w.gate == "head" else "forward_pipe_kda_kernel"
        return "%s<%d, %d, %s%s>" % (name, w.chunk, w.K, io[o_dtype], st)
    return "forward_kernel<%d, %d, %s, %s, %s%s>" % (w.chunk, w.K, io[w.io], io[o_dtype],
                                                     "true" if w.gate == "key" else "false", st)


def split_kernel_names(w, o_dtype):
    """The three launches of the scalar gate's sequence split (gdn_forward at a
    nonzero gdn_forward_split_point, or gdn_forward_split)."""
    ot = {"bf16": "bf16_t", "fp32": "float"}[o_dtype]
    return ("forward_pipe_kernel<%d, %d, %s, false, false, false, true> + split_state_kernel<%d, %d> "
            "+ split_out_kernel<%d, %d, %s>" % (w.chunk, w.K, ot, w.K, w.V, w.K, w.V, ot))


def source_digest():
    """sha256 over the HIP sources and the public header: a traffic figure
    measured on other sources no longer describes this kernel."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_gated_delta_prepare_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                   if f.endswith((".h", ".hip")))
    for p in files + [os.path.join(ROOT, "include", "libgdn.h")]:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(w, o_dtype, states=False):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel and workload (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the counter reads for a plain copy of known size), or None when there is
    none or it was taken on different sources.  For the per-key gate the
    figure covers the step's two launches (the Gram kernel and the re-scan),
    like the step's achieved figure."""
    short = kernel_name(w, o_dtype).split("<")[0]
    path = os.path.join(ROOT, "profiles", "%s.%s.%s%s.traffic.json"
                        % (short, w.name, o_dtype, ".states" if states else ""))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU only; --gpus %d is not supported "
              "(batch/head and sequence sharding across GPUs is a design note, not built)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

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

    if args.no_split:
        os.environ["GDN_FORWARD_NO_SPLIT"] = "1"
    w = WORKLOADS[args.workload]
    if args.chunk:
        import dataclasses
        w = dataclasses.replace(w, chunk=args.chunk)
    o_dtype = args.o_dtype or w.io
    inp = workload_inputs(w)
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[o_dtype]
    o = torch.empty(w.B, w.T, w.H, w.V, device=dev, dtype=tdt)
    hT = torch.empty(w.B, w.H, w.K, w.V, device=dev, dtype=torch.float32)
    # the per-key gate's Gram stage writes its triangular factors into a
    # workspace, and the scalar gate's sequence split its segment states and
    # correction basis; allocated here, outside the timed region
    iot = {"bf16": torch.bfloat16, "fp32": torch.float32}[w.io]
    ws_bytes = gdn.workspace_bytes(w.B, w.T, w.H, w.K, w.V, w.chunk, iot, w.gate == "key", tdt)
    # where gdn_forward cuts the streams (0: one pass)
    t_auto = gdn.forward_split_point(w.B, w.T, w.H, w.K, w.V, w.chunk, iot, w.gate == "key", tdt)
    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8) if ws_bytes else None

    n_seqs = 0
    if args.varlen:
        from chunked_gated_delta_prepare_amd.inputs import varlen_lengths
        lens = varlen_lengths(w.B * w.T)
        n_seqs = len(lens)
        import itertools
        cu = torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32, device=dev)
        flat = {n: d[n].reshape(1, w.B * w.T, *d[n].shape[2:]) for n in ("q", "k", "v", "beta", "g")}
        gen = torch.Generator().manual_seed(w.seed + 2000)
        h0v = (0.1 * torch.randn(n_seqs, w.H, w.K, w.V, generator=gen)).to(dev) if w.h0 else None
        ov = torch.empty(1, w.B * w.T, w.H, w.V, device=dev, dtype=tdt)
        hTv = torch.empty(n_seqs, w.H, w.K, w.V, device=dev, dtype=torch.float32)

        def step():
            gdn.forward_varlen(flat["q"], flat["k"], flat["v"], flat["beta"], flat["g"], cu, w.chunk,
                               h0v, o_dtype=tdt, o=ov, hT=hTv)
    elif args.chunk_dq:
        if w.io != "bf16":
            sys.exit("bench: --chunk-dq takes bf16 workloads (gdn_chunk_dq reads bf16 dO)")
        nt = (w.T + w.chunk - 1) // w.chunk
        gen = torch.Generator().manual_seed(w.seed + 1000)
        dout = torch.randn(w.B, w.T, w.H, w.V, generator=gen).to(d["q"].dtype).to(dev)
        hck = (0.1 * torch.randn(w.B, nt, w.H, w.K, w.V, generator=gen)).to(tdt).to(dev)
        dq = torch.empty(w.B, w.T, w.H, w.K, device=dev, dtype=torch.float32)

        def step():
            gdn.chunk_dq(dout, hck, w.chunk, dq=dq)
    elif args.rescan:
        nt = (w.T + w.chunk - 1) // w.chunk
        hck = torch.empty(w.B, nt, w.H, w.K, w.V, device=dev, dtype=tdt)
        vnew = torch.empty(w.B, w.T, w.H, w.V, device=dev, dtype=tdt)
        gen = torch.Generator().manual_seed(w.seed + 1000)
        dout = torch.randn(w.B, w.T, w.H, w.V, generator=gen).to(d["q"].dtype).to(dev)
        dq = torch.zeros(w.B, w.T, w.H, w.K, device=dev, dtype=torch.float32)

        def step():
            # (dq accumulates over the steps; the zeroing is the caller's and
            # not part of the timed re-scan)
            gdn.rescan_dq(d["q"], d["k"], d["v"], d["beta"], d["g"], dout, w.chunk, d["h0"],
                          o_dtype=tdt, hT=hT, hck=hck, vnew=vnew, dq=dq)
    elif args.split is not None:
        if w.gate != "head" or w.io != "bf16" or w.chunk != 64:
            sys.exit("bench: --split takes scalar-gate bf16 workloads at chunk 64")
        t_split = int(round(w.T * args.split / w.chunk)) * w.chunk
        t_split = min(max(t_split, w.chunk), (w.T - 1) // w.chunk * w.chunk)
        pr = gdn.Problem(w.B, w.T, w.H, w.K, w.V, w.chunk, gdn.GDN_BF16,
                         {"bf16": gdn.GDN_BF16, "fp32": gdn.GDN_F32}[o_dtype], gdn.GDN_GATE_HEAD)
        import ctypes
        ws_split = torch.empty(int(gdn.load_library().gdn_workspace_bytes_split(
            ctypes.byref(pr), ctypes.c_int64(t_split))), device=dev, dtype=torch.uint8)

        def step():
            gdn.forward_split(d["q"], d["k"], d["v"], d["beta"], d["g"], w.chunk, t_split, d["h0"],
                              o_dtype=tdt, o=o, hT=hT, workspace=ws_split)
    elif args.backward:
        if w.io != "bf16":
            sys.exit("bench: --backward takes bf16 workloads")
        tdt = torch.bfloat16
        o_dtype = "bf16"
        gen = torch.Generator().manual_seed(w.seed + 3000)
        dout = torch.randn(w.B, w.T, w.H, w.V, generator=gen).to(torch.bfloat16).to(dev)
        dhT = torch.randn(w.B, w.H, w.K, w.V, generator=gen).to(dev)
        _, _, hck, vnew = gdn.forward_states(d["q"], d["k"], d["v"], d["beta"], d["g"], w.chunk,
                                             d["h0"], o_dtype=tdt)
        f32 = dict(device=dev, dtype=torch.float32)
        gsh = (w.B, w.T, w.H, w.K) if w.gate == "key" else (w.B, w.T, w.H)
        grads = dict(dq=torch.empty(w.B, w.T, w.H, w.K, **f32), dk=torch.empty(w.B, w.T, w.H, w.K, **f32),
                     dv=torch.empty(w.B, w.T, w.H, w.V, **f32), dbeta=torch.empty(w.B, w.T, w.H, **f32),
                     dg=torch.empty(*gsh, **f32), dh0=torch.empty(w.B, w.H, w.K, w.V, **f32))
        pr = gdn.Problem(w.B, w.T, w.H, w.K, w.V, w.chunk, gdn.GDN_BF16, gdn.GDN_BF16,
                         gdn.GDN_GATE_KEY if w.gate == "key" else gdn.GDN_GATE_HEAD)
        import ctypes
        ws_b = torch.empty(int(gdn.load_library().gdn_workspace_bytes_backward(ctypes.byref(pr))),
                           device=dev, dtype=torch.uint8)

        def step():
            gdn.backward(d["q"], d["k"], d["v"], d["beta"], d["g"], dout, w.chunk, hck, vnew, dhT,
                         workspace=ws_b, **grads)
    elif args.states:
        nt = (w.T + w.chunk - 1) // w.chunk
        hck = torch.empty(w.B, nt, w.H, w.K, w.V, device=dev, dtype=tdt)
        vnew = torch.empty(w.B, w.T, w.H, w.V, device=dev, dtype=tdt)

        def step():
            gdn.forward_states(d["q"], d["k"], d["v"], d["beta"], d["g"], w.chunk, d["h0"],
                               o_dtype=tdt, o=o, hT=hT, hck=hck, vnew=vnew)
    else:
        def step():
            gdn.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], w.chunk, d["h0"],
                        o_dtype=tdt, o=o, hT=hT, workspace=ws)

    print("bench: workload %s warmup %d" % (w.name, args.warmup), file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- the timed region: exactly K steps, each bracketed by its own
    # events on the stream the library launches on; between steps, outside
    # the brackets, a buffer larger than the Infinity Cache is written
    stream = torch.cuda.current_stream()
    flush = (torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
             if args.flush_mib > 0 else None)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        if flush is not None:
            flush.fill_(1)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = sorted(a.elapsed_time(b) for a, b in evs)
    ms_step = sum(times) / len(times)
    ms_median = times[len(times) // 2] if len(times) % 2 else 0.5 * (
        times[len(times) // 2 - 1] + times[len(times) // 2])
    ms_min = times[0]
    tokens = w.B * w.T
    value = tokens / (ms_step * 1e-3)
    print("bench: %d steps, mean %.4f ms, median %.4f, min %.4f (wall %.4f ms/step with flushes)"
          % (args.steps, ms_step, ms_median, ms_min, wall * 1e3 / args.steps),
          file=sys.stderr, flush=True)
    del flush

    # ---- the dominant kernel.  Scalar gate: a step is one launch of the
    # fused forward kernel, so its mean event-timed duration is ms_step; where
    # gdn_forward splits the sequence, the step is the split instance and its
    # two combine launches.  Per-key gate: a step is the Gram launch then the
    # re-scan launch on one stream.  The events bracket the whole step, so
    # the figure is that of the step's launches together (the kernel trace
    # splits it)
    ms_launch = ms_step
    fbytes, fflops = forward_bytes(w, o_dtype, args.states, args.rescan), forward_flops(w)
    kname = kernel_name(w, o_dtype, args.states, args.rescan)
    if args.varlen:
        # one state per sequence instead of per batch row; the VL instance
        fbytes += 4 * w.K * w.V * w.H * (n_seqs - w.B) * (2 if w.h0 else 1)
        kname = kname[:-1] + ", false, true>"
    if args.chunk_dq:
        fbytes, fflops = chunk_dq_bytes(w, o_dtype), 2.0 * w.B * w.T * w.H * w.K * w.V
        kname = "chunk_dq_kernel<%d, %d, %d, %s>" % (w.chunk, w.K, w.V,
                                                     {"bf16": "bf16_t", "fp32": "float"}[o_dtype])
    launches = 1
    if args.backward:
        fbytes, fflops = backward_bytes(w), backward_flops(w)
        if w.gate == "key":
            launches = 4
            kname = ("bwd_prep_kda_kernel<%d, %d> + bwd_dh_kda_kernel<%d, %d> + bwd_grad_kda_kernel<%d, %d, %d> "
                     "+ bwd_dec_kda_kernel<%d, %d>" % (w.chunk, w.K, w.chunk, w.K, w.chunk, w.K, w.V, w.chunk, w.K))
        else:
            launches = 3
            kname = "bwd_prep_kernel<%d, %d> + bwd_dh_kernel<%d, %d> + bwd_grad_kernel<%d, %d, %d>" % (
                w.chunk, w.K, w.chunk, w.K, w.chunk, w.K, w.V)
    plain = not (args.states or args.rescan or args.varlen or args.chunk_dq or args.backward
                 or args.split is not None)
    if args.split is not None or (plain and t_auto > 0):
        launches = 3
        kname = split_kernel_names(w, o_dtype)
    if w.gate == "key" and not args.chunk_dq and not args.backward:
        launches = 2
        kname = "kda_gram_kernel<%d, %d, %s%s> + %s" % (
            w.chunk, w.K, {"bf16": "bf16_t", "fp32": "float"}[w.io],
            ", true" if args.varlen else ", false", kname)
    achieved = fbytes / (ms_launch * 1e-3) / 1e9
    mfma_peak = MFMA_PEAK_TFLOPS["f16" if w.io == "bf16" else "f32"]
    roofline = {"kernel": kname, "bound": "hbm",
                "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": (None if args.rescan or args.chunk_dq or args.varlen or args.split is not None
                            or args.backward or args.no_split
                            else measured_traffic(w, o_dtype, args.states)),
                "ms_per_launch": round(ms_launch, 5), "launches_per_step": launches,
                "algorithmic_bytes_per_launch": fbytes,
                "algorithmic_flops_per_launch": fflops,
                "mfma_frac": round(fflops / (ms_launch * 1e-3) / 1e12 / mfma_peak, 4),
                "mfma_peak_tflops": mfma_peak}

    # ---- what a plain device copy reaches on this GPU, for scale
    copy_ref = copy_bandwidth(torch, dev)

    # ---- the oracle on the host's cores, on a bounded sample of the workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, args.cpu_seconds)

    line = {
        "metric": (METRIC.replace("forward", "backward") if args.backward else METRIC),
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "ms_median": round(ms_median, 5), "ms_min": round(ms_min, 5),
        "flush_between_steps_bytes": args.flush_mib << 20,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.io == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "K": w.K, "V": w.V,
                   "chunk": w.chunk, "io": w.io, "o_dtype": o_dtype, "gate": w.gate,
                   "h0": w.h0, "states": bool(args.states), "rescan": bool(args.rescan),
                   "chunk_dq": bool(args.chunk_dq), "varlen_seqs": n_seqs or None,
                   "split_at": (t_split if args.split is not None else (t_auto if plain and t_auto else None)),
                   "backward": bool(args.backward),
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "copy_ref": copy_ref,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def copy_bandwidth(torch, dev, mib=1024, reps=10):
    """A plain device-to-device copy of `mib` MiB (torch's copy kernel), timed
    with events: bytes read plus written per second, the practical ceiling a
    streaming kernel can reach on this GPU."""
    n = mib << 20
    x = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    gbs = 2 * n / (ms * 1e-3) / 1e9
    del x, y
    return {"bytes_read": n, "bytes_written": n, "ms": round(ms, 4), "GB/s": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inp, target_s):
    """Time the fp64 oracle on whole (batch, head) sequences of the same
    workload: grow the sample until one pass takes a quarter of target_s (or
    covers every sequence), then repeat that pass until about target_s of
    wall time has been spent, and report the mean rate."""
    import oracle

    # one thread per (batch, head) sequence, on the cores this process may
    # use, at most 16: a GPU host's CPU share per GPU
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    nthreads = max(1, min(avail, 16))
    q = inp["q"].float().numpy()
    k = inp["k"].float().numpy()
    v = inp["v"].float().numpy()
    beta, g = inp["beta"].numpy(), inp["g"].numpy()
    h0 = None if inp["h0"] is None else inp["h0"].numpy()
    pairs = w.B * w.H

    def run(n):
        t0 = time.perf_counter()
        oracle.token_recurrence(q, k, v, beta, g, h0, heads=list(range(n)), nthreads=nthreads,
                                want_hT=False)
        return time.perf_counter() - t0

    n = min(pairs, nthreads)
    while True:
        spent = run(n)
        if spent >= target_s / 4 or n >= pairs:
            break
        n = min(pairs, max(n + 1, int(n * min(8.0, target_s / max(spent, 1e-3)))))
    times = [spent]
    while sum(times) < target_s and len(times) < 100:
        times.append(run(n))
    token_heads_per_s = n * w.T * len(times) / sum(times)
    return {"value": round(token_heads_per_s / w.H, 1), "unit": "tokens/s",
            "cores": min(nthreads, n), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "cpus_usable": avail,
            "sample": "%d of %d (batch, head) sequences of %d tokens, %d passes; fp64 token "
                      "recurrence in C, one thread per sequence; tokens/s = token-heads/s / H"
                      % (n, pairs, w.T, len(times)),
            "seconds": round(sum(times), 3)}


if __name__ == "__main__":
    main()
