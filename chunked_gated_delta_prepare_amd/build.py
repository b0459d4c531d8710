"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

Run ``python -m chunked_gated_delta_prepare_amd.build`` or call ``build()``.
Each translation unit is compiled to a relocatable object with its own flags,
then linked; the result is loaded once with every symbol resolved, because a
device-side compiler crash can otherwise still leave a linkable library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# translation unit -> extra flags
UNITS = {
    "gdn_api.hip": [],
    # schedule for ILP: with one wave per SIMD nothing else hides LDS latency,
    # so fragment loads must run ahead of the matrix instructions using them
    "gdn_forward.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "gdn_forward_pipe.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    # (the ILP scheduler crashes the compiler on these instances)
    "gdn_forward_pipe_c32.hip": [],
    "gdn_forward_states.hip": [],
    "gdn_forward_states_c64.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "gdn_forward_varlen.hip": [],
    "gdn_forward_varlen_c64.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "gdn_forward_pipe_kda.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "gdn_forward_pipe_dq.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "gdn_chunk_dq.hip": [],
    "gdn_kda_gram.hip": [],
    "gdn_forward_pipe_split.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "gdn_split.hip": [],
    "gdn_backward.hip": [],
    "gdn_backward_kda.hip": [],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    bad = res.returncode != 0 or "error:" in res.stderr or "Segmentation fault" in res.stderr
    return bad, res.stdout + res.stderr


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source into libgdn.so; returns the library path."""
    tag = ".tmp%d" % os.getpid()
    objs, jobs = [], []
    for unit, flags in UNITS.items():
        obj = os.path.join(CSRC, unit.replace(".hip", ".o") + tag)
        objs.append(obj)
        jobs.append([HIPCC] + COMMON + flags + list(extra_flags or [])
                    + ["-c", os.path.join(CSRC, unit), "-o", obj])
    try:
        with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
            results = list(ex.map(lambda c: _run(c, verbose), jobs))
        for (bad, log), cmd in zip(results, jobs):
            if bad:
                sys.stderr.write(log[-8000:])
                raise RuntimeError("hipcc failed: %s" % " ".join(cmd[-3:]))
        tmp = LIB + tag
        bad, log = _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs,
                        verbose)
        if bad:
            sys.stderr.write(log[-8000:])
            raise RuntimeError("hipcc failed linking libgdn.so")
        # every kernel symbol must resolve (RTLD_NOW fails on any missing one)
        ctypes.CDLL(tmp, mode=os.RTLD_NOW)
        os.replace(tmp, LIB)
    finally:
        for p in objs + [LIB + tag]:
            if os.path.exists(p):
                os.remove(p)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
