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
# the debug build: every pipelined kernel fills its LDS stages with NaN once
# their last reader is done (GDN_POISON_LDS); same ABI, same entry points
POISON_LIB = os.path.join(HERE, "libgdn_poison.so")
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


def build(verbose: bool = False, extra_flags=None, poison: bool = False) -> str:
    """Compile every HIP source into libgdn.so (or, with poison, the debug
    library libgdn_poison.so); returns the library path."""
    tag = ".tmp%d%s" % (os.getpid(), "p" if poison else "")
    out = POISON_LIB if poison else LIB
    extra_flags = list(extra_flags or []) + (["-DGDN_POISON_LDS=1"] if poison else [])
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
        tmp = out + tag
        bad, log = _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs,
                        verbose)
        if bad:
            sys.stderr.write(log[-8000:])
            raise RuntimeError("hipcc failed linking libgdn.so")
        # every kernel symbol must resolve (RTLD_NOW fails on any missing one)
        ctypes.CDLL(tmp, mode=os.RTLD_NOW)
        os.replace(tmp, out)
    finally:
        for p in objs + [out + tag]:
            if os.path.exists(p):
                os.remove(p)
    return out


def build_all(verbose: bool = False) -> None:
    """Both libraries: libgdn.so and the debug libgdn_poison.so."""
    build(verbose=verbose)
    build(verbose=verbose, poison=True)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, poison=True))
