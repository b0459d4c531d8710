"""Host-only checks of the gfx950 code objects inside libgdn.so and its debug
build libgdn_poison.so (both built here from this repository's sources):
every kernel the dispatch can launch is present, no kernel uses scratch
memory, and no vector-memory store writes more than 8 bytes per lane.

Scratch: a register array indexed with a run-time value is moved to
per-lane scratch memory, which silently costs a large factor in speed; the
kernels index their register arrays with constants only.

The second rule guards against a miscompile seen with this toolchain: after
a 12- or 16-byte buffer/global store, the compiler may let the next vector
instruction overwrite the store's data registers before the store has read
them, and some lanes then store the new value.  The kernels only use stores
of at most 8 bytes, and this test keeps it that way."""
import os
import re
import shutil
import subprocess

import pytest

LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip("%s not available" % path)
    return path


@pytest.fixture(scope="module", params=["libgdn", "libgdn_poison"])
def disassembly(tmp_path_factory, request):
    import chunked_gated_delta_prepare_amd as gdn
    poison = request.param == "libgdn_poison"
    path = gdn.POISON_LIB_PATH if poison else gdn.LIB_PATH
    if not os.path.exists(path):
        from chunked_gated_delta_prepare_amd import build
        build.build(poison=poison)
    objcopy, bundler, objdump, readelf = (_tool("llvm-objcopy"), _tool("clang-offload-bundler"),
                                          _tool("llvm-objdump"), _tool("llvm-readelf"))
    d = tmp_path_factory.mktemp("co")
    fat = d / "fatbin.bin"
    subprocess.run([objcopy, "--dump-section", ".hip_fatbin=%s" % fat, path], check=True)
    data = fat.read_bytes()
    # one offload bundle per translation unit, concatenated in the section
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in libgdn.so"
    text, notes = [], []
    for n, s in enumerate(starts):
        e = starts[n + 1] if n + 1 < len(starts) else len(data)
        b = d / ("b%d.bin" % n)
        b.write_bytes(data[s:e])
        co = d / ("co%d.o" % n)
        subprocess.run([bundler, "--unbundle", "--type=o", "--targets=" + TARGET,
                        "--input=%s" % b, "--output=%s" % co], check=True)
        text.append(subprocess.run([objdump, "-d", str(co)], capture_output=True, text=True,
                                   check=True).stdout)
        notes.append(subprocess.run([readelf, "--notes", str(co)], capture_output=True, text=True,
                                    check=True).stdout)
    yield "\n".join(text), "\n".join(notes)
    shutil.rmtree(d, ignore_errors=True)


def test_no_vector_memory_store_wider_than_8_bytes(disassembly):
    wide = re.findall(r"\b((?:buffer|global|flat)_store_(?:dwordx3|dwordx4|b96|b128))\b",
                      disassembly[0])
    assert not wide, "wide vector-memory stores in libgdn: %s" % sorted(set(wide))


def test_every_dispatched_kernel_is_present(disassembly):
    names = set(re.findall(r"^[0-9a-f]+ <(_ZN3gdn\w+)>:", disassembly[0], flags=re.M))
    demangled = " ".join(names)
    for kernel in ("forward_pipe_kernelILi64ELi128ENS_6bf16_t", "forward_pipe_kernelILi64ELi128Ef",
                   "forward_pipe_kernelILi32ELi64ENS_6bf16_t", "forward_pipe_kernelILi32ELi128ENS_6bf16_t",
                   "forward_kernelILi64ELi128ENS_6bf16_tES1_Lb1", "forward_kernelILi64ELi64EffLb0",
                   "forward_pipe_kda_kernelILi64ELi128ENS_6bf16_t",
                   "forward_pipe_kda_kernelILi32ELi64ENS_6bf16_t",
                   # instances that save states (ST) and read packed sequences (VL)
                   "forward_pipe_kernelILi64ELi128ENS_6bf16_tELb1ELb0",
                   "forward_pipe_kernelILi64ELi128ENS_6bf16_tELb0ELb1",
                   "forward_pipe_kda_kernelILi64ELi128ENS_6bf16_tELb1ELb0",
                   "forward_pipe_kda_kernelILi64ELi128ENS_6bf16_tELb0ELb1",
                   # the re-scan with dq (DQ) and dq from saved states
                   "forward_pipe_kernelILi64ELi128ENS_6bf16_tELb1ELb0ELb1",
                   "forward_pipe_kda_kernelILi64ELi128ENS_6bf16_tELb1ELb0ELb1",
                   "chunk_dq_kernelILi64ELi128ELi128E", "chunk_dq_kernelILi32ELi64ELi64E",
                   "prepare_kernel", "scan_kernel"):
        assert kernel in demangled, kernel


def test_no_kernel_uses_scratch(disassembly):
    meta = disassembly[1]
    names = re.findall(r"^\s+\.name:\s+(_ZN3gdn\S+)", meta, flags=re.M)
    sizes = [int(s) for s in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", meta)]
    assert names and len(names) == len(sizes), "kernel metadata not parsed"
    bad = [(n, s) for n, s in zip(names, sizes) if s]
    assert not bad, "kernels with scratch: %s" % bad
