"""Every kernel of the built library runs without scratch memory and issues its copies
without per-lane resource loops.

A kernel that runs out of registers can have the compiler move state to per-lane scratch
(private) memory; the kernel stays correct but slows down several-fold, which no parity
test notices. This reads the code-object metadata of the library built in this tree (the
gfx950 bundle of every object in its .hip_fatbin section) and checks each kernel's
private segment size.

Likewise, a buffer load whose resource (base address, range) the compiler cannot prove
equal in every lane is wrapped in a loop over the distinct resources of the wave's lanes
(v_readfirstlane of the resource, a compare, and an exec-mask loop around the load). The
result is the same; the copies issue several times slower. The disassembly of the same
code objects is checked for buffer loads issued under such a loop.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from learned_context_ranking_amd import sas

LLVM = "/opt/rocm/llvm/bin"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.access(path, os.X_OK):
        pytest.skip(f"{path} not available")
    return path


def _code_objects(lib_path: str, tmp: str) -> list[str]:
    """Paths of the gfx950 code objects embedded in the library, unbundled into tmp."""
    objcopy, bundler = _tool("llvm-objcopy"), _tool("clang-offload-bundler")
    fat = os.path.join(tmp, "fatbin")
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", lib_path], check=True)
    data = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)]
    assert starts, "no offload bundle in .hip_fatbin"
    cos = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        part, co = os.path.join(tmp, f"b{n}"), os.path.join(tmp, f"b{n}.co")
        with open(part, "wb") as f:
            f.write(data[a:b])
        subprocess.run([bundler, "--unbundle", "--type=o", f"--targets={TARGET}", f"--input={part}",
                        f"--output={co}"], check=True)
        cos.append(co)
    return cos


def kernel_private_sizes(lib_path: str) -> dict[str, int]:
    """Kernel name -> private segment bytes, from the library's embedded code objects."""
    readelf = _tool("llvm-readelf")
    sizes: dict[str, int] = {}
    with tempfile.TemporaryDirectory() as tmp:
        for co in _code_objects(lib_path, tmp):
            notes = subprocess.run([readelf, "--notes", co], check=True, capture_output=True, text=True).stdout
            name = None
            for line in notes.splitlines():
                m = re.match(r"\s+\.name:\s+(\S+)", line)
                if m:
                    name = m.group(1)
                m = re.match(r"\s+\.private_segment_fixed_size:\s+(\d+)", line)
                if m and name is not None:
                    sizes[name] = int(m.group(1))
                    name = None
    return sizes


def resource_loop_loads(lib_path: str) -> dict[str, int]:
    """Kernel name -> number of buffer loads issued inside a per-lane resource loop: a
    buffer load right after an s_and_saveexec whose mask came from comparing the lanes'
    resource registers with the first active lane's (v_readfirstlane)."""
    objdump = _tool("llvm-objdump")
    found: dict[str, int] = {}
    with tempfile.TemporaryDirectory() as tmp:
        for co in _code_objects(lib_path, tmp):
            text = subprocess.run([objdump, "-d", "--no-show-raw-insn", co], check=True, capture_output=True,
                                  text=True).stdout
            name, window = None, []
            for line in text.splitlines():
                m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
                if m:
                    name, window = m.group(1), []
                    continue
                ins = line.strip().split(" ")[0] if line.strip() else ""
                if not ins or name is None:
                    continue
                if ins.startswith("buffer_load") and window and window[-1] == "s_and_saveexec_b64" \
                        and "v_readfirstlane_b32" in window:
                    found[name] = found.get(name, 0) + 1
                window = (window + [ins])[-10:]
    return found


def test_no_kernel_uses_scratch():
    if not os.path.exists(sas.LIB_PATH):
        pytest.skip("library not built")
    sizes = kernel_private_sizes(sas.LIB_PATH)
    assert len(sizes) >= 20, sizes   # every object's kernels were found
    assert any("decode_split_kernel" in k for k in sizes) and any("dkv_kernel" in k for k in sizes)
    spilled = {k: v for k, v in sizes.items() if v != 0}
    assert not spilled, f"kernels using scratch memory: {spilled}"


def test_no_copy_in_a_resource_loop():
    if not os.path.exists(sas.LIB_PATH):
        pytest.skip("library not built")
    loops = resource_loop_loads(sas.LIB_PATH)
    assert not loops, f"buffer loads inside per-lane resource loops: {loops}"
