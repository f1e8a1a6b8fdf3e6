"""Every kernel of the built library runs without scratch memory.

A kernel that runs out of registers can have the compiler move state to per-lane scratch
(private) memory; the kernel stays correct but slows down several-fold, which no parity
test notices. This reads the code-object metadata of the library built in this tree (the
gfx950 bundle of every object in its .hip_fatbin section) and checks each kernel's
private segment size.
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


def kernel_private_sizes(lib_path: str) -> dict[str, int]:
    """Kernel name -> private segment bytes, from the library's embedded code objects."""
    objcopy, bundler, readelf = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), _tool("llvm-readelf")
    sizes: dict[str, int] = {}
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", lib_path], check=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)]
        assert starts, "no offload bundle in .hip_fatbin"
        for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            part, co = os.path.join(tmp, f"b{n}"), os.path.join(tmp, f"b{n}.co")
            with open(part, "wb") as f:
                f.write(data[a:b])
            subprocess.run([bundler, "--unbundle", "--type=o", f"--targets={TARGET}", f"--input={part}",
                            f"--output={co}"], check=True)
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


def test_no_kernel_uses_scratch():
    if not os.path.exists(sas.LIB_PATH):
        pytest.skip("library not built")
    sizes = kernel_private_sizes(sas.LIB_PATH)
    assert len(sizes) >= 20, sizes   # every object's kernels were found
    assert any("decode_split_kernel" in k for k in sizes) and any("dkv_kernel" in k for k in sizes)
    spilled = {k: v for k, v in sizes.items() if v != 0}
    assert not spilled, f"kernels using scratch memory: {spilled}"
