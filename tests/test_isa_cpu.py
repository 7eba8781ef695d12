"""The built library's gfx950 machine code (CPU; our own build only).

A flat memory instruction resolves its address at run time to LDS, scratch
or global memory; a flat access whose base lands outside the LDS aperture
while meant for LDS faults the GPU (a row-window kernel once did exactly
that).  Every kernel of libgattn addresses global memory through global_*
or buffer_* instructions and LDS through ds_* instructions, so the code
objects must hold no flat_* memory instruction at all.  The code objects
are taken from the offload bundles in the built libgattn.so and
disassembled with the ROCm toolchain's llvm-objdump.
"""
import os
import re
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def code_objects(lib_path, arch="gfx950"):
    """The device code objects for `arch` in the offload bundles of a built
    shared library (uncompressed bundles: magic, entry count, then per entry
    offset, size, id length and id)."""
    data = open(lib_path, "rb").read()
    out, pos = [], 0
    while True:
        i = data.find(BUNDLE_MAGIC, pos)
        if i < 0:
            return out
        count = struct.unpack_from("<Q", data, i + len(BUNDLE_MAGIC))[0]
        off = i + len(BUNDLE_MAGIC) + 8
        for _ in range(count):
            o, size, idlen = struct.unpack_from("<QQQ", data, off)
            off += 24
            ident = data[off:off + idlen].decode()
            off += idlen
            if arch in ident and size > 0:
                out.append(data[i + o:i + o + size])
        pos = i + 1


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="ROCm llvm-objdump not installed")
def test_no_flat_memory_instructions(tmp_path):
    from graph_sparse_attention_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    objs = code_objects(b.LIB, b.ARCH)
    assert len(objs) == sum(s.endswith(".hip") for s in b.SOURCES), "one gfx950 code object per HIP source"
    flat = re.compile(r"^\s+flat_\w+", re.M)
    kernels = 0
    for k, blob in enumerate(objs):
        path = tmp_path / f"co{k}.o"
        path.write_bytes(blob)
        asm = subprocess.run([OBJDUMP, "-d", f"--mcpu={b.ARCH}", str(path)], capture_output=True, text=True,
                             check=True).stdout
        kernels += len(re.findall(r"^[0-9a-f]+ <(\w+)>:", asm, re.M))
        hits = flat.findall(asm)
        assert not hits, f"code object {k}: {len(hits)} flat memory instructions, e.g. {hits[0].strip()}"
    assert kernels > 0
