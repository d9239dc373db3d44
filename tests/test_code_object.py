"""Static checks of the gfx950 code objects inside the built libbgb.so (our
own build, read with the ROCm LLVM tools). Nothing runs on a GPU.

Every kernel must contain an s_endpgm: a kernel whose body the compiler has
removed (undefined behaviour in the source lets it do that) has none, and its
waves would run on into whatever code follows. Every kernel must also run
without scratch memory and without register spills, which the launch paths
are designed to avoid (scalar registers parked in vector-register lanes
are allowed: that costs no memory traffic).
"""
import os
import re
import struct
import subprocess

import pytest

import bit_gemm_binarize_amd as bgb

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def code_objects(path):
    """The gfx950 entries of every offload bundle embedded in the shared library."""
    blob = open(path, "rb").read()
    out = []
    i = blob.find(MAGIC)
    while i >= 0:
        (count,) = struct.unpack_from("<Q", blob, i + len(MAGIC))
        off = i + len(MAGIC) + 8
        for _ in range(count):
            o, size, tlen = struct.unpack_from("<QQQ", blob, off)
            off += 24
            triple = blob[off:off + tlen].decode()
            off += tlen
            if "gfx950" in triple and size:
                out.append(blob[i + o:i + o + size])
        i = blob.find(MAGIC, i + 1)
    return out


@pytest.fixture(scope="module")
def objects(tmp_path_factory):
    if not os.path.exists(bgb.lib_path()):
        pytest.fail("libbgb.so is not built (python -m bit_gemm_binarize_amd.build)")
    if not os.path.exists(os.path.join(LLVM, "llvm-objdump")):
        pytest.skip("ROCm LLVM tools not installed")
    d = tmp_path_factory.mktemp("co")
    paths = []
    for n, co in enumerate(code_objects(bgb.lib_path())):
        p = d / f"co{n}.elf"
        p.write_bytes(co)
        paths.append(str(p))
    assert paths, "no gfx950 code object in libbgb.so"
    return paths


def run(*args):
    return subprocess.run(args, capture_output=True, text=True, check=True).stdout


def kernels_meta(path):
    notes = run(f"{LLVM}/llvm-readelf", "--notes", path)
    metas = []
    for block in re.split(r"\n  - ", notes)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        get = lambda k: int(re.search(r"\." + k + r":\s+(\d+)", block).group(1))
        metas.append(dict(name=name.group(1), scratch=get("private_segment_fixed_size"),
                          vspill=get("vgpr_spill_count")))
    return metas


def test_every_kernel_ends(objects):
    total = 0
    for path in objects:
        metas = kernels_meta(path)
        dis = run(f"{LLVM}/llvm-objdump", "-d", "--no-show-raw-insn", path)
        bodies = {}
        for m in re.finditer(r"^[0-9a-f]+ <([^>]+)>:\n(.*?)(?=^[0-9a-f]+ <|\Z)", dis, re.M | re.S):
            bodies[m.group(1)] = m.group(2)
        for k in metas:
            total += 1
            assert k["name"] in bodies, f"{k['name']} has no code"
            assert "s_endpgm" in bodies[k["name"]], f"{k['name']} has no s_endpgm (body removed)"
    assert total > 20


def test_no_scratch_or_spills(objects):
    for path in objects:
        for k in kernels_meta(path):
            assert k["scratch"] == 0 and k["vspill"] == 0, k
