"""Checks on the machine code of the built library (gfx950 code objects
disassembled on the host; no GPU).

* m0 is written only right before an LDS-DMA transfer.  The tile loaders set
  m0 from inline assembly and do not restore it, which is sound only while
  the compiler itself keeps nothing in m0 (no indexed register access, no
  messages, no LDS-DMA builtins): no other instruction may name m0.
* No packed fp32 VALU instructions: the library is built with them turned
  off, and nothing may bring them back.
* No kernel uses scratch memory: the prefill kernels run at 256 VGPRs, and a
  register spill to memory would add a memory round trip per spilled value
  inside their loops.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "long_context_decayed_amd", "liblightning_attn.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    tools = [_tool(t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
    if not all(tools) or not os.path.exists(LIB):
        pytest.skip("ROCm LLVM tools or the built library not found")
    objcopy, bundler, objdump = tools
    d = tmp_path_factory.mktemp("codegen")
    fat = d / "fat.bin"
    subprocess.run([objcopy, "--dump-section", ".hip_fatbin=%s" % fat, LIB], check=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in .hip_fatbin"
    text, notes = [], []
    readelf = _tool("llvm-readelf")
    for i, a in enumerate(starts):
        b = starts[i + 1] if i + 1 < len(starts) else len(data)
        part, co = d / ("b%d.bin" % i), d / ("b%d.co" % i)
        part.write_bytes(data[a:b])
        subprocess.run([bundler, "--unbundle", "--type=o", "--input=%s" % part, "--targets=" + TARGET,
                        "--output=%s" % co], check=True)
        out = subprocess.run([objdump, "-d", "--mcpu=gfx950", str(co)], check=True, capture_output=True, text=True)
        text.append(out.stdout)
        if readelf:
            notes.append(subprocess.run([readelf, "--notes", str(co)], check=True, capture_output=True,
                                        text=True).stdout)
    lines = [l.split("//")[0].strip() for l in "\n".join(text).splitlines()]
    ins = [l for l in lines if l and not l.endswith(":") and not l.startswith("Disassembly")
           and "file format" not in l]
    assert sum(1 for l in ins if l.startswith("v_mfma")) > 100, "disassembly looks empty"
    return {"ins": ins, "notes": "\n".join(notes)}


def _names_m0(ins):
    return re.search(r"\bm0\b", ins) is not None


def test_m0_only_feeds_lds_dma(disassembly):
    ins = disassembly["ins"]
    writes = 0
    for i, l in enumerate(ins):
        if not _names_m0(l):
            continue
        op = l.split()[0]
        assert op == "s_mov_b32", "instruction other than s_mov_b32 names m0: %s" % l
        if re.match(r"s_mov_b32\s+m0\s*,", l):
            writes += 1
            follow = ins[i + 1:i + 3]
            restore = i > 0 and ins[i - 1].startswith("global_load_lds")  # the row-by-row loader's restore
            assert restore or any(f.startswith("global_load_lds") for f in follow), \
                "m0 written without an LDS-DMA transfer right after it: %s / %s" % (l, follow)
        else:
            # a save of m0 into an SGPR (the row-by-row loader restores it)
            assert re.match(r"s_mov_b32\s+s\d+\s*,\s*m0$", l), l
    assert writes > 0


def test_no_packed_fp32(disassembly):
    bad = [l for l in disassembly["ins"] if re.match(r"v_pk_(add|mul|fma)_f32\b", l)]
    assert not bad, bad[:5]


def test_no_scratch(disassembly):
    notes = disassembly["notes"]
    if not notes:
        pytest.skip("llvm-readelf not found")
    names = re.findall(r"\.name:\s+(\S+)", notes)
    sizes = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)]
    assert len(sizes) >= 20 and len(sizes) == len([n for n in names if n.startswith("_Z")]), (len(sizes), len(names))
    kernels = [n for n in names if n.startswith("_Z")]
    bad = [(k, z) for k, z in zip(kernels, sizes) if z != 0]
    assert not bad, bad
