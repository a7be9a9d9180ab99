"""Host-only checks of the C ABI: the library loads, exports every symbol that
include/lightning_attn.h declares, and rejects bad arguments before any HIP
call (every call here fails validation, so no device is touched)."""
import ctypes
import os
import re

import pytest

import long_context_decayed_amd as la
from long_context_decayed_amd import build as la_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lightning_attn.h")

LA_OK, LA_ERR_INVALID, LA_ERR_UNSUPPORTED, LA_ERR_HIP, LA_ERR_NOMEM, LA_ERR_WORKSPACE = range(6)

# Fake, 256-byte-aligned, never-dereferenced device addresses.
FAKE = [ctypes.c_void_p(0x7F0000000000 + i * (1 << 36)) for i in range(8)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(la.LIB_PATH):
        la_build.build()
    return la.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|int64_t|const char\*)\s+(lightning_attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("lightning_attn_fwd", "lightning_attn_fwd_f32", "lightning_attn_fwd_bf16_f32out",
                     "lightning_attn_fwd_ex", "lightning_attn_decode_step", "lightning_attn_fwd_workspace_bytes",
                     "lightning_attn_fwd_workspace_bytes_ex",
                     "lightning_attn_fwd_chunk", "lightning_attn_strerror", "lightning_attn_runtime_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_is_gfx950_only(lib):
    """Every device code object embedded in the library targets gfx950, and the
    bundles are uncompressed (the runtime torch ships may predate the format)."""
    blob = open(la.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", blob))
    assert targets == {b"gfx950"}, targets
    assert b"CCOB" not in blob


def _fwd(lib, q=FAKE[0], k=FAKE[1], v=FAKE[2], decay=FAKE[3], out=FAKE[4], kv_in=None, kv_out=None,
         B=1, H=2, N=128, d=64, block=64, ind=0, outd=0, chunk=0, ws=None, wsb=0, flags=0, warm_chunk=0):
    return lib.lightning_attn_fwd_ex(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, block, ind, outd, chunk,
                                     warm_chunk, flags, ws, wsb, None, None, None)


def test_null_pointers_rejected(lib):
    assert _fwd(lib, q=None) == LA_ERR_INVALID
    assert _fwd(lib, k=None) == LA_ERR_INVALID
    assert _fwd(lib, v=None) == LA_ERR_INVALID
    assert _fwd(lib, decay=None) == LA_ERR_INVALID
    assert _fwd(lib, out=None) == LA_ERR_INVALID
    for fn in (lib.lightning_attn_fwd, lib.lightning_attn_fwd_f32, lib.lightning_attn_fwd_bf16_f32out):
        assert fn(None, FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, None, 1, 1, 64, 64, 64, None) == LA_ERR_INVALID


def test_sizes_rejected(lib):
    for kw in (dict(B=0), dict(H=0), dict(N=0), dict(d=0), dict(B=-1), dict(N=-5)):
        assert _fwd(lib, **kw) == LA_ERR_INVALID, kw
    for block in (0, 32, 100, 512):
        assert _fwd(lib, block=block) == LA_ERR_INVALID, block
    for d in (32, 96, 256):
        assert _fwd(lib, d=d) == LA_ERR_UNSUPPORTED, d
    assert _fwd(lib, N=(1 << 24) + 1) == LA_ERR_UNSUPPORTED


def test_dtypes(lib):
    assert _fwd(lib, ind=1, outd=0) == LA_ERR_UNSUPPORTED      # fp32 in, bf16 out
    assert _fwd(lib, ind=2) == LA_ERR_INVALID
    assert _fwd(lib, outd=7) == LA_ERR_INVALID
    assert _fwd(lib, ind=1, outd=1, d=128, block=128) == LA_ERR_UNSUPPORTED  # fp32 d=128 needs block 64


def test_chunk_rejected(lib):
    assert _fwd(lib, chunk=100) == LA_ERR_INVALID
    assert _fwd(lib, chunk=-64) == LA_ERR_INVALID
    assert _fwd(lib, block=128, chunk=64) == LA_ERR_INVALID


def test_alignment_and_overlap(lib):
    assert _fwd(lib, q=ctypes.c_void_p(FAKE[0].value + 2)) == LA_ERR_INVALID
    assert _fwd(lib, kv_in=ctypes.c_void_p(FAKE[5].value + 4)) == LA_ERR_INVALID
    assert _fwd(lib, decay=ctypes.c_void_p(FAKE[3].value + 2)) == LA_ERR_INVALID
    assert _fwd(lib, out=FAKE[0]) == LA_ERR_INVALID                                  # out == q
    assert _fwd(lib, out=ctypes.c_void_p(FAKE[1].value + 64)) == LA_ERR_INVALID       # out inside k
    assert _fwd(lib, out=FAKE[5], kv_out=ctypes.c_void_p(FAKE[5].value + 16)) == LA_ERR_INVALID


def test_workspace_checks(lib):
    need = lib.lightning_attn_fwd_workspace_bytes(1, 2, 128, 64, 64)
    assert need > 0
    assert _fwd(lib, ws=FAKE[6], wsb=need - 1) == LA_ERR_WORKSPACE
    assert _fwd(lib, ws=ctypes.c_void_p(FAKE[6].value + 16), wsb=need) == LA_ERR_INVALID


def test_workspace_and_chunk_values(lib):
    # million-token prefill: 64 heads, d=128, block 256 -> 16384-token chunks, 64 per head (4096 workgroups)
    assert lib.lightning_attn_fwd_chunk(1, 64, 1 << 20, 256, 0) == 16384
    tbl = 64 * 320 * 4
    states = 64 * 64 * 128 * 128 * 4
    guard = 64 * 64 * 8 * 4  # the warm-start check: 8 floats per (b, h, chunk), then one int per (b, h)
    assert lib.lightning_attn_fwd_workspace_bytes(1, 64, 1 << 20, 128, 256) == tbl + states + guard + 64 * 4
    assert lib.lightning_attn_fwd_workspace_bytes_ex(1, 64, 1 << 20, 128, 256, 0) == tbl + states + guard + 64 * 4
    # an explicit chunk: 4096 tokens -> 256 chunk states per head
    assert lib.lightning_attn_fwd_workspace_bytes_ex(1, 64, 1 << 20, 128, 256, 4096) == (
        tbl + 4 * states + 4 * guard + 64 * 4)
    assert lib.lightning_attn_fwd_workspace_bytes_ex(1, 64, 1 << 20, 128, 256, 100) == 0  # not a multiple of block
    # batched: 4 x 64 heads x 65536 tokens -> halve once to reach 2048 workgroups
    assert lib.lightning_attn_fwd_chunk(4, 64, 65536, 64, 0) == 8192
    # 8192 tokens x 64 heads: chunks would halve until >= 2048 workgroups, but
    # stop at the floor N/8 = 1024 (chunk states as large as the data below it)
    assert lib.lightning_attn_fwd_chunk(1, 64, 8192, 256, 0) == 1024
    assert lib.lightning_attn_fwd_chunk(1, 64, 4096, 64, 0) == 512
    assert lib.lightning_attn_fwd_chunk(1, 64, 16384, 64, 0) == 1024
    assert lib.lightning_attn_fwd_chunk(1, 64, 65536, 64, 0) == 2048   # 2048 workgroups above the floor
    # tiny: floor at 256 tokens, capped by the block-rounded length
    assert lib.lightning_attn_fwd_chunk(1, 2, 1024, 64, 0) == 256
    assert lib.lightning_attn_fwd_chunk(1, 1, 100, 64, 0) == 128
    assert lib.lightning_attn_fwd_chunk(1, 1, 100, 64, 192) == 192
    assert lib.lightning_attn_fwd_chunk(1, 1, 100, 64, 100) == -1
    assert lib.lightning_attn_fwd_workspace_bytes(1, 1, 0, 64, 64) == 0
    assert lib.lightning_attn_fwd_workspace_bytes_ex(1, 1, 0, 64, 64, 0) == 0


def test_decode_validation(lib):
    f = lib.lightning_attn_decode_step
    assert f(None, FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, None, 1, 1, 128, None) == LA_ERR_INVALID
    assert f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, None, 0, 1, 128, None) == LA_ERR_INVALID
    assert f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, None, 1, 1, 96, None) == LA_ERR_UNSUPPORTED
    assert f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[0], None, None, 1, 1, 128, None) == LA_ERR_INVALID


def test_decode_slots_validation(lib):
    f = lib.lightning_attn_decode_slots
    ok = (FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], FAKE[5], FAKE[6])
    assert f(None, *ok[1:], 1, 1, 128, 4, None) == LA_ERR_INVALID
    assert f(*ok[:6], None, 1, 1, 128, 4, None) == LA_ERR_INVALID          # no slot table
    assert f(*ok[:5], None, FAKE[6], 1, 1, 128, 4, None) == LA_ERR_INVALID  # no pool
    assert f(*ok, 1, 1, 128, 0, None) == LA_ERR_INVALID                    # empty pool
    assert f(*ok, 0, 1, 128, 4, None) == LA_ERR_INVALID
    assert f(*ok, 1, 1, 96, 4, None) == LA_ERR_UNSUPPORTED
    assert f(*ok[:4], FAKE[0], *ok[5:], 1, 1, 128, 4, None) == LA_ERR_INVALID   # out overlaps q
    assert f(*ok[:5], FAKE[6], FAKE[6], 1, 1, 128, 4, None) == LA_ERR_INVALID   # slots inside the pool


def test_unknown_flags_rejected(lib):
    assert _fwd(lib, flags=4) == LA_ERR_INVALID
    assert _fwd(lib, flags=0x80000000) == LA_ERR_INVALID


def test_silu_flag_rules(lib):
    """LA_FLAG_SILU_QKV (2): forward entry points only, bf16 inputs, block 64."""
    # accepted: validation passes and stops at the too-small workspace, before any HIP call
    for flags in (2, 3):
        assert _fwd(lib, flags=flags, ws=FAKE[5], wsb=1) == LA_ERR_WORKSPACE
    assert _fwd(lib, flags=2, ind=1, outd=1) == LA_ERR_UNSUPPORTED        # fp32 inputs
    for block in (128, 256):
        assert _fwd(lib, flags=2, block=block) == LA_ERR_UNSUPPORTED
    f = lib.lightning_attn_fwd_slots
    base = [FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], FAKE[5], FAKE[6], 1, 1, 128, 64, 4, 256, 0, 0, 2, None]
    assert f(*base) == LA_ERR_UNSUPPORTED                                 # block 256
    bwd = lib.lightning_attn_bwd
    assert bwd(*FAKE[:5], None, None, FAKE[5], FAKE[6], FAKE[7], None, 1, 2, 64, 64, 0, 0, 2, None, 0,
               None) == LA_ERR_INVALID                                   # the backward takes activated inputs


def test_fwd_slots_validation(lib):
    f = lib.lightning_attn_fwd_slots
    base = [FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], FAKE[5], FAKE[6], 1, 1, 128, 64, 4, 64, 0, 0, 0, None]
    assert f(*base[:5], None, *base[6:]) == LA_ERR_INVALID          # no pool
    assert f(*base[:6], None, *base[7:]) == LA_ERR_INVALID          # no slot table
    a = list(base); a[11] = 0
    assert f(*a) == LA_ERR_INVALID                                  # empty pool
    a = list(base); a[12] = 100
    assert f(*a) == LA_ERR_INVALID                                  # bad block
    a = list(base); a[10] = 96
    assert f(*a) == LA_ERR_UNSUPPORTED
    a = list(base); a[5] = FAKE[0]
    assert f(*a) == LA_ERR_INVALID                                  # pool overlaps q
    a = list(base); a[6] = FAKE[5]
    assert f(*a) == LA_ERR_INVALID                                  # slot table inside the pool
    a = list(base); a[15] = 4
    assert f(*a) == LA_ERR_INVALID                                  # unknown flag


def test_fused_validation(lib):
    f = lib.lightning_attn_decode_fused
    ok = [FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], FAKE[5], None, 4, 1, None, ctypes.c_float(1e-5), None,
          4, 2, 128, None]
    a = list(ok); a[5] = None
    assert f(*a) == LA_ERR_INVALID                      # no pool
    a = list(ok); a[7] = 3
    assert f(*a) == LA_ERR_INVALID                      # no slot table and fewer slots than rows
    a = list(ok); a[10] = ctypes.c_float(-1.0)
    assert f(*a) == LA_ERR_INVALID                      # negative eps
    a = list(ok); a[14] = 96
    assert f(*a) == LA_ERR_UNSUPPORTED
    a = list(ok); a[11] = FAKE[4]
    assert f(*a) == LA_ERR_INVALID                      # gate is the output
    g = lib.lightning_attn_norm_gate
    base = [FAKE[0], 0, None, None, ctypes.c_float(1e-5), FAKE[1], 1, 2, 100, 128, None]
    a = list(base); a[1] = 5
    assert g(*a) == LA_ERR_INVALID                      # bad dtype
    a = list(base); a[9] = 96
    assert g(*a) == LA_ERR_UNSUPPORTED
    a = list(base); a[5] = ctypes.c_void_p(FAKE[0].value + 256)
    assert g(*a) == LA_ERR_INVALID                      # out overlaps o, not in place
    a = list(base); a[1] = 1; a[5] = FAKE[0]
    assert g(*a) == LA_ERR_INVALID                      # in place needs a bf16 o
    s = lib.lightning_attn_silu
    assert s(None, 5, None) == LA_ERR_INVALID
    assert s(FAKE[0], -1, None) == LA_ERR_INVALID
    assert s(None, 0, None) == LA_OK                    # nothing to do, no device call
    assert s(ctypes.c_void_p(FAKE[0].value + 2), 8, None) == LA_ERR_INVALID


def test_bwd_validation(lib):
    f = lib.lightning_attn_bwd
    q, k, v, dec, g = FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4]
    dq, dk, dv = FAKE[5], FAKE[6], FAKE[7]
    args = lambda **kw: [kw.get("q", q), k, v, dec, kw.get("g", g), None, None, kw.get("dq", dq), dk, dv, None,
                         kw.get("B", 1), 1, kw.get("N", 128), kw.get("d", 128), kw.get("idt", 0), kw.get("od", 0),
                         kw.get("fl", 0), None, 0, None]
    assert f(*args(q=None)) == LA_ERR_INVALID
    assert f(*args(g=None)) == LA_ERR_INVALID
    assert f(*args(B=0)) == LA_ERR_INVALID
    assert f(*args(od=7)) == LA_ERR_INVALID
    assert f(*args(idt=7)) == LA_ERR_INVALID
    assert f(*args(idt=1, od=0)) == LA_ERR_UNSUPPORTED           # fp32 in needs fp32 out
    assert f(*args(fl=2)) == LA_ERR_INVALID                        # unknown flag
    assert f(*args(d=96)) == LA_ERR_UNSUPPORTED
    assert f(*args(dq=FAKE[0])) == LA_ERR_INVALID            # dq overlaps q
    assert f(*args(dq=ctypes.c_void_p(FAKE[5].value + 8))) == LA_ERR_INVALID   # misaligned
    small = (ctypes.c_uint8 * 16)()
    a = args()
    a[18], a[19] = FAKE[5], 16                                 # workspace too small
    assert f(*a) == LA_ERR_WORKSPACE
    need = lib.lightning_attn_bwd_workspace_bytes(1, 64, 1 << 20, 128)
    fwd = lib.lightning_attn_fwd_workspace_bytes(1, 64, 1 << 20, 128, 64)
    tbl = 64 * 128 * 4  # decay table: H rows of 128 floats (block + 1 rounded up to 64)
    assert need == fwd + (fwd - tbl) + 2 * 64 * 128 * 128 * 4  # second chunk-state area, S0^T, dS_N^T
    assert lib.lightning_attn_bwd_workspace_bytes(1, 1, 0, 128) == 0


def test_strerror(lib):
    for code in range(6):
        s = lib.lightning_attn_strerror(code).decode()
        assert s and s != "unknown status"
    assert lib.lightning_attn_strerror(99).decode() == "unknown status"


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(la, "_lib", None)
    monkeypatch.setattr(la, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        la.load()


def test_sizes_beyond_the_byte_arithmetic_rejected(lib):
    """B, H and the row counts stay below 2^31 and B*H*N below 2^48, so that no
    byte count overflows int64 (the pointers are fake; nothing is launched)."""
    big = 1 << 40
    for kw in (dict(B=big), dict(H=big), dict(B=1 << 16, H=1 << 16), dict(B=1 << 20, H=1 << 10, N=1 << 24)):
        assert _fwd(lib, **kw) == LA_ERR_UNSUPPORTED, kw
    # B*H*N = 2^48 exactly passes validation (pointers 2^57 apart, one chunk so the
    # grid fits) and stops at the too-small workspace, before any HIP call
    far = [ctypes.c_void_p((i + 1) << 57) for i in range(6)]
    assert _fwd(lib, *far[:5], B=1 << 14, H=1 << 10, N=1 << 24, chunk=1 << 24, ws=far[5], wsb=1) == LA_ERR_WORKSPACE
    dec = lib.lightning_attn_decode_step
    assert dec(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, None, big, big, 64, None) == LA_ERR_UNSUPPORTED
    slots = lib.lightning_attn_decode_slots
    assert slots(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], FAKE[5], FAKE[6], 1, 1 << 16, 64, 1 << 16,
                 None) == LA_ERR_UNSUPPORTED
    fs = lib.lightning_attn_fwd_slots
    assert fs(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], FAKE[5], FAKE[6], 1, 1 << 16, 64, 64, 1 << 16, 64, 0, 0,
              0, None) == LA_ERR_UNSUPPORTED
    bwd = lib.lightning_attn_bwd
    assert bwd(*FAKE[:5], None, None, FAKE[5], FAKE[6], FAKE[7], None, big, 2, 64, 64, 0, 0, 0, None, 0,
               None) == LA_ERR_UNSUPPORTED
    ng = lib.lightning_attn_norm_gate
    assert ng(FAKE[0], 0, None, None, ctypes.c_float(1e-5), FAKE[1], big, big, 64, 64, None) == LA_ERR_UNSUPPORTED
    assert lib.lightning_attn_silu(FAKE[0], (1 << 44) + 8, None) == LA_ERR_UNSUPPORTED


def test_partially_overlapping_states_rejected(lib):
    """kv_in and kv_out are the same tensor or apart: a shifted alias would let
    one (b, h) overwrite another's state before it is read."""
    st = 2 * 64 * 64 * 4  # B=1, H=2, d=64
    base = FAKE[5].value
    same = dict(kv_in=ctypes.c_void_p(base), kv_out=ctypes.c_void_p(base))
    shifted = dict(kv_in=ctypes.c_void_p(base), kv_out=ctypes.c_void_p(base + 64 * 64 * 4))
    apart = dict(kv_in=ctypes.c_void_p(base), kv_out=ctypes.c_void_p(base + st))
    assert _fwd(lib, **shifted) == LA_ERR_INVALID
    # validation passes for the other two; they then stop at the too-small workspace
    for kw in (same, apart):
        assert _fwd(lib, ws=FAKE[6], wsb=1, **kw) == LA_ERR_WORKSPACE
    dec = lib.lightning_attn_decode_step
    assert dec(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], shifted["kv_in"], shifted["kv_out"], 1, 2, 64,
               None) == LA_ERR_INVALID


def test_warm_chunk_rules(lib):
    """The warm-start chunk: default up to four times the scan's default chunk
    while at least 512 workgroups (one round at two per CU) remain; an
    explicit chunk sets both unless warm_chunk is given; an explicit
    warm_chunk is a multiple of 64 and at least the scan's chunk."""
    wc = lib.lightning_attn_fwd_warm_chunk
    assert lib.lightning_attn_fwd_chunk(1, 64, 1 << 20, 64, 0) == 16384
    assert wc(1, 64, 1 << 20, 64, 0, 0) == 65536          # four times the chunk: 16 chunks x 64 heads
    assert wc(1, 32, 1 << 20, 64, 0, 0) == 65536          # 16 x 32 = 512
    assert wc(1, 8, 1 << 20, 64, 0, 0) == 16384           # chunk 4096; 64 x 8 = 512
    assert wc(4, 64, 1 << 16, 64, 0, 0) == 32768          # chunk 8192 for >= 2048; 4 x 64 x 2 = 512
    assert wc(1, 64, 8192, 64, 0, 0) == 1024              # the chunk itself (1024: 8 x 64 = 512 already)
    assert wc(1, 64, 16384, 64, 0, 0) == 2048             # chunk 1024; 8 x 64 = 512
    assert wc(1, 8, 3000, 64, 0, 0) == 256                # too few workgroups to grow
    assert wc(1, 64, 1 << 20, 64, 4096, 0) == 4096        # an explicit chunk sets both
    assert wc(1, 64, 1 << 20, 64, 4096, 32768) == 32768
    assert wc(1, 64, 1 << 20, 64, 4096, 2048) == -1       # shorter than the scan's chunk
    assert wc(1, 64, 1 << 20, 64, 4096, 4100) == -1       # not a multiple of 64
    assert _fwd(lib, chunk=256, warm_chunk=128) == LA_ERR_INVALID
    assert _fwd(lib, chunk=256, warm_chunk=320, ws=FAKE[5], wsb=1) == LA_ERR_WORKSPACE


def test_header_is_plain_c(tmp_path):
    """include/lightning_attn.h compiles as C99 on its own, and every declared
    entry point can be referenced from C (a C caller needs no C++ at all)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc") or shutil.which("cc")
    if gcc is None:
        pytest.skip("no C compiler on this host")
    names = declared_functions()
    src = tmp_path / "use_header.c"
    src.write_text('#include "lightning_attn.h"\n'
                   "const void* entry_points[] = {\n" + "".join("    (const void*)&%s,\n" % n for n in names) +
                   "};\n")
    res = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-Wno-pedantic", "-c",
                          "-I", os.path.join(ROOT, "include"), str(src), "-o", str(tmp_path / "use_header.o")],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_noalloc_scratch_size_matches_binding():
    m = re.search(r"#define\s+LA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*\*\s*(\d+)u\s*\*\s*(\d+)u\)", open(HEADER).read())
    assert m, "LA_NOALLOC_SCRATCH_BYTES not found in the header"
    assert int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == la.NOALLOC_SCRATCH_BYTES


def _noalloc(lib, B=1, H=2, N=128, d=64, chunk=0, warm_chunk=0, flags=0, ind=0, outd=0, q=FAKE[0]):
    return lib.lightning_attn_fwd_noalloc(q, FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, None, B, H, N, d, ind, outd,
                                          chunk, warm_chunk, flags, None)


def test_noalloc_rejects_sizes_beyond_its_array(lib):
    """Workspaces larger than the library's array are refused with
    LA_ERR_WORKSPACE before any HIP call (fake pointers, no device)."""
    # explicit chunk whose chunk states (16 x 64 heads x 256 chunks x 64 KiB) cannot fit
    assert _noalloc(lib, B=16, H=64, N=1 << 16, d=128, chunk=256) == LA_ERR_WORKSPACE
    # default chunk: doubled up to the whole sequence, the states of 4096 heads still need 256 MiB
    assert _noalloc(lib, B=64, H=64, N=1 << 16, d=128) == LA_ERR_WORKSPACE
    # the usual validation still comes first
    assert _noalloc(lib, q=None) == LA_ERR_INVALID
    assert _noalloc(lib, d=96) == LA_ERR_UNSUPPORTED
    assert _noalloc(lib, chunk=100) == LA_ERR_INVALID
    assert _noalloc(lib, flags=4) == LA_ERR_INVALID
    assert _noalloc(lib, warm_chunk=96) == LA_ERR_INVALID


def test_decode_layers_validation(lib):
    P = FAKE

    def call(q=P[0], states=P[5], slots=None, L=2, B=3, H=4, d=64, num_slots=3, eps=1e-5, gamma=None, gate=None):
        return lib.lightning_attn_decode_layers(q, P[1], P[2], P[3], P[4], states, slots, L, B, H, d, num_slots, 0,
                                                gamma, ctypes.c_float(eps), gate, None)

    assert call(q=None) == LA_ERR_INVALID
    assert call(states=None) == LA_ERR_INVALID
    for kw in (dict(L=0), dict(B=0), dict(H=0), dict(num_slots=0), dict(d=0)):
        assert call(**kw) == LA_ERR_INVALID, kw
    assert call(num_slots=2) == LA_ERR_INVALID          # no slot table: the pool must hold the batch
    assert call(eps=-1.0) == LA_ERR_INVALID
    assert call(d=96) == LA_ERR_UNSUPPORTED
    assert call(states=ctypes.c_void_p(P[5].value + 4)) == LA_ERR_INVALID  # misaligned
    assert call(states=P[4]) == LA_ERR_INVALID           # the pool overlapping the output


def test_fwd_fused_validation(lib):
    P = FAKE

    def call(q=P[0], gamma=None, gate=None, eps=1e-5, out=P[4], d=64, outd=0, flags=0, B=1, H=2, N=128):
        return lib.lightning_attn_fwd_fused(q, P[1], P[2], P[3], gamma, ctypes.c_float(eps), gate, out, None, None,
                                            B, H, N, d, outd, 0, 0, flags, None, 0, None, None, None)

    assert call(q=None) == LA_ERR_INVALID
    assert call(eps=-1.0) == LA_ERR_INVALID
    assert call(eps=2.0) == LA_ERR_INVALID
    assert call(flags=8) == LA_ERR_INVALID
    assert call(gamma=ctypes.c_void_p(P[5].value + 4)) == LA_ERR_INVALID   # misaligned
    assert call(gate=P[4]) == LA_ERR_INVALID                               # gate overlapping the output
    assert call(gamma=ctypes.c_void_p(P[4].value + 64)) == LA_ERR_INVALID  # gamma inside the output
    assert call(d=96) == LA_ERR_UNSUPPORTED
    assert call(outd=7) == LA_ERR_INVALID


def test_binding_rejects_a_stream_of_another_device():
    """The binding launches on the tensors' device: a caller's stream on
    another device is refused before the library is called."""
    import torch

    class _Stream:
        device = torch.device("cuda", 1)
        cuda_stream = 0

    with pytest.raises(ValueError, match="stream is on"):
        la._stream(_Stream(), torch.device("cuda", 0))
    assert la._stream(_Stream(), torch.device("cuda", 1)).value is None  # same device: passed through


def test_written_buffers_apart_from_every_input(lib):
    """A buffer a call writes may overlap no other argument (bar the in-place
    state): each case is refused before any HIP call."""
    inside = lambda p, off=64: ctypes.c_void_p(p.value + off)
    # prefill: the final state inside q, k or v or on the decays; the output on the decays
    assert _fwd(lib, kv_out=inside(FAKE[0])) == LA_ERR_INVALID
    assert _fwd(lib, kv_out=inside(FAKE[2])) == LA_ERR_INVALID
    assert _fwd(lib, kv_out=FAKE[3]) == LA_ERR_INVALID
    assert _fwd(lib, out=FAKE[3]) == LA_ERR_INVALID
    # a caller's workspace over q, over the output, over the decays
    need = lib.lightning_attn_fwd_workspace_bytes(1, 2, 128, 64, 64)
    for target in (FAKE[0], FAKE[4], FAKE[3]):
        assert _fwd(lib, ws=target, wsb=need) == LA_ERR_INVALID
    # decode: the written state over q, the output over the decays
    dec = lib.lightning_attn_decode_step
    assert dec(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, inside(FAKE[0]), 1, 2, 64, None) == LA_ERR_INVALID
    assert dec(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[3], None, FAKE[5], 1, 2, 64, None) == LA_ERR_INVALID
    # a state pool over k
    slots = lib.lightning_attn_decode_slots
    assert slots(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], inside(FAKE[1]), FAKE[6], 1, 2, 64, 4, None) \
        == LA_ERR_INVALID
    # backward: a caller's workspace over dq, dk over the decays
    f = lib.lightning_attn_bwd
    base = [FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, None, FAKE[5], FAKE[6], FAKE[7], None,
            1, 1, 128, 128, 0, 0, 0, None, 0, None]
    a = list(base)
    a[18], a[19] = FAKE[5], lib.lightning_attn_bwd_workspace_bytes(1, 1, 128, 128)
    assert f(*a) == LA_ERR_INVALID
    a = list(base)
    a[8] = FAKE[3]
    assert f(*a) == LA_ERR_INVALID
