"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

import decode_attention_paged_append_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIBRARY_PATH):
        pytest.fail("libpagedattn.so not built (python -m decode_attention_paged_append_amd.build)")
    return pa.library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.pa_abi_version() == int(re.search(r"PA_ABI_VERSION (\d+)", open(HEADER).read())[1])
    assert lib.pa_status_string(WORKSPACE) == b"workspace too small"


def desc(nb=64, hkv=2, bs=16, d=128, dtype=1):
    return pa.CacheDesc(nb, hkv, bs, d, dtype)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


def test_append_argument_checks(lib):
    d = desc()
    assert lib.pa_kv_append(FAKE, FAKE, FAKE, 4, FAKE, FAKE, None, None) == INVALID
    assert lib.pa_kv_append(FAKE, FAKE, FAKE, -1, FAKE, FAKE, ctypes.byref(d), None) == INVALID
    assert lib.pa_kv_append(FAKE, None, FAKE, 4, FAKE, FAKE, ctypes.byref(d), None) == INVALID
    assert lib.pa_kv_append(None, None, None, 0, None, None, ctypes.byref(d), None) == OK
    bad = desc(d=96)
    assert lib.pa_kv_append(FAKE, FAKE, FAKE, 4, FAKE, FAKE, ctypes.byref(bad), None) == UNSUPPORTED
    assert b"head_dim 96" in lib.pa_last_error()
    bad = desc(bs=12)
    assert lib.pa_kv_append(FAKE, FAKE, FAKE, 4, FAKE, FAKE, ctypes.byref(bad), None) == UNSUPPORTED
    i8 = desc(dtype=3)
    assert lib.pa_kv_append(FAKE, FAKE, FAKE, 4, FAKE, FAKE, ctypes.byref(i8), None) == UNSUPPORTED
    assert lib.pa_kv_append_int8(FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d),
                                 None) == UNSUPPORTED
    assert lib.pa_kv_append_int8(FAKE, FAKE, FAKE, 4, FAKE, FAKE, None, FAKE, ctypes.byref(i8),
                                 None) == INVALID
    fp8 = desc(dtype=4)
    assert lib.pa_kv_append(FAKE, FAKE, FAKE, 4, FAKE, FAKE, ctypes.byref(fp8), None) == UNSUPPORTED
    assert lib.pa_kv_append_fp8(FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d),
                                None) == UNSUPPORTED
    assert b"fp8 cache" in lib.pa_last_error()
    assert lib.pa_kv_append_fp8(FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, ctypes.byref(i8),
                                None) == UNSUPPORTED
    assert lib.pa_kv_append_int8(FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, ctypes.byref(fp8),
                                 None) == UNSUPPORTED
    assert lib.pa_kv_append_fp8(FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None, ctypes.byref(fp8),
                                None) == INVALID


def test_check_slot_mapping_argument_checks(lib):
    """Host-side checks of the slot check, before any launch."""
    flags = ctypes.c_void_p(0x2000)
    assert lib.pa_check_slot_mapping(FAKE, -1, 64, flags, None) == INVALID
    assert lib.pa_check_slot_mapping(FAKE, 4, 0, flags, None) == INVALID
    assert lib.pa_check_slot_mapping(FAKE, 4, 64, None, None) == INVALID
    assert lib.pa_check_slot_mapping(None, 4, 64, flags, None) == INVALID
    assert lib.pa_check_slot_mapping(FAKE, 4, 64, ctypes.c_void_p(0x2002), None) == INVALID
    assert b"aligned" in lib.pa_last_error()


def test_copy_blocks_argument_checks(lib):
    """Quantized pools need both scale pointers; a negative count is rejected
    and an empty one is a no-op (all on the host, before any launch)."""
    i8 = desc(dtype=3)
    assert lib.pa_copy_blocks(FAKE, FAKE, None, FAKE, FAKE, 1, ctypes.byref(i8), None) == INVALID
    assert b"NULL" in lib.pa_last_error()
    assert lib.pa_copy_blocks(FAKE, FAKE, FAKE, None, FAKE, 1, ctypes.byref(i8), None) == INVALID
    assert lib.pa_copy_blocks(FAKE, FAKE, None, None, FAKE, -1, ctypes.byref(desc()),
                              None) == INVALID
    assert lib.pa_copy_blocks(None, None, None, None, None, 0, ctypes.byref(desc()), None) == OK


def test_decode_argument_checks(lib):
    d = desc()
    call = lambda hq, ws, wsb, desc_=d, s=4, maxb=16: lib.pa_paged_decode_attention(
        FAKE, FAKE, FAKE, FAKE, maxb, FAKE, s, hq, 0.1, FAKE, ctypes.byref(desc_), ws, wsb, None)
    assert call(3, FAKE, 1 << 30) == INVALID            # 3 query heads over 2 KV heads
    assert call(0, FAKE, 1 << 30) == INVALID
    assert call(4, FAKE, 1 << 30, s=-1) == INVALID
    assert call(4, FAKE, 1 << 30, maxb=0) == INVALID
    assert call(4, FAKE, 1 << 30, desc_=desc(dtype=3)) == UNSUPPORTED  # int8 needs its entry
    assert call(4, FAKE, 1 << 30, desc_=desc(dtype=7)) == UNSUPPORTED
    assert call(4, FAKE, 1 << 30, desc_=desc(dtype=4)) == UNSUPPORTED  # fp8 needs its entry
    assert b"pa_paged_decode_attention_fp8" in lib.pa_last_error()
    fp8 = desc(dtype=4)
    i8 = desc(dtype=3)
    assert lib.pa_paged_decode_attention_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 4,
                                             0.1, FAKE, ctypes.byref(i8), FAKE, 1 << 30,
                                             None) == UNSUPPORTED
    assert lib.pa_paged_decode_attention_int8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 4,
                                              0.1, FAKE, ctypes.byref(fp8), FAKE, 1 << 30,
                                              None) == UNSUPPORTED
    assert lib.pa_paged_decode_attention_fp8(FAKE, FAKE, FAKE, None, FAKE, FAKE, 16, FAKE, 4, 4,
                                             0.1, FAKE, ctypes.byref(fp8), FAKE, 1 << 30,
                                             None) == INVALID
    need = lib.pa_decode_workspace_bytes(ctypes.byref(d), 4, 4, 16, 64)
    assert need > 0
    assert lib.pa_decode_partitions(FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE, 4, 4, 0.1, 64,
                                    FAKE, ctypes.byref(d), FAKE, need - 1, None) == WORKSPACE
    assert lib.pa_decode_partitions(FAKE, FAKE, FAKE, None, None, FAKE, 16, FAKE, 4, 4, 0.1, 24,
                                    FAKE, ctypes.byref(d), FAKE, need, None) == INVALID
    assert b"multiple of the tile" in lib.pa_last_error()
    assert call(4, None, 0, s=0) == OK                  # nothing to do
    assert lib.pa_lse_merge(FAKE, 0, FAKE, 4, 4, 128, 16, 16, 64, 1, FAKE, None) == WORKSPACE
    assert lib.pa_lse_merge(FAKE, 1 << 30, FAKE, 4, 4, 128, 16, 16, 256, 1, FAKE, None) == INVALID
    assert lib.pa_lse_merge(FAKE, 1 << 30, FAKE, 4, 4, 128, 16, 16, 64, 3, FAKE, None) == UNSUPPORTED


def test_decode_step_quant_argument_checks(lib):
    """pa_decode_step_quant / _partitions_quant: quantized caches only, both
    new rows and both scale arrays, workspace and partition checks; the
    16-bit step entry points point quantized caches to them."""
    f16, i8, fp8, i4 = desc(), desc(dtype=3), desc(dtype=4), desc(dtype=5)
    step = lambda d_, kn=FAKE, ks=FAKE, s=4, ws=FAKE, wsb=1 << 30: lib.pa_decode_step_quant(
        FAKE, kn, FAKE, FAKE, FAKE, ks, FAKE, FAKE, 16, FAKE, s, 4, 0.1, FAKE, ctypes.byref(d_),
        ws, wsb, None)
    assert step(f16) == UNSUPPORTED
    assert b"int8, fp8 or int4" in lib.pa_last_error()
    for d_ in (i8, fp8, i4):
        assert step(d_, kn=None) == INVALID
        assert step(d_, ks=None) == INVALID
        assert b"k_scale" in lib.pa_last_error()
        assert step(d_, kn=None, ks=None, s=0, ws=None, wsb=0) == OK   # nothing to do
    part = lambda d_, pt, wsb, kn=FAKE: lib.pa_decode_step_partitions_quant(
        FAKE, kn, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 4, 0.1, pt, FAKE,
        ctypes.byref(d_), FAKE, wsb, None)
    need = lib.pa_decode_workspace_bytes(ctypes.byref(i8), 4, 4, 16, 64)
    assert need > 0
    assert part(i8, 64, need - 1) == WORKSPACE
    assert part(i8, 24, need) == INVALID
    assert b"multiple of the tile" in lib.pa_last_error()
    assert part(i8, 64, need, kn=None) == INVALID
    assert part(f16, 64, need) == UNSUPPORTED
    # the 16-bit step entry points name the quantized ones
    assert lib.pa_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 4, 0.1, FAKE,
                              ctypes.byref(i8), FAKE, 1 << 30, None) == UNSUPPORTED
    assert b"pa_decode_step_quant" in lib.pa_last_error()
    assert lib.pa_decode_step_partitions(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 4, 0.1,
                                         64, FAKE, ctypes.byref(fp8), FAKE, 1 << 30,
                                         None) == UNSUPPORTED
    assert b"pa_decode_step_partitions_quant" in lib.pa_last_error()


def test_decode_step_window_argument_checks(lib):
    """pa_decode_step_window: both new rows, a non-negative window, scales for
    quantized caches, the window workspace; nothing to do at S = 0."""
    f16, i8 = desc(), desc(dtype=3)
    step = lambda d_, kn=FAKE, ks=FAKE, w=2048, s=4, ws=FAKE, wsb=1 << 30: \
        lib.pa_decode_step_window(FAKE, kn, FAKE, FAKE, FAKE, ks, FAKE, FAKE, 256, FAKE, s, 4,
                                  0.1, w, FAKE, ctypes.byref(d_), ws, wsb, None)
    assert step(f16, kn=None) == INVALID
    assert step(f16, w=-1) == INVALID
    assert b"window" in lib.pa_last_error()
    assert step(i8, ks=None) == INVALID
    need = lib.pa_decode_window_workspace_bytes(ctypes.byref(f16), 4, 4, 256, 2048)
    assert need > 0
    assert step(f16, wsb=need - 1) == WORKSPACE
    assert step(f16, kn=None, s=0, ws=None, wsb=0) == OK


@pytest.mark.parametrize("dtype,d,bs,tile", [(0, 64, 4, 4), (1, 128, 16, 16), (1, 64, 4, 8),
                                              (3, 64, 4, 16), (3, 128, 32, 32), (0, 128, 8, 8),
                                              (4, 64, 4, 16), (4, 128, 16, 16)])
def test_workspace_and_plan(lib, dtype, d, bs, tile):
    dd = desc(nb=4096, hkv=8, bs=bs, d=d, dtype=dtype)
    s, hq, maxb = 16, 32, 4096 // bs
    part = lib.pa_decode_partition_tokens(ctypes.byref(dd), s, hq, maxb)
    assert part > 0 and part % tile == 0 and part % bs == 0
    nparts = -(-maxb * bs // part)
    ws = lib.pa_decode_workspace_bytes(ctypes.byref(dd), s, hq, maxb, 0)
    if nparts == 1:
        assert ws == 0
    else:
        a256 = lambda x: (x + 255) // 256 * 256
        ml = s * hq * nparts * 2 * 4
        assert ws == a256(ml) + s * hq * nparts * d * 4
    # an explicit partition covering the whole table needs no workspace
    assert lib.pa_decode_workspace_bytes(ctypes.byref(dd), s, hq, maxb, maxb * bs) == 0


def test_read_probe_argument_checks(lib):
    """Rejected on the host: NULL src or sink, a size that is zero or not a
    multiple of 4096, a source that is not 16-byte aligned (the pointers here
    are never dereferenced)."""
    src, sink = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    assert lib.pa_hbm_read_probe(None, 4096, None, sink, None) == INVALID
    assert lib.pa_hbm_read_probe(src, 4096, None, None, None) == INVALID
    assert lib.pa_hbm_read_probe(src, 0, None, sink, None) == INVALID
    assert lib.pa_hbm_read_probe(src, 4112, None, sink, None) == INVALID
    assert lib.pa_hbm_read_probe(ctypes.c_void_p(4104), 8192, None, sink, None) == INVALID
    assert b"multiple of 4096" in lib.pa_last_error()


def test_prefill_argument_checks_on_host(lib):
    """Prefill rejects bad shapes before any launch: a non-16-bit cache, a
    non-positive scale, heads that do not divide, and a chunk whose query
    rows need more than 65535 row tiles of the grid."""
    d = desc(hkv=2)
    call = lambda maxq, hq=16, scale=0.1, desc_=d: lib.pa_paged_prefill_attention(
        FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE, 4, maxq, hq, scale, FAKE, ctypes.byref(desc_),
        None)
    assert call(8, desc_=desc(dtype=0)) == UNSUPPORTED          # fp32 cache
    assert call(8, scale=0.0) == INVALID
    assert call(8, hq=3) == INVALID
    assert call(0) == OK                                         # nothing to do
    assert call(1 << 24) == UNSUPPORTED                          # 2^27 rows: 524288 tiles
    assert b"65535" in lib.pa_last_error()
