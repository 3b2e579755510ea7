"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

Python binding of ``libpagedattn.so`` (the C ABI in ``include/pagedattn.h``).
Each function here carries the C entry point's name without its ``pa_``
prefix and only marshals arguments: it checks that torch tensors are on the
GPU, contiguous and of the right type, then passes their device pointers and
torch's current HIP stream to the library.  Every step of the computation
runs in the library's HIP kernels; there is no CPU fallback -- importing
works without the library, but any call raises if it is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "PagedAttnError", "library", "CacheDesc", "slot_mapping", "decode_slot_mapping",
    "kv_append", "kv_append_int8", "check_slot_mapping", "SLOT_REPEATED", "SLOT_OUTSIDE_POOL", "decode_workspace_bytes", "decode_partition_tokens",
    "paged_decode_attention", "paged_decode_attention_int8", "decode_step", "decode_partitions",
    "kv_append_fp8", "paged_decode_attention_fp8", "kv_append_int4",
    "paged_decode_attention_int4", "int4_desc",
    "decode_step_partitions", "decode_step_quant", "decode_step_partitions_quant", "lse_merge", "gather_kv", "abi_version", "OutOfBlocks",
    "hbm_read_probe",
    "BlockManager", "copy_blocks", "paged_prefill_attention", "paged_decode_attention_window",
    "decode_window_workspace_bytes", "decode_step_window", "decode_step_noalloc",
]

# PA_LIBRARY_PATH may name another build of the same library (e.g. a variant
# under test); by default the in-tree build next to this file is loaded.
LIBRARY_PATH = os.environ.get(
    "PA_LIBRARY_PATH",
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so"))
# fp8 caches hold OCP E4M3 codes (torch.float8_e4m3fn storage).
DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.int8: 3,
              torch.float8_e4m3fn: 4}
QUANTIZED = (torch.int8, torch.float8_e4m3fn)
CODE_DTYPE = {v: k for k, v in DTYPE_CODE.items()}


class PagedAttnError(RuntimeError):
    """A non-OK status from the library."""


class OutOfBlocks(PagedAttnError):
    """The block pool cannot hold the request (PA_ERR_OUT_OF_BLOCKS)."""


OUT_OF_BLOCKS = 5


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]

    @classmethod
    def of(cls, k_cache: torch.Tensor) -> "CacheDesc":
        nb, hkv, bs, d = k_cache.shape
        return cls(nb, hkv, bs, d, DTYPE_CODE[k_cache.dtype])


_lib = None


def library() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY_PATH):
            raise PagedAttnError(
                f"{LIBRARY_PATH} is missing: build it with "
                "`python -m decode_attention_paged_append_amd.build`")
        _lib = _declare(ctypes.CDLL(LIBRARY_PATH))
    return _lib


def _declare(lib):
    P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    D = ctypes.POINTER(CacheDesc)
    sig = {
        "pa_slot_mapping": [P, i32, i32, P, P, i64, i32, P, P],
        "pa_decode_slot_mapping": [P, i32, P, i32, i32, P, P],
        "pa_kv_append": [P, P, P, i64, P, P, D, P],
        "pa_check_slot_mapping": [P, i64, i64, P, P],
        "pa_kv_append_int8": [P, P, P, i64, P, P, P, P, D, P],
        "pa_kv_append_fp8": [P, P, P, i64, P, P, P, P, D, P],
        "pa_kv_append_int4": [P, P, P, i64, P, P, P, P, D, P],
        "pa_paged_decode_attention": [P, P, P, P, i32, P, i32, i32, f32, P, D, P, sz, P],
        "pa_paged_decode_attention_int8": [P, P, P, P, P, P, i32, P, i32, i32, f32, P, D, P, sz, P],
        "pa_paged_decode_attention_fp8": [P, P, P, P, P, P, i32, P, i32, i32, f32, P, D, P, sz, P],
        "pa_paged_decode_attention_int4": [P, P, P, P, P, P, i32, P, i32, i32, f32, P, D, P, sz, P],
        "pa_decode_partitions": [P, P, P, P, P, P, i32, P, i32, i32, f32, i32, P, D, P, sz, P],
        "pa_lse_merge": [P, sz, P, i32, i32, i32, i32, i32, i32, i32, P, P],
        "pa_decode_step": [P, P, P, P, P, P, i32, P, i32, i32, f32, P, D, P, sz, P],
        "pa_decode_step_partitions": [P, P, P, P, P, P, i32, P, i32, i32, f32, i32, P, D, P, sz,
                                      P],
        "pa_decode_step_noalloc": [P, P, P, P, P, P, i32, P, i32, i32, f32, P, D, P],
        "pa_decode_step_quant": [P, P, P, P, P, P, P, P, i32, P, i32, i32, f32, P, D, P, sz, P],
        "pa_decode_step_partitions_quant": [P, P, P, P, P, P, P, P, i32, P, i32, i32, f32, i32, P,
                                            D, P, sz, P],
        "pa_gather_kv": [P, P, P, P, P, i32, P, i32, P, P, P, P, D, P],
        "pa_copy_blocks": [P, P, P, P, P, i32, D, P],
        "pa_hbm_read_probe": [P, sz, P, P, P],
        "pa_paged_prefill_attention": [P, P, P, P, i32, P, P, i32, i32, i32, f32, P, D, P],
        "pa_paged_decode_attention_window": [P, P, P, P, P, P, i32, P, i32, i32, f32, i32, P, D,
                                             P, sz, P],
        "pa_decode_step_window": [P, P, P, P, P, P, P, P, i32, P, i32, i32, f32, i32, P, D, P,
                                  sz, P],
        "pa_bm_create": [i32, i32, ctypes.POINTER(P)],
        "pa_bm_add_sequence": [P, ctypes.POINTER(i32)],
        "pa_bm_fork": [P, i32, i32, ctypes.POINTER(i32)],
        "pa_bm_free_sequence": [P, i32],
        "pa_bm_append": [P, P, P, i32, P, i64, P, i32, ctypes.POINTER(i32)],
        "pa_bm_block_tables": [P, P, i32, i32, P, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.pa_decode_workspace_bytes.argtypes = [D, i32, i32, i32, i32]
    lib.pa_decode_workspace_bytes.restype = sz
    lib.pa_decode_window_workspace_bytes.argtypes = [D, i32, i32, i32, i32]
    lib.pa_decode_window_workspace_bytes.restype = sz
    lib.pa_decode_partition_tokens.argtypes = [D, i32, i32, i32]
    lib.pa_decode_partition_tokens.restype = i32
    lib.pa_bm_destroy.argtypes = [P]
    lib.pa_bm_destroy.restype = None
    for name, args in (("pa_bm_num_free_blocks", [P]), ("pa_bm_ref_count", [P, i32]),
                       ("pa_bm_sequence_length", [P, i32])):
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = i32
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_abi_version.restype = i32
    return lib


def _ok(status: int, lib) -> None:
    if status != 0:
        cls = OutOfBlocks if status == OUT_OF_BLOCKS else PagedAttnError
        raise cls(f"{lib.pa_status_string(status).decode()}: "
                             f"{lib.pa_last_error().decode()}")


def _dev(t: torch.Tensor | None, name: str, dtype=None, ndim=None):
    """Device pointer of a contiguous GPU tensor (None stays NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _nbytes(t: torch.Tensor | None) -> int:
    """Size in bytes of a workspace tensor of any dtype (0 for None)."""
    return 0 if t is None else t.numel() * t.element_size()


def _check_pools(k_cache, v_cache, k_scale=None, v_scale=None, int4=False):
    """The V pool must be the K pool's twin (shape and dtype), since the
    library sizes both from one descriptor; a quantized cache (int8, fp8,
    int4) needs fp16 scales [NB, Hkv, BS] (int4: [NB, Hkv, BS, D/32]) for
    both pools.  Raises ValueError before anything reaches the GPU."""
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache must be [NB, Hkv, BS, D], got {tuple(k_cache.shape)}")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError(f"v_cache {tuple(v_cache.shape)} {v_cache.dtype} must match k_cache "
                         f"{tuple(k_cache.shape)} {k_cache.dtype}")
    if int4 or k_cache.dtype in QUANTIZED:
        want = tuple(k_cache.shape[:3]) + ((2 * k_cache.shape[3] // INT4_GROUP,) if int4 else ())
        for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            if sc is None:
                raise ValueError(f"a quantized cache needs {name}")
            if tuple(sc.shape) != want or sc.dtype != torch.float16:
                raise ValueError(f"{name} must be float16 {want}, got {sc.dtype} "
                                 f"{tuple(sc.shape)}")


def abi_version() -> int:
    return library().pa_abi_version()


# ---------------------------------------------------------------- slots

def slot_mapping(block_tables, token_seq, token_pos, block_size, out=None):
    """int64 slot of each (sequence, position) pair; see pa_slot_mapping."""
    lib = library()
    n = token_seq.numel()
    out = torch.empty(n, dtype=torch.int64, device=block_tables.device) if out is None else out
    _ok(lib.pa_slot_mapping(_dev(block_tables, "block_tables", torch.int32, 2),
                            block_tables.shape[1], block_tables.shape[0],
                            _dev(token_seq, "token_seq", torch.int32),
                            _dev(token_pos, "token_pos", torch.int32), n, block_size,
                            _dev(out, "slot_mapping", torch.int64), _stream(block_tables)), lib)
    return out


def decode_slot_mapping(block_tables, context_lens, block_size, out=None):
    """Slot of each sequence's newest position context_lens[s]-1 (-1 if empty)."""
    lib = library()
    s = context_lens.numel()
    out = torch.empty(s, dtype=torch.int64, device=block_tables.device) if out is None else out
    _ok(lib.pa_decode_slot_mapping(_dev(block_tables, "block_tables", torch.int32, 2),
                                   block_tables.shape[1],
                                   _dev(context_lens, "context_lens", torch.int32), s, block_size,
                                   _dev(out, "slot_mapping", torch.int64),
                                   _stream(block_tables)), lib)
    return out


SLOT_REPEATED, SLOT_OUTSIDE_POOL = 1, 2


def check_slot_mapping(slot_mapping, pool_slots, flags=None):
    """Device int32 [1] flags of a slot mapping (see pa_check_slot_mapping):
    SLOT_REPEATED if some slot >= 0 repeats, | SLOT_OUTSIDE_POOL if some slot
    is >= pool_slots; 0 when the mapping is fit for one append.  Nothing is
    synchronized: read the flags when convenient."""
    lib = library()
    if flags is None:
        flags = torch.empty(1, dtype=torch.int32, device=slot_mapping.device)
    _ok(lib.pa_check_slot_mapping(_dev(slot_mapping, "slot_mapping", torch.int64),
                                  slot_mapping.numel(), int(pool_slots),
                                  _dev(flags, "flags", torch.int32), _stream(slot_mapping)), lib)
    return flags


# ---------------------------------------------------------------- append

def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache):
    """Scatter k_new/v_new [T, Hkv, D] into the [NB, Hkv, BS, D] pools."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    _check_pools(k_cache, v_cache)
    t = slot_mapping.numel()
    if k_new.shape != (t, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{t}, {desc.num_kv_heads}, {desc.head_dim}]")
    _ok(lib.pa_kv_append(_dev(k_new, "k_new", k_cache.dtype), _dev(v_new, "v_new", k_cache.dtype),
                         _dev(slot_mapping, "slot_mapping", torch.int64), t,
                         _dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", ndim=4),
                         ctypes.byref(desc), _stream(k_cache)), lib)


def kv_append_int8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """Quantize fp16 rows [T, Hkv, D] and store codes + fp16 scales."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    t = slot_mapping.numel()
    if k_new.shape != (t, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{t}, {desc.num_kv_heads}, {desc.head_dim}]")
    _check_pools(k_cache, v_cache, k_scale, v_scale)
    _ok(lib.pa_kv_append_int8(_dev(k_new, "k_new", torch.float16), _dev(v_new, "v_new", torch.float16),
                              _dev(slot_mapping, "slot_mapping", torch.int64), t,
                              _dev(k_cache, "k_cache", torch.int8, 4),
                              _dev(v_cache, "v_cache", torch.int8, 4),
                              _dev(k_scale, "k_scale", torch.float16),
                              _dev(v_scale, "v_scale", torch.float16), ctypes.byref(desc),
                              _stream(k_cache)), lib)


INT4 = 5        # pa_dtype of an int4 cache
INT4_GROUP = 32


def int4_desc(k_cache) -> CacheDesc:
    """Descriptor of an int4 pool held as uint8 [NB, Hkv, BS, D/2] (two codes
    per byte; torch has no 4-bit type)."""
    if k_cache.dtype != torch.uint8 or k_cache.dim() != 4:
        raise ValueError("an int4 pool is a uint8 tensor [NB, Hkv, BS, D/2]")
    nb, hkv, bs, half = k_cache.shape
    return CacheDesc(nb, hkv, bs, 2 * half, INT4)


def kv_append_int4(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """Quantize fp16 rows [T, Hkv, D] to int4 codes (uint8 pools [NB, Hkv, BS,
    D/2]) with fp16 scales per 32 dims ([NB, Hkv, BS, D/32])."""
    lib = library()
    desc = int4_desc(k_cache)
    t = slot_mapping.numel()
    if k_new.shape != (t, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{t}, {desc.num_kv_heads}, {desc.head_dim}]")
    _check_pools(k_cache, v_cache, k_scale, v_scale, int4=True)
    _ok(lib.pa_kv_append_int4(_dev(k_new, "k_new", torch.float16), _dev(v_new, "v_new", torch.float16),
                              _dev(slot_mapping, "slot_mapping", torch.int64), t,
                              _dev(k_cache, "k_cache", torch.uint8, 4),
                              _dev(v_cache, "v_cache", torch.uint8, 4),
                              _dev(k_scale, "k_scale", torch.float16),
                              _dev(v_scale, "v_scale", torch.float16), ctypes.byref(desc),
                              _stream(k_cache)), lib)


def kv_append_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """Quantize fp16 rows [T, Hkv, D] to fp8 E4M3 codes + fp16 scales."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    t = slot_mapping.numel()
    if k_new.shape != (t, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{t}, {desc.num_kv_heads}, {desc.head_dim}]")
    _check_pools(k_cache, v_cache, k_scale, v_scale)
    e4m3 = torch.float8_e4m3fn
    _ok(lib.pa_kv_append_fp8(_dev(k_new, "k_new", torch.float16), _dev(v_new, "v_new", torch.float16),
                             _dev(slot_mapping, "slot_mapping", torch.int64), t,
                             _dev(k_cache, "k_cache", e4m3, 4), _dev(v_cache, "v_cache", e4m3, 4),
                             _dev(k_scale, "k_scale", torch.float16),
                             _dev(v_scale, "v_scale", torch.float16), ctypes.byref(desc),
                             _stream(k_cache)), lib)


# ---------------------------------------------------------------- attention

def decode_workspace_bytes(k_cache, num_seqs, num_q_heads, max_blocks, partition_tokens=0) -> int:
    desc = k_cache if isinstance(k_cache, CacheDesc) else CacheDesc.of(k_cache)
    return int(library().pa_decode_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads,
                                                   max_blocks, partition_tokens))


def decode_partition_tokens(k_cache, num_seqs, num_q_heads, max_blocks) -> int:
    desc = k_cache if isinstance(k_cache, CacheDesc) else CacheDesc.of(k_cache)
    return int(library().pa_decode_partition_tokens(ctypes.byref(desc), num_seqs, num_q_heads,
                                                    max_blocks))


def _workspace(ws, nbytes, device):
    """The caller's workspace, or a new one of the size the plan needs."""
    if ws is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return ws


def _shapes(q, k_cache, v_cache, block_tables, context_lens, out, int4=False, k_scale=None,
            v_scale=None):
    """(S, Hq, max_blocks) of a decode call, after checking the pools
    (_check_pools), q / out / table / length shapes and head_dim."""
    _check_pools(k_cache, v_cache, k_scale, v_scale, int4)
    if q.dim() != 3:
        raise ValueError(f"q must be [S, Hq, D], got {tuple(q.shape)}")
    s, hq, d = q.shape
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or context_lens.numel() != s:
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    if k_cache.shape[3] * (2 if int4 else 1) != d:
        raise ValueError("head_dim of q and cache differ")
    return s, hq, block_tables.shape[1]


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                           workspace=None):
    """out[s,h] = softmax(q[s,h] . K_s^T * scale) . V_s over the paged cache."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out)
    need = decode_workspace_bytes(desc, s, hq, maxb)
    ws = _workspace(workspace, need, q.device)
    _ok(lib.pa_paged_decode_attention(
        _dev(q, "q", k_cache.dtype, 3), _dev(k_cache, "k_cache", ndim=4),
        _dev(v_cache, "v_cache", k_cache.dtype, 4), _dev(block_tables, "block_tables", torch.int32),
        maxb, _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale),
        _dev(out, "out", k_cache.dtype), ctypes.byref(desc), _dev(ws, "workspace"), _nbytes(ws),
        _stream(q)), lib)
    return out


def paged_decode_attention_int8(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                context_lens, scale, out, workspace=None):
    """Decode attention over an int8 cache with fp16 per-(token, head) scales."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out, False, k_scale,
                          v_scale)
    need = decode_workspace_bytes(desc, s, hq, maxb)
    ws = _workspace(workspace, need, q.device)
    _ok(lib.pa_paged_decode_attention_int8(
        _dev(q, "q", torch.float16, 3), _dev(k_cache, "k_cache", torch.int8, 4),
        _dev(v_cache, "v_cache", torch.int8, 4), _dev(k_scale, "k_scale", torch.float16),
        _dev(v_scale, "v_scale", torch.float16), _dev(block_tables, "block_tables", torch.int32),
        maxb, _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale),
        _dev(out, "out", torch.float16), ctypes.byref(desc), _dev(ws, "workspace"), _nbytes(ws),
        _stream(q)), lib)
    return out


def paged_decode_attention_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                               context_lens, scale, out, workspace=None):
    """Decode attention over an fp8 (E4M3) cache with fp16 per-(token, head) scales."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out, False, k_scale,
                          v_scale)
    need = decode_workspace_bytes(desc, s, hq, maxb)
    ws = _workspace(workspace, need, q.device)
    e4m3 = torch.float8_e4m3fn
    _ok(lib.pa_paged_decode_attention_fp8(
        _dev(q, "q", torch.float16, 3), _dev(k_cache, "k_cache", e4m3, 4),
        _dev(v_cache, "v_cache", e4m3, 4), _dev(k_scale, "k_scale", torch.float16),
        _dev(v_scale, "v_scale", torch.float16), _dev(block_tables, "block_tables", torch.int32),
        maxb, _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale),
        _dev(out, "out", torch.float16), ctypes.byref(desc), _dev(ws, "workspace"), _nbytes(ws),
        _stream(q)), lib)
    return out


def paged_decode_attention_int4(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                context_lens, scale, out, workspace=None):
    """Decode attention over an int4 cache (uint8 pools [NB, Hkv, BS, D/2],
    fp16 scales [NB, Hkv, BS, D/32])."""
    lib = library()
    desc = int4_desc(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out, True, k_scale,
                          v_scale)
    need = decode_workspace_bytes(desc, s, hq, maxb)
    ws = _workspace(workspace, need, q.device)
    _ok(lib.pa_paged_decode_attention_int4(
        _dev(q, "q", torch.float16, 3), _dev(k_cache, "k_cache", torch.uint8, 4),
        _dev(v_cache, "v_cache", torch.uint8, 4), _dev(k_scale, "k_scale", torch.float16),
        _dev(v_scale, "v_scale", torch.float16), _dev(block_tables, "block_tables", torch.int32),
        maxb, _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale),
        _dev(out, "out", torch.float16), ctypes.byref(desc), _dev(ws, "workspace"), _nbytes(ws),
        _stream(q)), lib)
    return out


def decode_step(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
                workspace=None):
    """One decode step: store each sequence's k_new/v_new [S, Hkv, D] rows at
    position context_lens[s]-1 inside the attention launch and attend over
    all context_lens[s] rows (see pa_decode_step)."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out)
    if k_new.shape != (s, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{s}, {desc.num_kv_heads}, {desc.head_dim}]")
    need = decode_workspace_bytes(desc, s, hq, maxb)
    ws = _workspace(workspace, need, q.device)
    _ok(lib.pa_decode_step(
        _dev(q, "q", k_cache.dtype, 3), _dev(k_new, "k_new", k_cache.dtype),
        _dev(v_new, "v_new", k_cache.dtype), _dev(k_cache, "k_cache", ndim=4),
        _dev(v_cache, "v_cache", k_cache.dtype, 4), _dev(block_tables, "block_tables", torch.int32),
        maxb, _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale),
        _dev(out, "out", k_cache.dtype), ctypes.byref(desc), _dev(ws, "workspace"), _nbytes(ws),
        _stream(q)), lib)
    return out


def decode_step_noalloc(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                        out):
    """decode_step with no workspace: the partials go to the library's
    static device scratch (see pa_decode_step_noalloc), so the call
    allocates nothing; calls that overlap on one device race."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out)
    if k_new.shape != (s, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{s}, {desc.num_kv_heads}, {desc.head_dim}]")
    _ok(lib.pa_decode_step_noalloc(
        _dev(q, "q", k_cache.dtype, 3), _dev(k_new, "k_new", k_cache.dtype),
        _dev(v_new, "v_new", k_cache.dtype), _dev(k_cache, "k_cache", ndim=4),
        _dev(v_cache, "v_cache", k_cache.dtype, 4), _dev(block_tables, "block_tables", torch.int32),
        maxb, _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale),
        _dev(out, "out", k_cache.dtype), ctypes.byref(desc), _stream(q)), lib)
    return out


def decode_partitions(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                      partition_tokens, workspace, k_scale=None, v_scale=None, int4=False):
    """Phase 1 with an explicit partition length (see pa_decode_partitions);
    int4: uint8 pools [NB, Hkv, BS, D/2] hold int4 codes."""
    lib = library()
    desc = int4_desc(k_cache) if int4 else CacheDesc.of(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out, int4, k_scale,
                          v_scale)
    q_dtype = torch.float16 if int4 or k_cache.dtype in QUANTIZED else k_cache.dtype
    _ok(lib.pa_decode_partitions(
        _dev(q, "q", q_dtype, 3), _dev(k_cache, "k_cache", ndim=4),
        _dev(v_cache, "v_cache", k_cache.dtype, 4), _dev(k_scale, "k_scale", torch.float16),
        _dev(v_scale, "v_scale", torch.float16), _dev(block_tables, "block_tables", torch.int32),
        maxb, _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale),
        int(partition_tokens), _dev(out, "out", q_dtype), ctypes.byref(desc),
        _dev(workspace, "workspace"), _nbytes(workspace), _stream(q)),
        lib)
    return out


def decode_step_partitions(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                           out, partition_tokens, workspace):
    """Phase 1 of decode_step with an explicit partition length."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out)
    if k_new.shape != (s, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{s}, {desc.num_kv_heads}, {desc.head_dim}]")
    _ok(lib.pa_decode_step_partitions(
        _dev(q, "q", k_cache.dtype, 3), _dev(k_new, "k_new", k_cache.dtype),
        _dev(v_new, "v_new", k_cache.dtype), _dev(k_cache, "k_cache", ndim=4),
        _dev(v_cache, "v_cache", k_cache.dtype, 4), _dev(block_tables, "block_tables", torch.int32),
        maxb, _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale),
        int(partition_tokens), _dev(out, "out", k_cache.dtype), ctypes.byref(desc),
        _dev(workspace, "workspace"), _nbytes(workspace), _stream(q)),
        lib)
    return out


def _quant_step_args(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                     context_lens, out, int4):
    """Shared checks of the quantized decode-step calls: the cache descriptor,
    (S, Hq, max_blocks) and the marshalled tensor pointers up to context_lens."""
    desc = int4_desc(k_cache) if int4 else CacheDesc.of(k_cache)
    if desc.dtype not in (DTYPE_CODE[torch.int8], DTYPE_CODE[torch.float8_e4m3fn], INT4):
        raise ValueError("a quantized decode step needs an int8, fp8 or int4 cache")
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out, int4, k_scale,
                          v_scale)
    if k_new.shape != (s, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{s}, {desc.num_kv_heads}, {desc.head_dim}]")
    ptrs = (_dev(q, "q", torch.float16, 3), _dev(k_new, "k_new", torch.float16),
            _dev(v_new, "v_new", torch.float16), _dev(k_cache, "k_cache", ndim=4),
            _dev(v_cache, "v_cache", k_cache.dtype, 4), _dev(k_scale, "k_scale", torch.float16),
            _dev(v_scale, "v_scale", torch.float16),
            _dev(block_tables, "block_tables", torch.int32), maxb,
            _dev(context_lens, "context_lens", torch.int32), s, hq)
    return desc, s, hq, maxb, ptrs


def decode_step_quant(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                      context_lens, scale, out, workspace=None, int4=False):
    """One decode step over a quantized cache: quantize each sequence's fp16
    k_new/v_new [S, Hkv, D] rows into codes and scales at position
    context_lens[s]-1 inside the attention launch, then attend over all
    context_lens[s] rows (see pa_decode_step_quant).  int4: uint8 pools
    [NB, Hkv, BS, D/2] hold int4 codes."""
    lib = library()
    desc, s, hq, maxb, ptrs = _quant_step_args(q, k_new, v_new, k_cache, v_cache, k_scale,
                                               v_scale, block_tables, context_lens, out, int4)
    ws = _workspace(workspace, decode_workspace_bytes(desc, s, hq, maxb), q.device)
    _ok(lib.pa_decode_step_quant(*ptrs, float(scale), _dev(out, "out", torch.float16),
                                 ctypes.byref(desc), _dev(ws, "workspace"), _nbytes(ws),
                                 _stream(q)), lib)
    return out


def decode_step_partitions_quant(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                                 block_tables, context_lens, scale, out, partition_tokens,
                                 workspace, int4=False):
    """Phase 1 of decode_step_quant with an explicit partition length."""
    lib = library()
    desc, _, _, _, ptrs = _quant_step_args(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                                           block_tables, context_lens, out, int4)
    _ok(lib.pa_decode_step_partitions_quant(
        *ptrs, float(scale), int(partition_tokens), _dev(out, "out", torch.float16),
        ctypes.byref(desc), _dev(workspace, "workspace"), _nbytes(workspace), _stream(q)), lib)
    return out


def lse_merge(workspace, context_lens, num_q_heads, head_dim, max_blocks, block_size,
              partition_tokens, out):
    """Phase 2: merge the partials phase 1 left in the workspace into out."""
    lib = library()
    _ok(lib.pa_lse_merge(_dev(workspace, "workspace"), _nbytes(workspace),
                         _dev(context_lens, "context_lens", torch.int32), context_lens.numel(),
                         num_q_heads, head_dim, max_blocks, block_size, int(partition_tokens),
                         DTYPE_CODE[out.dtype], _dev(out, "out"), _stream(out)), lib)
    return out


# ---------------------------------------------------------------- gather

def gather_kv(k_cache, v_cache, block_tables, context_lens, k_out, v_out, k_scale=None,
              v_scale=None, k_scale_out=None, v_scale_out=None, int4=False):
    """Un-page to dense [S, max_blocks*BS, Hkv, D] (int4: packed [..., D/2]);
    rows past a length untouched."""
    lib = library()
    desc = int4_desc(k_cache) if int4 else CacheDesc.of(k_cache)
    _check_pools(k_cache, v_cache, k_scale, v_scale, int4)
    if block_tables.dim() != 2 or context_lens.numel() != block_tables.shape[0]:
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    s, maxb = block_tables.shape
    quant = int4 or k_cache.dtype in QUANTIZED
    if quant and (k_scale_out is None) != (v_scale_out is None):
        raise ValueError("k_scale_out and v_scale_out go together")
    if quant and k_scale_out is not None:
        swant = (s, maxb * desc.block_size, desc.num_kv_heads) + (
            (desc.head_dim // INT4_GROUP,) if int4 else ())
        for name, t in (("k_scale_out", k_scale_out), ("v_scale_out", v_scale_out)):
            if tuple(t.shape) != swant or t.dtype != torch.float16:
                raise ValueError(f"{name} must be float16 {swant}")
    want = (s, maxb * desc.block_size, desc.num_kv_heads, k_cache.shape[3])
    if tuple(k_out.shape) != want or tuple(v_out.shape) != want:
        raise ValueError(f"k_out/v_out must be {want}")
    _ok(lib.pa_gather_kv(_dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", k_cache.dtype, 4),
                         _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"),
                         _dev(block_tables, "block_tables", torch.int32), maxb,
                         _dev(context_lens, "context_lens", torch.int32), s,
                         _dev(k_out, "k_out", k_cache.dtype), _dev(v_out, "v_out", k_cache.dtype),
                         _dev(k_scale_out, "k_scale_out"), _dev(v_scale_out, "v_scale_out"),
                         ctypes.byref(desc), _stream(k_cache)), lib)


# ---------------------------------------------------------------- sliding window

def decode_window_workspace_bytes(k_cache, num_seqs, num_q_heads, max_blocks, window) -> int:
    desc = k_cache if isinstance(k_cache, CacheDesc) else CacheDesc.of(k_cache)
    return library().pa_decode_window_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads,
                                                      max_blocks, window)


def paged_decode_attention_window(q, k_cache, v_cache, block_tables, context_lens, scale, window,
                                  out, k_scale=None, v_scale=None, workspace=None, int4=False):
    """Decode attention over each sequence's last `window` positions (0: all);
    any cache format, scales for int8 / fp8 / int4 (see pa_paged_decode_attention_window)."""
    lib = library()
    desc = int4_desc(k_cache) if int4 else CacheDesc.of(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out, int4, k_scale,
                          v_scale)
    quant = int4 or k_cache.dtype in QUANTIZED
    q_dtype = torch.float16 if quant else k_cache.dtype
    need = decode_window_workspace_bytes(desc, s, hq, maxb, int(window))
    ws = _workspace(workspace, need, q.device)
    _ok(lib.pa_paged_decode_attention_window(
        _dev(q, "q", q_dtype, 3), _dev(k_cache, "k_cache", ndim=4),
        _dev(v_cache, "v_cache", k_cache.dtype, 4),
        _dev(k_scale, "k_scale", torch.float16) if quant else None,
        _dev(v_scale, "v_scale", torch.float16) if quant else None,
        _dev(block_tables, "block_tables", torch.int32), maxb,
        _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale), int(window),
        _dev(out, "out", q_dtype), ctypes.byref(desc), _dev(ws, "workspace"), _nbytes(ws),
        _stream(q)), lib)
    return out


def decode_step_window(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                       window, out, k_scale=None, v_scale=None, workspace=None, int4=False):
    """One decode step with a sliding window: store (or, for int8 / fp8 /
    int4 caches, quantize from fp16) each sequence's k_new/v_new [S, Hkv, D]
    rows at position context_lens[s]-1 inside the attention launch, then
    attend over the last `window` positions (see pa_decode_step_window)."""
    lib = library()
    desc = int4_desc(k_cache) if int4 else CacheDesc.of(k_cache)
    s, hq, maxb = _shapes(q, k_cache, v_cache, block_tables, context_lens, out, int4, k_scale,
                          v_scale)
    quant = int4 or k_cache.dtype in QUANTIZED
    q_dtype = torch.float16 if quant else k_cache.dtype
    if k_new.shape != (s, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{s}, {desc.num_kv_heads}, {desc.head_dim}]")
    need = decode_window_workspace_bytes(desc, s, hq, maxb, int(window))
    ws = _workspace(workspace, need, q.device)
    _ok(lib.pa_decode_step_window(
        _dev(q, "q", q_dtype, 3), _dev(k_new, "k_new", q_dtype), _dev(v_new, "v_new", q_dtype),
        _dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", k_cache.dtype, 4),
        _dev(k_scale, "k_scale", torch.float16) if quant else None,
        _dev(v_scale, "v_scale", torch.float16) if quant else None,
        _dev(block_tables, "block_tables", torch.int32), maxb,
        _dev(context_lens, "context_lens", torch.int32), s, hq, float(scale), int(window),
        _dev(out, "out", q_dtype), ctypes.byref(desc), _dev(ws, "workspace"), _nbytes(ws),
        _stream(q)), lib)
    return out


# ---------------------------------------------------------------- prefill

def paged_prefill_attention(q, k_cache, v_cache, block_tables, query_start, context_lens, scale,
                            out, max_query_len: int | None = None):
    """Causal attention of query chunks over the paged cache (prefill and
    chunked prefill; see pa_paged_prefill_attention).  q, out: [total, Hq, D];
    query_start: int32 [S+1] on the GPU; sequence s's query tokens are its
    last query_start[s+1]-query_start[s] cached positions.  max_query_len
    (the longest chunk) sizes the grid; when None it is read from
    query_start, which synchronizes."""
    lib = library()
    desc = CacheDesc.of(k_cache)
    _check_pools(k_cache, v_cache)
    if q.dtype != k_cache.dtype or out.dtype != q.dtype:
        raise ValueError("q, caches and out must share one format")
    s = block_tables.shape[0]
    if query_start.numel() != s + 1 or context_lens.numel() != s:
        raise ValueError("query_start must hold S+1 entries and context_lens S")
    if max_query_len is None:
        qs = query_start.cpu()
        max_query_len = int((qs[1:] - qs[:-1]).max()) if s else 0
    if q.shape != out.shape or q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q and out must be [total, Hq, D] alike")
    _ok(lib.pa_paged_prefill_attention(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32, 2), block_tables.shape[1],
        _dev(query_start, "query_start", torch.int32), _dev(context_lens, "context_lens",
                                                           torch.int32),
        s, int(max_query_len), q.shape[1], float(scale), _dev(out, "out"), ctypes.byref(desc),
        _stream(q)), lib)
    return out


# ---------------------------------------------------------------- block pool

def _host_i32(a, name):
    """A contiguous int32 host array and its address (ctypes.cast, which
    data_as uses, costs ~15 us a call; the plain address does not)."""
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data


class BlockManager:
    """The library's host-side block pool (pa_bm_*): block tables, context
    lengths and slots for the append and attention calls, with shared
    prefixes and copy-on-write.  Not thread-safe."""

    def __init__(self, num_blocks: int, block_size: int):
        lib = library()
        handle = ctypes.c_void_p()
        _ok(lib.pa_bm_create(num_blocks, block_size, ctypes.byref(handle)), lib)
        self._lib, self._h = lib, handle
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self) -> None:
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self) -> int:
        sid = ctypes.c_int32()
        _ok(self._lib.pa_bm_add_sequence(self._h, ctypes.byref(sid)), self._lib)
        return sid.value

    def fork(self, parent: int, prefix: int | None = None) -> int:
        sid = ctypes.c_int32()
        _ok(self._lib.pa_bm_fork(self._h, parent, -1 if prefix is None else prefix,
                                 ctypes.byref(sid)), self._lib)
        return sid.value

    def free(self, seq: int) -> None:
        _ok(self._lib.pa_bm_free_sequence(self._h, seq), self._lib)

    def append(self, requests):
        """requests: [(seq, n_tokens)].  Returns (slots int64 [sum n], copies
        int32 [k, 2] of (source, destination) blocks to copy first)."""
        return self.append_arrays([r[0] for r in requests], [r[1] for r in requests])

    def append_arrays(self, seqs, num_tokens):
        """append() with the requests as two int32 arrays (sequence ids and
        token counts)."""
        seqs, sp = _host_i32(seqs, "seqs")
        ntok, np_ = _host_i32(num_tokens, "num_tokens")
        total = int(ntok[ntok > 0].sum()) if ntok.size else 0
        slots = np.empty(max(total, 1), np.int64)
        copies = np.empty((max(seqs.size, 1), 2), np.int32)
        n = ctypes.c_int32()
        _ok(self._lib.pa_bm_append(self._h, sp, np_, seqs.size,
                                   slots.ctypes.data, slots.size,
                                   copies.ctypes.data, copies.shape[0],
                                   ctypes.byref(n)), self._lib)
        return slots[:total], copies[:n.value]

    def block_tables(self, seqs, max_blocks: int):
        """(int32 [len(seqs), max_blocks] tables padded with -1, int32 lengths)."""
        ids, ip = _host_i32(seqs, "seqs")
        tables = np.empty((max(ids.size, 1), max_blocks), np.int32)
        lens = np.empty(max(ids.size, 1), np.int32)
        _ok(self._lib.pa_bm_block_tables(self._h, ip, ids.size, max_blocks,
                                         tables.ctypes.data,
                                         lens.ctypes.data), self._lib)
        return tables[:ids.size], lens[:ids.size]

    def num_free(self) -> int:
        return self._lib.pa_bm_num_free_blocks(self._h)

    def ref_count(self, block: int) -> int:
        return self._lib.pa_bm_ref_count(self._h, block)

    def length(self, seq: int) -> int:
        return self._lib.pa_bm_sequence_length(self._h, seq)


def hbm_read_probe(src: torch.Tensor, sink: torch.Tensor, chunk_order=None) -> None:
    """Read every byte of the contiguous device tensor src once, as 4 KiB
    chunks in sequence or in the order of the device int32 tensor
    chunk_order (see pa_hbm_read_probe); sink: a device int32 tensor of one
    element or more, written only for an improbable data value."""
    lib = library()
    if not src.is_contiguous() or src.device.type != "cuda":
        raise ValueError("src must be a contiguous device tensor")
    if sink.device != src.device or sink.dtype not in (torch.int32, torch.uint32):
        raise ValueError("sink must be an int32 tensor on src's device")
    nbytes = src.numel() * src.element_size()
    if chunk_order is not None and (chunk_order.device != src.device or chunk_order.dtype !=
                                    torch.int32 or chunk_order.numel() != nbytes // 4096):
        raise ValueError("chunk_order must be an int32 device tensor of bytes // 4096 entries")
    _ok(lib.pa_hbm_read_probe(ctypes.c_void_p(src.data_ptr()), nbytes,
                              None if chunk_order is None else ctypes.c_void_p(chunk_order.data_ptr()),
                              ctypes.c_void_p(sink.data_ptr()), _stream(src)), lib)


def copy_blocks(k_cache, v_cache, block_pairs, k_scale=None, v_scale=None, int4=False):
    """Copy whole blocks (every KV head) from source to destination inside one
    pool; block_pairs is int32 [n, 2] (a host array is moved to the GPU)."""
    lib = library()
    if not isinstance(block_pairs, torch.Tensor) or not block_pairs.is_cuda:
        block_pairs = torch.as_tensor(np.ascontiguousarray(block_pairs, np.int32).reshape(-1, 2),
                                      device=k_cache.device)
    n = block_pairs.shape[0]
    i8 = int4 or k_cache.dtype in QUANTIZED
    desc = int4_desc(k_cache) if int4 else CacheDesc.of(k_cache)
    _check_pools(k_cache, v_cache, k_scale, v_scale, int4)
    _ok(lib.pa_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(k_scale, "k_scale", torch.float16) if i8 else None,
                           _dev(v_scale, "v_scale", torch.float16) if i8 else None,
                           _dev(block_pairs, "block_pairs", torch.int32, 2), n,
                           ctypes.byref(desc), _stream(k_cache)), lib)
