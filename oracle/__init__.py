"""CPU oracle for paged KV-cache decode attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never touches it.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only builds
it with gcc, loads it with ctypes and marshals numpy arrays.  Which passage of
the pages each function follows is stated beside it in ``oracle.c``.

Parity status: every function is pinned by tests against values the pages
print, closed forms, special cases or a library routine, except the int8
quantizer's exact codes, which the pages do not define ("parity unpinned":
pinned only by its own error bound and special cases).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

F32, F16, BF16, I8, FP8, I4 = 0, 1, 2, 3, 4, 5
_ERRORS = {
    -1: "bad argument",
    -2: "slot outside the pool",
    -3: "slot used twice",
    -4: "context length outside the block table",
    -5: "block id outside the pool",
    -6: "out of memory",
}

_lock = threading.Lock()
_lib = None


def build(output: str = LIBRARY, source: str = SOURCE, extra_flags=()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", *extra_flags, source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library (building it first if it is not there)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                build()
            _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = dbl
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = dbl
    lib.oracle_double_to_f16_bits.argtypes = [dbl]
    lib.oracle_double_to_f16_bits.restype = ctypes.c_uint16
    lib.oracle_slot_mapping.argtypes = [P, i32, P, P, i64, i32, P]
    lib.oracle_decode_slot_mapping.argtypes = [P, i32, P, i32, i32, P]
    lib.oracle_kv_append.argtypes = [P, P, P, i64, P, P, i32, i32, i32, i32, i32]
    lib.oracle_fp8_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_e4m3_to_double.restype = dbl
    lib.oracle_double_to_fp8_e4m3.argtypes = [dbl]
    lib.oracle_double_to_fp8_e4m3.restype = ctypes.c_uint8
    lib.oracle_quantize_row_fp8.argtypes = [P, i32, P, P]
    lib.oracle_quantize_row_fp8.restype = None
    lib.oracle_kv_append_fp8.argtypes = [P, P, P, i64, P, P, P, P, i32, i32, i32, i32]
    lib.oracle_quantize_row_int4.argtypes = [P, i32, P, P]
    lib.oracle_quantize_row_int4.restype = None
    lib.oracle_kv_append_int4.argtypes = [P, P, P, i64, P, P, P, P, i32, i32, i32, i32]
    lib.oracle_quantize_row_int8.argtypes = [P, i32, P, P]
    lib.oracle_quantize_row_int8.restype = None
    lib.oracle_kv_append_int8.argtypes = [P, P, P, i64, P, P, P, P, i32, i32, i32, i32]
    lib.oracle_attention_dense.argtypes = [P, P, P, i64, i32, dbl, P, P]
    lib.oracle_paged_decode_attention.argtypes = [
        P, i32, P, P, P, P, i32, P, i32, P, i32, i32, i32, i32, i32, i32, dbl, P, i64, P, i32]
    lib.oracle_paged_decode_attention_window.argtypes = [
        P, i32, P, P, P, P, i32, P, i32, P, i32, i32, i32, i32, i32, i32, dbl, i32, P, i64, P,
        i32]
    lib.oracle_paged_prefill_attention.argtypes = [
        P, i32, P, P, P, P, i32, P, i32, P, P, i32, i32, i32, i32, i32, i32, dbl, P, i64, P,
        i32]
    lib.oracle_gather_kv.argtypes = [P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32,
                                     P, P, P, P]
    lib.oracle_project_row.argtypes = [P, P, i32, i32, P]
    lib.oracle_project_row.restype = None
    lib.oracle_kv_bytes_per_token.argtypes = [i64, i64, i64, i64]
    lib.oracle_kv_bytes_per_token.restype = i64
    lib.oracle_max_threads.restype = i32
    for name in ("oracle_slot_mapping", "oracle_decode_slot_mapping", "oracle_kv_append",
                 "oracle_kv_append_int8", "oracle_kv_append_fp8", "oracle_kv_append_int4",
                 "oracle_attention_dense",
                 "oracle_paged_decode_attention", "oracle_paged_prefill_attention",
                 "oracle_paged_decode_attention_window",
                 "oracle_gather_kv"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


class OracleError(RuntimeError):
    pass


def _check(code: int) -> None:
    if code != 0:
        raise OracleError(_ERRORS.get(code, f"oracle error {code}"))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dtype_code(a: np.ndarray, bf16: bool = False, int4: bool = False) -> int:
    """Format code of a numpy array; bf16 data travels as uint16 bit patterns."""
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.uint16:
        return BF16 if bf16 else F16
    if a.dtype == np.int8:
        return I8
    if a.dtype == np.uint8:          # fp8 E4M3 codes, or packed int4 pairs
        return I4 if int4 else FP8
    raise TypeError(f"unsupported oracle dtype {a.dtype}")


# --------------------------------------------------------------------------
# thin wrappers (marshalling only)

def f16_to_double(bits: int, lib=None) -> float:
    return (lib or load()).oracle_f16_to_double(int(bits))


def bf16_to_double(bits: int, lib=None) -> float:
    return (lib or load()).oracle_bf16_to_double(int(bits))


def double_to_f16_bits(x: float, lib=None) -> int:
    return (lib or load()).oracle_double_to_f16_bits(float(x))


def slot_mapping(block_tables, token_seq, token_pos, block_size, lib=None) -> np.ndarray:
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    seq = np.ascontiguousarray(token_seq, dtype=np.int32)
    pos = np.ascontiguousarray(token_pos, dtype=np.int32)
    out = np.empty(seq.shape[0], dtype=np.int64)
    _check((lib or load()).oracle_slot_mapping(_ptr(bt), bt.shape[1], _ptr(seq), _ptr(pos),
                                               seq.shape[0], block_size, _ptr(out)))
    return out


def decode_slot_mapping(block_tables, context_lens, block_size, lib=None) -> np.ndarray:
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.empty(ctx.shape[0], dtype=np.int64)
    _check((lib or load()).oracle_decode_slot_mapping(_ptr(bt), bt.shape[1], _ptr(ctx),
                                                      ctx.shape[0], block_size, _ptr(out)))
    return out


def kv_append(k_new, v_new, slots, k_cache, v_cache, bf16=False, lib=None) -> None:
    """In-place scatter of [T, Hkv, D] rows into [NB, Hkv, BS, D] caches."""
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    nb, hkv, bs, d = k_cache.shape
    assert k_new.shape == (slots.shape[0], hkv, d) and v_new.shape == k_new.shape
    assert k_new.dtype == k_cache.dtype == v_cache.dtype == v_new.dtype
    _check((lib or load()).oracle_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(slots), slots.shape[0], _ptr(k_cache), _ptr(v_cache),
        nb, hkv, bs, d, _dtype_code(k_cache, bf16)))


def quantize_row_int8(x_f16: np.ndarray, lib=None):
    x = np.ascontiguousarray(x_f16, dtype=np.float16).view(np.uint16)
    q = np.empty(x.shape[0], dtype=np.int8)
    s = np.empty(1, dtype=np.uint16)
    (lib or load()).oracle_quantize_row_int8(_ptr(x), x.shape[0], _ptr(q), _ptr(s))
    return q, s.view(np.float16)[0]


def kv_append_int8(k_new, v_new, slots, k_cache, v_cache, k_scale, v_scale, lib=None) -> None:
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    nb, hkv, bs, d = k_cache.shape
    kn = np.ascontiguousarray(k_new, dtype=np.float16).view(np.uint16)
    vn = np.ascontiguousarray(v_new, dtype=np.float16).view(np.uint16)
    assert k_cache.dtype == np.int8 and k_scale.dtype == np.float16
    _check((lib or load()).oracle_kv_append_int8(
        _ptr(kn), _ptr(vn), _ptr(slots), slots.shape[0], _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale.view(np.uint16)), _ptr(v_scale.view(np.uint16)), nb, hkv, bs, d))


def fp8_e4m3_to_double(code: int, lib=None) -> float:
    return (lib or load()).oracle_fp8_e4m3_to_double(code)


def double_to_fp8_e4m3(x: float, lib=None) -> int:
    return int((lib or load()).oracle_double_to_fp8_e4m3(x))


def quantize_row_fp8(x_f16: np.ndarray, lib=None):
    """(uint8 E4M3 codes, fp16 scale) of one row."""
    x = np.ascontiguousarray(x_f16, dtype=np.float16).view(np.uint16)
    q = np.empty(x.shape[0], dtype=np.uint8)
    s = np.empty(1, dtype=np.uint16)
    (lib or load()).oracle_quantize_row_fp8(_ptr(x), x.shape[0], _ptr(q), _ptr(s))
    return q, s.view(np.float16)[0]


def kv_append_fp8(k_new, v_new, slots, k_cache, v_cache, k_scale, v_scale, lib=None) -> None:
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    nb, hkv, bs, d = k_cache.shape
    kn = np.ascontiguousarray(k_new, dtype=np.float16).view(np.uint16)
    vn = np.ascontiguousarray(v_new, dtype=np.float16).view(np.uint16)
    assert k_cache.dtype == np.uint8 and k_scale.dtype == np.float16
    _check((lib or load()).oracle_kv_append_fp8(
        _ptr(kn), _ptr(vn), _ptr(slots), slots.shape[0], _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale.view(np.uint16)), _ptr(v_scale.view(np.uint16)), nb, hkv, bs, d))


INT4_GROUP = 32


def quantize_row_int4(x_f16: np.ndarray, lib=None):
    """(packed uint8 [n/2], fp16 scales [n/32]) of one row."""
    x = np.ascontiguousarray(x_f16, dtype=np.float16).view(np.uint16)
    q = np.empty(x.shape[0] // 2, dtype=np.uint8)
    s = np.empty(x.shape[0] // INT4_GROUP, dtype=np.uint16)
    (lib or load()).oracle_quantize_row_int4(_ptr(x), x.shape[0], _ptr(q), _ptr(s))
    return q, s.view(np.float16)


def kv_append_int4(k_new, v_new, slots, k_cache, v_cache, k_scale, v_scale, lib=None) -> None:
    """k_cache, v_cache: uint8 [NB, Hkv, BS, D/2]; scales fp16 [NB, Hkv, BS, D/32]."""
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    nb, hkv, bs, half = k_cache.shape
    kn = np.ascontiguousarray(k_new, dtype=np.float16).view(np.uint16)
    vn = np.ascontiguousarray(v_new, dtype=np.float16).view(np.uint16)
    assert k_cache.dtype == np.uint8 and k_scale.shape == (nb, hkv, bs, 2 * half // INT4_GROUP)
    _check((lib or load()).oracle_kv_append_int4(
        _ptr(kn), _ptr(vn), _ptr(slots), slots.shape[0], _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale.view(np.uint16)), _ptr(v_scale.view(np.uint16)), nb, hkv, bs, 2 * half))


def attention_dense(q, K, V, scale, lib=None):
    """softmax(q K^T scale) V for one query; returns (out, weights), fp64."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    n, d = K.shape
    out = np.empty(d, dtype=np.float64)
    w = np.empty(max(n, 1), dtype=np.float64)
    _check((lib or load()).oracle_attention_dense(_ptr(q), _ptr(K), _ptr(V), n, d,
                                                  float(scale), _ptr(out), _ptr(w)))
    return out, w[:n]


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale,
                           k_scale=None, v_scale=None, pairs=None, bf16=False, int4=False,
                           num_threads=0, lib=None) -> np.ndarray:
    """fp64 attention output for every (seq, head) pair, or for the listed pairs.

    q: [S, Hq, D] (float32 / float16 / uint16 bf16 bits); caches [NB, Hkv, BS, D]
    (same format, or int8 with fp16 scales [NB, Hkv, BS] and fp16 q).
    Returns [S, Hq, D] when pairs is None, else [len(pairs), D].
    """
    q = np.ascontiguousarray(q)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    nb, hkv, bs, d = k_cache.shape
    if int4:                     # packed pairs: D / 2 bytes per row
        d *= 2
    s_, hq, dq = q.shape
    assert dq == d and bt.shape[0] == s_ and ctx.shape[0] == s_
    cache_code = _dtype_code(k_cache, bf16, int4)
    q_code = _dtype_code(q, bf16)
    ks = None if k_scale is None else np.ascontiguousarray(k_scale).view(np.uint16)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale).view(np.uint16)
    if pairs is None:
        out = np.empty((s_, hq, d), dtype=np.float64)
        pp, n_pairs = None, s_ * hq
    else:
        pp = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
        n_pairs = pp.shape[0]
        out = np.empty((n_pairs, d), dtype=np.float64)
    _check((lib or load()).oracle_paged_decode_attention(
        _ptr(q), q_code, _ptr(k_cache), _ptr(v_cache), _ptr(ks), _ptr(vs), cache_code,
        _ptr(bt), bt.shape[1], _ptr(ctx), s_, hq, hkv, nb, bs, d, float(scale), _ptr(pp),
        n_pairs, _ptr(out), int(num_threads)))
    return out


def paged_decode_attention_window(q, k_cache, v_cache, block_tables, context_lens, scale,
                                  window, k_scale=None, v_scale=None, pairs=None, bf16=False,
                                  int4=False,
                                  num_threads=0, lib=None) -> np.ndarray:
    """fp64 decode attention over each sequence's last `window` positions
    (window <= 0: all).  Arguments and result as paged_decode_attention."""
    q = np.ascontiguousarray(q)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    nb, hkv, bs, d = k_cache.shape
    if int4:                     # packed pairs: D / 2 bytes per row
        d *= 2
    s_, hq, dq = q.shape
    assert dq == d and bt.shape[0] == s_ and ctx.shape[0] == s_
    ks = None if k_scale is None else np.ascontiguousarray(k_scale).view(np.uint16)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale).view(np.uint16)
    if pairs is None:
        out = np.empty((s_, hq, d), dtype=np.float64)
        pp, n_pairs = None, s_ * hq
    else:
        pp = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
        n_pairs = pp.shape[0]
        out = np.empty((n_pairs, d), dtype=np.float64)
    _check((lib or load()).oracle_paged_decode_attention_window(
        _ptr(q), _dtype_code(q, bf16), _ptr(k_cache), _ptr(v_cache), _ptr(ks), _ptr(vs),
        _dtype_code(k_cache, bf16, int4), _ptr(bt), bt.shape[1], _ptr(ctx), s_, hq, hkv, nb, bs, d,
        float(scale), int(window), _ptr(pp), n_pairs, _ptr(out), int(num_threads)))
    return out


def paged_prefill_attention(q, k_cache, v_cache, block_tables, query_start, context_lens,
                            scale, k_scale=None, v_scale=None, rows=None, bf16=False,
                            num_threads=0, lib=None) -> np.ndarray:
    """fp64 causal attention of every query token (or the listed (token, head)
    rows) over the paged cache.  q: [total, Hq, D]; query_start: int32 [S+1];
    sequence s's tokens sit at its last query_start[s+1]-query_start[s]
    positions.  Returns [total, Hq, D] when rows is None, else [len(rows), D]."""
    q = np.ascontiguousarray(q)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    nb, hkv, bs, d = k_cache.shape
    total, hq, dq = q.shape
    assert dq == d and bt.shape[0] == ctx.shape[0] == qs.shape[0] - 1 and qs[-1] == total
    ks = None if k_scale is None else np.ascontiguousarray(k_scale).view(np.uint16)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale).view(np.uint16)
    if rows is None:
        out = np.empty((total, hq, d), dtype=np.float64)
        rp, n_rows = None, total * hq
    else:
        rp = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
        n_rows = rp.shape[0]
        out = np.empty((n_rows, d), dtype=np.float64)
    _check((lib or load()).oracle_paged_prefill_attention(
        _ptr(q), _dtype_code(q, bf16), _ptr(k_cache), _ptr(v_cache), _ptr(ks), _ptr(vs),
        _dtype_code(k_cache, bf16), _ptr(bt), bt.shape[1], _ptr(qs), _ptr(ctx), ctx.shape[0],
        hq, hkv, nb, bs, d, float(scale), _ptr(rp), n_rows, _ptr(out), int(num_threads)))
    return out


def gather_kv(k_cache, v_cache, block_tables, context_lens, k_out, v_out,
              k_scale=None, v_scale=None, k_scale_out=None, v_scale_out=None,
              bf16=False, int4=False, lib=None) -> None:
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    nb, hkv, bs, d = k_cache.shape
    if int4:                     # packed pairs: D / 2 bytes per row
        d *= 2

    def u16(a):
        return None if a is None else a.view(np.uint16)

    _check((lib or load()).oracle_gather_kv(
        _ptr(k_cache), _ptr(v_cache), _ptr(u16(k_scale)), _ptr(u16(v_scale)), _ptr(bt),
        bt.shape[1], _ptr(ctx), bt.shape[0], nb, hkv, bs, d, _dtype_code(k_cache, bf16, int4),
        _ptr(k_out), _ptr(v_out), _ptr(u16(k_scale_out)), _ptr(u16(v_scale_out))))


def project_row(x, W, lib=None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    W = np.ascontiguousarray(W, dtype=np.float64)
    y = np.empty(W.shape[1], dtype=np.float64)
    (lib or load()).oracle_project_row(_ptr(x), _ptr(W), W.shape[0], W.shape[1], _ptr(y))
    return y


def kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_number, lib=None) -> int:
    return int((lib or load()).oracle_kv_bytes_per_token(n_layers, n_kv_heads, head_dim,
                                                         bytes_per_number))


def max_threads(lib=None) -> int:
    return int((lib or load()).oracle_max_threads())
