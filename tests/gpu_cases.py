"""Helpers for the GPU parity tests: run the HIP path through the binding and
the CPU oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import decode_attention_paged_append_amd as pa
import oracle
import workloads as W

# max-abs tolerances of the attention output against the fp64 oracle
# (int8 and fp8 caches: against the oracle over the same codes and scales)
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 8e-3, "i8": 1e-2, "fp8": 1e-2}
ELEM = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "fp8": 1}


def dev():
    return torch.device("cuda", 0)


def host(t: torch.Tensor):
    return W.to_numpy_bits(t)


def tile_tokens(dtype: str, d: int, bs: int) -> int:
    return max(bs, 64 * 16 // (d * ELEM[dtype]))


def decode_gpu(q, kc, vc, bt, ctx, scale, partition_tokens=None, k_scale=None, v_scale=None):
    """HIP decode attention; partition_tokens None = the library's own plan."""
    out = torch.empty_like(q)
    s, hq, d = q.shape
    maxb, bs = bt.shape[1], kc.shape[2]
    if partition_tokens is None:
        if kc.dtype == torch.int8:
            pa.paged_decode_attention_int8(q, kc, vc, k_scale, v_scale, bt, ctx, scale, out)
        elif kc.dtype == torch.float8_e4m3fn:
            pa.paged_decode_attention_fp8(q, kc, vc, k_scale, v_scale, bt, ctx, scale, out)
        else:
            pa.paged_decode_attention(q, kc, vc, bt, ctx, scale, out)
    else:
        nbytes = pa.decode_workspace_bytes(kc, s, hq, maxb, partition_tokens)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        pa.decode_partitions(q, kc, vc, bt, ctx, scale, out, partition_tokens, ws, k_scale, v_scale)
        if -(-maxb * bs // partition_tokens) > 1:
            pa.lse_merge(ws, ctx, hq, d, maxb, bs, partition_tokens, out)
    torch.cuda.synchronize()
    return out


def decode_oracle(q, kc, vc, bt, ctx, scale, pairs=None, k_scale=None, v_scale=None):
    """fp64 oracle from host copies of the same tensors."""
    bf16 = kc.dtype == torch.bfloat16
    return oracle.paged_decode_attention(
        host(q), host(kc), host(vc), host(bt), host(ctx), scale,
        k_scale=None if k_scale is None else host(k_scale),
        v_scale=None if v_scale is None else host(v_scale), pairs=pairs, bf16=bf16)


def max_abs_err(out: torch.Tensor, ref: np.ndarray, pairs=None) -> float:
    got = out.detach().double().cpu().numpy()
    if pairs is not None:
        got = np.stack([got[s, h] for s, h in pairs])
    return float(np.max(np.abs(got - ref))) if ref.size else 0.0


def quantize_pool_gpu(src_k, src_v, layout_blocks, fmt="i8"):
    """int8 / fp8 pool filled by the GPU append of every pool row (identity slots)."""
    nb, hkv, bs, d = src_k.shape
    rows_k = src_k.permute(0, 2, 1, 3).reshape(nb * bs, hkv, d).contiguous()
    rows_v = src_v.permute(0, 2, 1, 3).reshape(nb * bs, hkv, d).contiguous()
    slots = torch.arange(nb * bs, dtype=torch.int64, device=src_k.device)
    codes = torch.int8 if fmt == "i8" else torch.float8_e4m3fn
    kq = torch.zeros((nb, hkv, bs, d), dtype=codes, device=src_k.device)
    vq = torch.zeros_like(kq)
    ks = torch.zeros((nb, hkv, bs), dtype=torch.float16, device=src_k.device)
    vs = torch.zeros_like(ks)
    append = pa.kv_append_int8 if fmt == "i8" else pa.kv_append_fp8
    append(rows_k, rows_v, slots, kq, vq, ks, vs)
    return kq, vq, ks, vs


def quantize_blocks_oracle(src_k, src_v, blocks, fmt="i8"):
    """Oracle int8 / fp8 / int4 pool holding only the given blocks (others
    zero), quantized from the fp16 pools [NB, Hkv, BS, D] on host threads."""
    nb, hkv, bs, d = src_k.shape
    blocks = np.asarray(sorted(set(int(b) for b in blocks)), dtype=np.int64)
    bi = torch.as_tensor(blocks, device=src_k.device)
    sk = host(src_k[bi])   # [n, Hkv, BS, D]
    sv = host(src_v[bi])
    rows_k = np.ascontiguousarray(sk.transpose(0, 2, 1, 3).reshape(-1, hkv, d))
    rows_v = np.ascontiguousarray(sv.transpose(0, 2, 1, 3).reshape(-1, hkv, d))
    del sk, sv
    slots = (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
    int4 = fmt == "i4"
    width = d // 2 if int4 else d
    kq = np.zeros((nb, hkv, bs, width), np.int8 if fmt == "i8" else np.uint8)
    vq = np.zeros_like(kq)
    ks = np.zeros((nb, hkv, bs) + ((d // 32,) if int4 else ()), np.float16)
    vs = np.zeros_like(ks)
    append = {"i8": oracle.kv_append_int8, "fp8": oracle.kv_append_fp8,
              "i4": oracle.kv_append_int4}[fmt]
    # chunks of whole blocks write disjoint slots: run them on host threads
    # (the oracle's C routine runs without the interpreter lock)
    n = rows_k.shape[0]
    workers = min(16, os.cpu_count() or 1)
    step = -(-max(n // bs, 1) // workers) * bs
    spans = [(a, min(a + step, n)) for a in range(0, n, step)]
    with ThreadPoolExecutor(len(spans)) as ex:
        list(ex.map(lambda s: append(rows_k[s[0]:s[1]], rows_v[s[0]:s[1]], slots[s[0]:s[1]],
                                     kq, vq, ks, vs), spans))
    return kq, vq, ks, vs, blocks
