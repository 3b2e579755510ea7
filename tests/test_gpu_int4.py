"""int4 caches on the GPU against the oracle (needs an MI355X): the
quantizing append bit-exact (packed codes and group scales), decode
attention over the same codes and scales within tolerance (the vector-ALU
kernel at one or two query heads per KV head, head_dim 64 or block 4; the
matrix-core kernels at 4, 8, 16 and 32 with head_dim 128 and blocks of 16 or
32: four heads per workgroup as (head, group) columns, eight or sixteen as one
head per column), windowed decode on both, the gather and the block copy, and
full-size cases."""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
import workloads as W
from gpu_cases import TOL, dev, host, max_abs_err
from test_gpu_kernels import make, to_dev

pytestmark = pytest.mark.gpu
TOL_I4 = TOL["i8"]    # quantized caches: against the oracle over the same codes


def int4_pools(nb, hkv, bs, d):
    kq = torch.full((nb, hkv, bs, d // 2), 0x5A, dtype=torch.uint8, device=dev())
    ks = torch.full((nb, hkv, bs, d // 32), float("nan"), dtype=torch.float16, device=dev())
    return kq, kq.clone(), ks, ks.clone()


def quantize_all_gpu(src_k, src_v):
    """Every pool row appended (identity slots) into fresh int4 pools."""
    nb, hkv, bs, d = src_k.shape
    rows = lambda x: x.permute(0, 2, 1, 3).reshape(nb * bs, hkv, d).contiguous()
    kq, vq, ks, vs = int4_pools(nb, hkv, bs, d)
    slots = torch.arange(nb * bs, dtype=torch.int64, device=dev())
    pa.kv_append_int4(rows(src_k), rows(src_v), slots, kq, vq, ks, vs)
    return kq, vq, ks, vs


def quantize_all_oracle(src_k, src_v, blocks=None):
    """Oracle int4 pools holding the given blocks (default: all; others zero)."""
    nb, hkv, bs, d = src_k.shape
    blocks = np.arange(nb) if blocks is None else np.asarray(sorted(set(blocks)), np.int64)
    bi = torch.as_tensor(blocks, device=src_k.device)
    rows = lambda x: np.ascontiguousarray(host(x[bi]).transpose(0, 2, 1, 3).reshape(-1, hkv, d))
    kq = np.zeros((nb, hkv, bs, d // 2), np.uint8)
    vq = np.zeros_like(kq)
    ks = np.zeros((nb, hkv, bs, d // 32), np.float16)
    vs = np.zeros_like(ks)
    slots = (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
    oracle.kv_append_int4(rows(src_k), rows(src_v), slots, kq, vq, ks, vs)
    return kq, vq, ks, vs


@pytest.mark.parametrize("d", [64, 128])
def test_kv_append_int4_bit_exact(d):
    nb, hkv, bs, t = 10, 2, 16, 40
    k_new = (torch.randn((t, hkv, d), generator=W.generator(29)) *
             torch.logspace(-4, 4, t)[:, None, None]).to(torch.float16)
    v_new = W.randn((t, hkv, d), "f16", 30)
    k_new[3] = 0                        # zero groups: scale 0, codes 0
    k_new[4, 0, :5] = torch.tensor([65504, -65504, 1e-7, 6e-8, -3.0])
    k_new[6, 1, :8] = torch.tensor([7, -3.5, 2.5, 0.5, -0.5, 6.5, -7, 0])   # ties, s = 1
    k_new[6, 1, 8:32] = 0
    v_new[8, 1, 2] = float("nan")       # a NaN codes as 0
    slots = torch.randperm(nb * bs, generator=W.generator(31))[:t].to(torch.int64)
    slots[5] = -1
    slots[9] = nb * bs                  # outside the pool: skipped
    kq, vq, ks, vs = int4_pools(nb, hkv, bs, d)
    hk, hv, hks, hvs = host(kq).copy(), host(vq).copy(), host(ks).copy(), host(vs).copy()
    print(f"kv_append_int4 d={d}", flush=True)
    kn, vn, sl = to_dev(k_new, v_new, slots)
    pa.kv_append_int4(kn, vn, sl, kq, vq, ks, vs)
    torch.cuda.synchronize()
    ok = slots.clone()
    ok[ok >= nb * bs] = -1
    oracle.kv_append_int4(host(k_new), host(v_new), ok.numpy(), hk, hv, hks, hvs)
    assert host(kq).tobytes() == hk.tobytes() and host(vq).tobytes() == hv.tobytes()
    assert host(ks).view(np.uint16).tobytes() == hks.view(np.uint16).tobytes()
    assert host(vs).view(np.uint16).tobytes() == hvs.view(np.uint16).tobytes()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [4, 16, 32])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (16, 2), (32, 2), (64, 2)])
def test_int4_decode_matches_oracle(d, bs, hq, hkv, orc):
    ctx = [1, bs + 3, 200, 513]
    shape, lay, case = make("f16", hq, hkv, d, bs, ctx, seed=5, spare_blocks=2)
    src_k = case.k_cache.nan_to_num(0.0).to(dev())
    src_v = case.v_cache.nan_to_num(0.0).to(dev())
    print(f"int4 decode d={d} bs={bs} hq={hq} hkv={hkv}", flush=True)
    kq, vq, ks, vs = quantize_all_gpu(src_k, src_v)
    okq, ovq, oks, ovs = quantize_all_oracle(src_k, src_v)
    assert host(kq).tobytes() == okq.tobytes() and host(vs).tobytes() == ovs.tobytes()
    q, bt, ctx_t = to_dev(case.q, lay.block_tables, lay.context_lens)
    ref = oracle.paged_decode_attention(host(case.q), okq, ovq, host(lay.block_tables),
                                        host(lay.context_lens), shape.scale, k_scale=oks,
                                        v_scale=ovs, int4=True, num_threads=8, lib=orc)
    out = torch.empty_like(q)
    pa.paged_decode_attention_int4(q, kq, vq, ks, vs, bt, ctx_t, shape.scale, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert max_abs_err(out, ref) <= TOL_I4
    # explicit partitions: one tile, and the whole table
    tile = max(bs, 1024 // (d // 2))
    for part in (tile, -(-lay.max_blocks * bs // tile) * tile):
        nbytes = pa.decode_workspace_bytes(pa.int4_desc(kq), len(ctx), hq, lay.max_blocks, part)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev())
        out = torch.empty_like(q)
        pa.decode_partitions(q, kq, vq, bt, ctx_t, shape.scale, out, part, ws, ks, vs, int4=True)
        if -(-lay.max_blocks * bs // part) > 1:
            pa.lse_merge(ws, ctx_t, hq, d, lay.max_blocks, bs, part, out)
        torch.cuda.synchronize()
        assert max_abs_err(out, ref) <= TOL_I4, part


def test_int4_window_gather_copy(orc):
    hq, hkv, d, bs = 8, 2, 128, 16
    ctx = [40, 300, 1029]
    shape, lay, case = make("f16", hq, hkv, d, bs, ctx, seed=6, spare_blocks=4)
    src_k = case.k_cache.nan_to_num(0.0).to(dev())
    src_v = case.v_cache.nan_to_num(0.0).to(dev())
    kq, vq, ks, vs = quantize_all_gpu(src_k, src_v)
    okq, ovq, oks, ovs = quantize_all_oracle(src_k, src_v)
    q, bt, ctx_t = to_dev(case.q, lay.block_tables, lay.context_lens)
    # window
    out = torch.empty_like(q)
    pa.paged_decode_attention_window(q, kq, vq, bt, ctx_t, shape.scale, 100, out, ks, vs,
                                     int4=True)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention_window(host(case.q), okq, ovq, host(lay.block_tables),
                                               host(lay.context_lens), shape.scale, 100,
                                               k_scale=oks, v_scale=ovs, int4=True, lib=orc)
    assert max_abs_err(out, ref) <= TOL_I4
    # gather: packed rows and their group scales
    cap = lay.max_blocks * bs
    ko = torch.zeros((3, cap, hkv, d // 2), dtype=torch.uint8, device=dev())
    vo = torch.zeros_like(ko)
    kso = torch.zeros((3, cap, hkv, d // 32), dtype=torch.float16, device=dev())
    vso = torch.zeros_like(kso)
    pa.gather_kv(kq, vq, bt, ctx_t, ko, vo, ks, vs, kso, vso, int4=True)
    torch.cuda.synchronize()
    rko, rvo = np.zeros((3, cap, hkv, d // 2), np.uint8), np.zeros((3, cap, hkv, d // 2), np.uint8)
    rkso = np.zeros((3, cap, hkv, d // 32), np.float16)
    rvso = np.zeros_like(rkso)
    oracle.gather_kv(okq, ovq, host(lay.block_tables), host(lay.context_lens), rko, rvo,
                     k_scale=oks, v_scale=ovs, k_scale_out=rkso, v_scale_out=rvso, int4=True,
                     lib=orc)
    assert host(ko).tobytes() == rko.tobytes() and host(vo).tobytes() == rvo.tobytes()
    assert host(kso).tobytes() == rkso.tobytes() and host(vso).tobytes() == rvso.tobytes()
    # block copy: codes and group scales move together
    free = sorted(set(range(lay.num_blocks)) - set(lay.block_tables[lay.block_tables >= 0].tolist()))
    src = lay.block_tables[1, :2].tolist()
    pairs = np.array([[src[0], free[0]], [src[1], free[1]]], np.int32)
    want = [host(t).copy() for t in (kq, vq, ks, vs)]
    for w in want:
        w[pairs[:, 1]] = w[pairs[:, 0]]
    pa.copy_blocks(kq, vq, pairs, ks, vs, int4=True)
    torch.cuda.synchronize()
    for g, w in zip((kq, vq, ks, vs), want):
        assert host(g).tobytes() == w.tobytes()


@pytest.mark.parametrize("hq,bs", [(16, 16), (32, 32)])
def test_int4_window_head_columns(hq, bs, orc):
    """Windowed decode with eight or sixteen query heads per KV head (one head
    per column), windows cutting tiles and partitions mid-way."""
    hkv, d = 2, 128
    ctx = [40, 300, 1029, 2100]
    shape, lay, case = make("f16", hq, hkv, d, bs, ctx, seed=8, spare_blocks=2)
    src_k = case.k_cache.nan_to_num(0.0).to(dev())
    src_v = case.v_cache.nan_to_num(0.0).to(dev())
    kq, vq, ks, vs = quantize_all_gpu(src_k, src_v)
    okq, ovq, oks, ovs = quantize_all_oracle(src_k, src_v)
    q, bt, ctx_t = to_dev(case.q, lay.block_tables, lay.context_lens)
    for window in (7, 100, 1000):
        print(f"int4 window hq={hq} bs={bs} window={window}", flush=True)
        out = torch.empty_like(q)
        pa.paged_decode_attention_window(q, kq, vq, bt, ctx_t, shape.scale, window, out, ks, vs,
                                         int4=True)
        torch.cuda.synchronize()
        ref = oracle.paged_decode_attention_window(host(case.q), okq, ovq,
                                                   host(lay.block_tables), host(lay.context_lens),
                                                   shape.scale, window, k_scale=oks, v_scale=ovs,
                                                   int4=True, lib=orc)
        assert torch.isfinite(out).all()
        assert max_abs_err(out, ref) <= TOL_I4, window


@pytest.mark.parametrize("shape", [W.LLAMA3_8B_I4, W.LLAMA3_70B_I4], ids=lambda s: s.name)
def test_int4_full_size(shape, orc):
    """The benchmark's int4 layers at full size (Llama-3-8B: 64 sequences x
    8192, four heads per workgroup; Llama-3-70B: 32 x 8192 with 64 query / 8
    KV heads, one head per column), the library's own plan: the whole pool
    bit-exact against the oracle's quantizer and every (sequence, head)
    output within tolerance of the oracle over that pool."""
    from gpu_cases import quantize_blocks_oracle
    lay = W.layout_for(shape)
    case = W.make_case(shape, lay, device=dev(), poison=False)
    print(f"int4 full size {shape.name}", flush=True)
    kq, vq, ks, vs = quantize_all_gpu(case.k_cache, case.v_cache)
    bt, ctx = lay.block_tables.to(dev()), lay.context_lens.to(dev())
    out = torch.empty_like(case.q)
    pa.paged_decode_attention_int4(case.q, kq, vq, ks, vs, bt, ctx, shape.scale, out)
    torch.cuda.synchronize()
    want = quantize_blocks_oracle(case.k_cache, case.v_cache, range(lay.num_blocks), "i4")[:4]
    for got, exp in zip((kq, vq, ks, vs), want):
        assert host(got).tobytes() == exp.tobytes()
    ref = oracle.paged_decode_attention(host(case.q), *want[:2], host(lay.block_tables),
                                        host(lay.context_lens), shape.scale, k_scale=want[2],
                                        v_scale=want[3], int4=True, lib=orc)
    assert torch.isfinite(out).all()
    assert max_abs_err(out, ref) <= TOL_I4
