"""The quantized decode step on the GPU against the oracle (needs an MI355X):
the quantizing append of the decoded token fused into the attention launch
(pa_decode_step_quant, pa_decode_step_partitions_quant) over int8, fp8 and
int4 caches, on every attention kernel those caches reach (vector ALU at one
or two query heads per KV head; matrix cores at four, eight and sixteen).

For each case: the pool after the step equals, bit for bit, the oracle's
quantizing append at the decode slots (ctx - 1) of the same starting pool,
whose new-token rows are poisoned first; the output is within tolerance of
the oracle's attention over that pool; and the separate calls (slot mapping,
standalone quantizing append, attention) agree with the fused step."""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
import workloads as W
from gpu_cases import TOL, dev, host, max_abs_err
from test_gpu_kernels import make, to_dev

pytestmark = pytest.mark.gpu

CODE_NP = {"i8": np.int8, "fp8": np.uint8, "i4": np.uint8}
ORACLE_APPEND = {"i8": oracle.kv_append_int8, "fp8": oracle.kv_append_fp8,
                 "i4": oracle.kv_append_int4}
GPU_APPEND = {"i8": pa.kv_append_int8, "fp8": pa.kv_append_fp8, "i4": pa.kv_append_int4}


def oracle_pool(fmt, src_k, src_v):
    """Oracle-quantized pools of every row of fp16 pools [NB, Hkv, BS, D]."""
    nb, hkv, bs, d = src_k.shape
    rows = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(-1, hkv, d))
    width = d // 2 if fmt == "i4" else d
    kq = np.zeros((nb, hkv, bs, width), CODE_NP[fmt])
    vq = np.zeros_like(kq)
    ks = np.zeros((nb, hkv, bs) + ((d // W.INT4_GROUP,) if fmt == "i4" else ()), np.float16)
    vs = np.zeros_like(ks)
    ORACLE_APPEND[fmt](rows(src_k), rows(src_v), np.arange(nb * bs, dtype=np.int64),
                       kq, vq, ks, vs)
    return kq, vq, ks, vs


def to_gpu(fmt, a):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    return t.view(torch.float8_e4m3fn) if fmt == "fp8" and a.dtype == np.uint8 else t


def poison_rows(pools, slots, bs):
    """Garbage codes and NaN scales at the given slots (host arrays, in place)."""
    kq, vq, ks, vs = pools
    for slot in slots:
        if slot < 0:
            continue
        b, o = divmod(int(slot), bs)
        kq[b, :, o] = 0x5A
        vq[b, :, o] = 0x5A
        ks[b, :, o] = np.float16("nan")
        vs[b, :, o] = np.float16("nan")


def setup(fmt, hq, hkv, d, bs, ctx, seed):
    shape, lay, case = make("f16", hq, hkv, d, bs, ctx, seed=seed, spare_blocks=3)
    start = list(oracle_pool(fmt, host(case.k_cache.nan_to_num(0.0)),
                             host(case.v_cache.nan_to_num(0.0))))
    slots = oracle.decode_slot_mapping(host(lay.block_tables), host(lay.context_lens), bs)
    poison_rows(start, slots, bs)
    want = [a.copy() for a in start]
    ORACLE_APPEND[fmt](host(case.k_new), host(case.v_new), slots, *want)
    return shape, lay, case, start, want


def same_bits(got: torch.Tensor, want: np.ndarray) -> bool:
    return host(got).tobytes() == np.ascontiguousarray(want).tobytes()


# (hq, hkv, d, bs): vector ALU at G = 1 and 2 (head_dim 64 and 128), matrix
# cores at G = 4, 8 and 16, blocks of 16 and 32
SHAPES = [(4, 4, 128, 16), (8, 4, 64, 16), (16, 4, 128, 16), (64, 8, 128, 16),
          (32, 2, 128, 16), (16, 4, 128, 32), (8, 2, 64, 32)]


@pytest.mark.parametrize("fmt", ["i8", "fp8", "i4"])
@pytest.mark.parametrize("hq,hkv,d,bs", SHAPES)
def test_decode_step_quant_matches_oracle(fmt, hq, hkv, d, bs, orc):
    ctx = [1, bs, bs + 1, 300, 2049, 700]
    print(f"decode_step_quant {fmt} hq={hq} hkv={hkv} d={d} bs={bs}", flush=True)
    shape, lay, case, start, want = setup(fmt, hq, hkv, d, bs, ctx, seed=17)
    int4 = fmt == "i4"
    ref = oracle.paged_decode_attention(host(case.q), want[0], want[1], host(lay.block_tables),
                                        host(lay.context_lens), shape.scale, k_scale=want[2],
                                        v_scale=want[3], int4=int4, num_threads=8, lib=orc)
    q, kn, vn, bt, ctx_t = to_dev(case.q, case.k_new, case.v_new, lay.block_tables,
                                  lay.context_lens)
    maxb = lay.max_blocks
    desc_of = (lambda k: pa.int4_desc(k)) if int4 else (lambda k: pa.CacheDesc.of(k))
    tile = max(bs, 1024 // (d // 2 if int4 else d))
    # None: the library's plan (one call, merge inside); else explicit
    # partitions: one tile, four tiles, the whole table
    for part in (None, tile, 4 * tile, -(-maxb * bs // tile) * tile):
        pools = [to_gpu(fmt, a) for a in start]
        out = torch.full_like(q, float("nan"))
        if part is None:
            pa.decode_step_quant(q, kn, vn, *pools, bt, ctx_t, shape.scale, out, int4=int4)
        else:
            nbytes = pa.decode_workspace_bytes(desc_of(pools[0]), len(ctx), hq, maxb, part)
            ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev())
            pa.decode_step_partitions_quant(q, kn, vn, *pools, bt, ctx_t, shape.scale, out,
                                            part, ws, int4=int4)
            if -(-maxb * bs // part) > 1:
                pa.lse_merge(ws, ctx_t, hq, d, maxb, bs, part, out)
        torch.cuda.synchronize()
        for got, exp in zip(pools, want):
            assert same_bits(got, exp), f"pool after the step differs (partition {part})"
        assert torch.isfinite(out).all()
        assert max_abs_err(out, ref) <= TOL["i8" if int4 else fmt], part

    # the separate calls on the library's plan
    pools = [to_gpu(fmt, a) for a in start]
    slots = pa.decode_slot_mapping(bt, ctx_t, bs)
    GPU_APPEND[fmt](kn, vn, slots, *pools)
    out2 = torch.empty_like(q)
    if fmt == "i8":
        pa.paged_decode_attention_int8(q, *pools, bt, ctx_t, shape.scale, out2)
    elif fmt == "fp8":
        pa.paged_decode_attention_fp8(q, *pools, bt, ctx_t, shape.scale, out2)
    else:
        pa.paged_decode_attention_int4(q, *pools, bt, ctx_t, shape.scale, out2)
    torch.cuda.synchronize()
    for got, exp in zip(pools, want):
        assert same_bits(got, exp)
    out = torch.empty_like(q)
    fused = [to_gpu(fmt, a) for a in start]
    pa.decode_step_quant(q, kn, vn, *fused, bt, ctx_t, shape.scale, out, int4=int4)
    torch.cuda.synchronize()
    assert (out.double() - out2.double()).abs().max().item() <= TOL["i8"]


@pytest.mark.parametrize("fmt", ["i8", "fp8", "i4"])
def test_decode_step_quant_edge_cases(fmt, orc):
    """Length-0 sequences append nothing and give zeros; a sequence whose new
    position's block id lies outside the pool appends nothing and gives NaN
    rows; every other row matches the oracle, and the pool is untouched
    outside the valid new slots."""
    hq, hkv, d, bs = 16, 4, 128, 16
    ctx = [0, 33, 16, 0, 257]
    print(f"decode_step_quant edge cases {fmt}", flush=True)
    shape, lay, case, start, want = setup(fmt, hq, hkv, d, bs, ctx, seed=23)
    int4 = fmt == "i4"
    bt_bad = lay.block_tables.clone()
    bt_bad[1, (33 - 1) // bs] = lay.num_blocks + 5      # sequence 1's new position
    # the oracle's pool: sequence 1's append is skipped (its slot is -1)
    want = [a.copy() for a in start]
    slots = oracle.decode_slot_mapping(host(lay.block_tables), host(lay.context_lens), bs)
    slots[1] = -1
    ORACLE_APPEND[fmt](host(case.k_new), host(case.v_new), slots, *want)
    good = [0, 2, 3, 4]
    pairs = [(s, h) for s in good for h in range(hq)]
    ref = oracle.paged_decode_attention(host(case.q), want[0], want[1], host(lay.block_tables),
                                        host(lay.context_lens), shape.scale, k_scale=want[2],
                                        v_scale=want[3], pairs=pairs, int4=int4, lib=orc)
    q, kn, vn, bt, ctx_t = to_dev(case.q, case.k_new, case.v_new, bt_bad, lay.context_lens)
    pools = [to_gpu(fmt, a) for a in start]
    out = torch.empty_like(q)
    pa.decode_step_quant(q, kn, vn, *pools, bt, ctx_t, shape.scale, out, int4=int4)
    torch.cuda.synchronize()
    for got, exp in zip(pools, want):
        assert same_bits(got, exp)
    assert torch.isnan(out[1]).all()
    assert (out[0] == 0).all() and (out[3] == 0).all()
    assert max_abs_err(out, ref, pairs) <= TOL["i8" if int4 else fmt]


def test_decode_step_quant_rejects_unquantized_cache():
    hq, hkv, d, bs = 8, 2, 64, 16
    shape, lay, case = make("f16", hq, hkv, d, bs, [5, 9], seed=3)
    q, kc, vc, kn, vn, bt, ctx_t = to_dev(case.q, case.k_cache, case.v_cache, case.k_new,
                                          case.v_new, lay.block_tables, lay.context_lens)
    sc = torch.zeros(kc.shape[:3], dtype=torch.float16, device=dev())
    with pytest.raises(ValueError):
        pa.decode_step_quant(q, kn, vn, kc, vc, sc, sc, bt, ctx_t, shape.scale,
                             torch.empty_like(q))


@pytest.mark.parametrize("shape", [W.LLAMA3_8B_I8, W.LLAMA3_8B_FP8, W.LLAMA3_8B_I4],
                         ids=lambda s: s.name)
def test_decode_step_quant_full_size(shape, orc):
    """The benchmark's quantized step at full size (64 sequences x 8192, the
    library's plan): the whole pool after the step -- every code and scale,
    the new rows included -- bit-exact against the oracle's quantizing append
    of every source row followed by its append of the new rows, whose pool
    slots were poisoned first; and every (sequence, head) output within
    tolerance of the oracle's attention over that pool."""
    from test_gpu_int4 import quantize_all_gpu
    from gpu_cases import quantize_blocks_oracle, quantize_pool_gpu

    fmt = shape.cache_dtype
    int4 = fmt == "i4"
    bs = shape.block_size
    print(f"decode_step_quant full size {shape.name}", flush=True)
    lay = W.layout_for(shape)
    case = W.make_case(shape, lay, device=dev(), seed=7, poison=False)
    if int4:
        pools = list(quantize_all_gpu(case.k_cache, case.v_cache))
    else:
        pools = list(quantize_pool_gpu(case.k_cache, case.v_cache, None, fmt))
    slots = oracle.decode_slot_mapping(host(lay.block_tables), host(lay.context_lens), bs)
    b_idx = torch.as_tensor(slots // bs, device=dev())
    o_idx = torch.as_tensor(slots % bs, device=dev())
    for t in pools[:2]:
        t.view(torch.uint8)[b_idx, :, o_idx] = 0x5A
    for t in pools[2:]:
        t[b_idx, :, o_idx] = float("nan")
    bt, ctx = lay.block_tables.to(dev()), lay.context_lens.to(dev())
    out = torch.empty_like(case.q)
    pa.decode_step_quant(case.q, case.k_new, case.v_new, *pools, bt, ctx, shape.scale, out,
                         int4=int4)
    torch.cuda.synchronize()

    # the new rows: the oracle's quantizer on the same fp16 rows
    s, hkv, d = case.k_new.shape
    width = d // 2 if int4 else d
    small = [np.zeros((s, hkv, bs, width), CODE_NP[fmt]) for _ in range(2)]
    small += [np.zeros((s, hkv, bs) + ((d // W.INT4_GROUP,) if int4 else ()), np.float16)
              for _ in range(2)]
    ORACLE_APPEND[fmt](host(case.k_new), host(case.v_new), np.arange(s, dtype=np.int64) * bs,
                       *small)
    for got, exp in zip(pools, small):
        assert same_bits(got[b_idx, :, o_idx], exp[:, :, 0])

    # every output, over the oracle's whole pool
    want = list(quantize_blocks_oracle(case.k_cache, case.v_cache, range(lay.num_blocks), fmt)[:4])
    ORACLE_APPEND[fmt](host(case.k_new), host(case.v_new), slots, *want)
    for got, exp in zip(pools, want):
        assert same_bits(got, exp)
    ref = oracle.paged_decode_attention(host(case.q), want[0], want[1], host(lay.block_tables),
                                        host(lay.context_lens), shape.scale, k_scale=want[2],
                                        v_scale=want[3], int4=int4, lib=orc)
    assert torch.isfinite(out).all()
    assert max_abs_err(out, ref) <= TOL["i8" if int4 else fmt]
