"""The paired plan of the matrix-core decode kernel on the GPU (needs an
MI355X): with one partition per sequence and enough (sequence, KV head) items
that half as many workgroups still meet the plan's target, each workgroup
ranks the context lengths on the device and attends the k-th longest and the
k-th shortest sequence.  Ragged batches of
an odd number of sequences, with zero lengths, equal lengths and broken
lengths among them (the ranking must still take every sequence exactly
once), against the oracle; the fused decode step through the same plan."""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
import workloads as W
from gpu_cases import (TOL, dev, host, max_abs_err, quantize_blocks_oracle,
                       quantize_pool_gpu)
from test_gpu_kernels import make, to_dev

pytestmark = pytest.mark.gpu


def ragged(n, bs, seed):
    rng = np.random.default_rng(seed)
    ctx = [int(x) for x in rng.integers(1, 40 * bs, n)]
    ctx[3] = ctx[10] = 0
    ctx[5] = ctx[6] = ctx[7] = 17 * bs     # ties
    ctx[-1] = 40 * bs
    return ctx


def whole_table(lay, bs):
    return lay.max_blocks * bs


# 16-bit caches pair from 512 items (two per CU); int8 and fp8 from 4096
# (their kernel's 2048-workgroup target, halved grid)
PAIRED = [(dt, hq, hkv, 65) for dt in ("f16", "bf16") for hq, hkv in ((32, 8), (64, 8), (128, 8))]
PAIRED += [(dt, 128, 32, 255) for dt in ("i8", "fp8")]


@pytest.mark.parametrize("dtype,hq,hkv,nseq", PAIRED)
def test_paired_plan_matches_oracle(dtype, hq, hkv, nseq, orc):
    d, bs = 128, 16
    ctx = ragged(nseq, bs, seed=hq)
    print(f"paired plan {dtype} hq={hq} hkv={hkv} seqs={nseq}", flush=True)
    src = "f16" if dtype in ("i8", "fp8") else dtype
    shape, lay, case = make(src, hq, hkv, d, bs, ctx, seed=31)
    q, bt = to_dev(case.q, lay.block_tables)
    # two broken lengths: their rows are NaN, the others unaffected
    ctx_bad = lay.context_lens.clone()
    ctx_bad[20] = -5
    ctx_bad[21] = lay.max_blocks * bs + 1
    ctx_t = ctx_bad.to(dev())
    good = [s for s in range(len(ctx)) if s not in (20, 21)]
    pairs = [(s, h) for s in good for h in range(hq)]
    if dtype in ("i8", "fp8"):
        kc, vc, ks, vs = quantize_pool_gpu(case.k_cache.nan_to_num(0.0).to(dev()),
                                           case.v_cache.nan_to_num(0.0).to(dev()), None, dtype)
        okq, ovq, oks, ovs, _ = quantize_blocks_oracle(case.k_cache.nan_to_num(0.0),
                                                      case.v_cache.nan_to_num(0.0),
                                                      range(lay.num_blocks), dtype)
        ref = oracle.paged_decode_attention(host(case.q), okq, ovq, host(lay.block_tables),
                                            host(lay.context_lens), shape.scale, k_scale=oks,
                                            v_scale=ovs, pairs=pairs, num_threads=8, lib=orc)
    else:
        kc, vc = to_dev(case.k_cache, case.v_cache)
        ks = vs = None
        ref = oracle.paged_decode_attention(host(case.q), host(case.k_cache), host(case.v_cache),
                                            host(lay.block_tables), host(lay.context_lens),
                                            shape.scale, pairs=pairs, bf16=dtype == "bf16",
                                            num_threads=8, lib=orc)
    tol = TOL[dtype]
    # one partition over the whole table: the paired plan
    part = whole_table(lay, bs)
    out = torch.full_like(q, 7.0)
    pa.decode_partitions(q, kc, vc, bt, ctx_t, shape.scale, out, part, None, ks, vs)
    torch.cuda.synchronize()
    assert torch.isnan(out[20]).all() and torch.isnan(out[21]).all()
    assert (out[3] == 0).all() and (out[10] == 0).all()
    assert max_abs_err(out, ref, pairs) <= tol
    # a multi-partition plan (never paired) on the same inputs agrees
    tile = 16
    nbytes = pa.decode_workspace_bytes(kc, len(ctx), hq, lay.max_blocks, 4 * tile)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev())
    out2 = torch.empty_like(q)
    pa.decode_partitions(q, kc, vc, bt, ctx_t, shape.scale, out2, 4 * tile, ws, ks, vs)
    pa.lse_merge(ws, ctx_t, hq, d, lay.max_blocks, bs, 4 * tile, out2)
    torch.cuda.synchronize()
    assert max_abs_err(out2, ref, pairs) <= tol
    assert torch.isnan(out2[20]).all() and torch.isnan(out2[21]).all()


def test_paired_fused_step_full_table():
    """pa_decode_step_partitions over the whole table (paired): the appended
    rows bit-exact against the oracle, every output within tolerance."""
    hq, hkv, d, bs = 64, 8, 128, 16
    ctx = ragged(67, bs, seed=5)
    ctx[3] = ctx[10] = 1
    print("paired fused step", flush=True)
    shape, lay, case = make("bf16", hq, hkv, d, bs, ctx, seed=41, poison_new=True)
    q, kc, vc, kn, vn, bt, ctx_t = to_dev(case.q, case.k_cache, case.v_cache, case.k_new,
                                          case.v_new, lay.block_tables, lay.context_lens)
    out = torch.empty_like(q)
    pa.decode_step_partitions(q, kn, vn, kc, vc, bt, ctx_t, shape.scale, out,
                              whole_table(lay, bs), None)
    torch.cuda.synchronize()
    slots = oracle.decode_slot_mapping(host(lay.block_tables), host(lay.context_lens), bs)
    kh, vh = host(case.k_cache).copy(), host(case.v_cache).copy()
    oracle.kv_append(host(case.k_new), host(case.v_new), slots, kh, vh, bf16=True)
    assert host(kc).tobytes() == kh.tobytes() and host(vc).tobytes() == vh.tobytes()
    ref = oracle.paged_decode_attention(host(case.q), kh, vh, host(lay.block_tables),
                                        host(lay.context_lens), shape.scale, bf16=True,
                                        num_threads=8)
    assert max_abs_err(out, ref) <= TOL["bf16"]
