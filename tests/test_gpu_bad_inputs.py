"""Broken device data on every decode kernel (needs an MI355X).

A context length past the table, a negative context length, or a block id
outside the pool makes that sequence's rows NaN -- on the vector-ALU and the
matrix-core kernels, for every cache format, with the library's own plan and
with explicit partitions.  The untouched sequence's rows equal those of the
same call over unbroken inputs bit for bit: a row's partitions and arithmetic
do not depend on the other sequences.  (The kernels check these inputs
themselves; nothing here reads outside a buffer.)"""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
from gpu_cases import decode_gpu, dev, quantize_pool_gpu
from test_gpu_int4 import quantize_all_gpu
from test_gpu_kernels import make, to_dev

pytestmark = pytest.mark.gpu

CASES = [  # (format, q heads, kv heads): G < 4 runs the vector-ALU kernel
    ("f16", 4, 4), ("f16", 8, 2), ("bf16", 16, 2), ("i8", 4, 4), ("i8", 8, 2),
    ("fp8", 4, 4), ("fp8", 8, 2), ("i4", 4, 4), ("i4", 8, 2), ("i4", 16, 2),
]


def pools(fmt, case):
    """Device K/V pools (and scales) of the format, from the case's fp16/bf16 rows."""
    if fmt in ("f16", "bf16"):
        return case.k_cache.to(dev()), case.v_cache.to(dev()), None, None
    src_k = case.k_cache.nan_to_num(0.0).to(dev())
    src_v = case.v_cache.nan_to_num(0.0).to(dev())
    if fmt == "i4":
        return quantize_all_gpu(src_k, src_v)
    return quantize_pool_gpu(src_k, src_v, None, fmt)


def run(fmt, q, kc, vc, ks, vs, bt, ctx, scale, part):
    if fmt != "i4":
        return decode_gpu(q, kc, vc, bt, ctx, scale, part, ks, vs)
    out = torch.empty_like(q)
    if part is None:
        pa.paged_decode_attention_int4(q, kc, vc, ks, vs, bt, ctx, scale, out)
    else:
        s, hq, d = q.shape
        maxb, bs = bt.shape[1], kc.shape[2]
        nbytes = pa.decode_workspace_bytes(pa.int4_desc(kc), s, hq, maxb, part)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev())
        pa.decode_partitions(q, kc, vc, bt, ctx, scale, out, part, ws, ks, vs, int4=True)
        if -(-maxb * bs // part) > 1:
            pa.lse_merge(ws, ctx, hq, d, maxb, bs, part, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fmt,hq,hkv", CASES)
@pytest.mark.parametrize("part", [None, 16, 64])
def test_bad_inputs_nan_only_their_sequence(fmt, hq, hkv, part):
    d, bs = 128, 16
    rows = "bf16" if fmt == "bf16" else "f16"
    shape, lay, case = make(rows, hq, hkv, d, bs, [40, 40, 40, 40], seed=21)
    kc, vc, ks, vs = pools(fmt, case)
    q, bt, ctx = to_dev(case.q, lay.block_tables, lay.context_lens)
    print(f"bad inputs {fmt} hq={hq} hkv={hkv} part={part}", flush=True)
    good = run(fmt, q, kc, vc, ks, vs, bt, ctx, shape.scale, part)
    bad_ctx, bad_bt = ctx.clone(), bt.clone()
    bad_ctx[1] = lay.max_blocks * bs + 1
    bad_ctx[2] = -3
    bad_bt[3, 1] = lay.num_blocks + 1000
    out = run(fmt, q, kc, vc, ks, vs, bad_bt, bad_ctx, shape.scale, part)
    assert torch.isfinite(good).all()
    assert torch.isnan(out[1:]).all()
    assert np.array_equal(out[0].view(torch.int16).cpu().numpy(),
                          good[0].view(torch.int16).cpu().numpy())
