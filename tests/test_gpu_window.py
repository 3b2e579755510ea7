"""Sliding-window decode attention on the GPU against the fp64 oracle (needs
an MI355X): every cache format and both attention kernels, windows from one
row to the whole context, windows that start mid-tile and mid-partition,
freed blocks before the window, and a full-size case."""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
import workloads as W
from gpu_cases import TOL, dev, host, max_abs_err, quantize_blocks_oracle, quantize_pool_gpu
from test_gpu_kernels import make, to_dev

pytestmark = pytest.mark.gpu


def setup(fmt, hq, hkv, d, bs, ctx, seed):
    shape, lay, case = make(fmt, hq, hkv, d, bs, ctx, seed=seed, spare_blocks=2)
    kc, vc = case.k_cache.to(dev()), case.v_cache.to(dev())
    ks = vs = oks = ovs = None
    okc, ovc = host(case.k_cache), host(case.v_cache)
    if fmt in W.QUANTIZED:
        src_k, src_v = kc.nan_to_num(0.0), vc.nan_to_num(0.0)
        kc, vc, ks, vs = quantize_pool_gpu(src_k, src_v, None, fmt)
        okc, ovc, oks, ovs, _ = quantize_blocks_oracle(src_k, src_v, range(lay.num_blocks), fmt)
    return shape, lay, case, kc, vc, ks, vs, okc, ovc, oks, ovs


def run(case, lay, kc, vc, ks, vs, scale, window, bt=None):
    q, ctx = to_dev(case.q, lay.context_lens)
    bt = to_dev(lay.block_tables)[0] if bt is None else bt
    out = torch.full_like(q, float("nan"))
    pa.paged_decode_attention_window(q, kc, vc, bt, ctx, scale, window, out, ks, vs)
    torch.cuda.synchronize()
    return out


CASES = [("f32", 4, 2, 64, 4), ("f16", 8, 2, 128, 16), ("f16", 8, 8, 64, 4),
         ("bf16", 16, 2, 128, 32), ("i8", 8, 2, 128, 16), ("fp8", 8, 2, 64, 16),
         ("fp8", 4, 4, 128, 8)]


@pytest.mark.parametrize("fmt,hq,hkv,d,bs", CASES)
@pytest.mark.parametrize("window", [1, 7, 37, 256, 1000, 0])
def test_window_matches_oracle(fmt, hq, hkv, d, bs, window, orc):
    ctx = [1, 5, 40, 300, 1029, 2048]
    shape, lay, case, kc, vc, ks, vs, okc, ovc, oks, ovs = setup(fmt, hq, hkv, d, bs, ctx, 7)
    print(f"window {fmt} hq={hq} hkv={hkv} d={d} bs={bs} w={window}", flush=True)
    out = run(case, lay, kc, vc, ks, vs, shape.scale, window)
    ref = oracle.paged_decode_attention_window(
        host(case.q), okc, ovc, host(lay.block_tables), host(lay.context_lens), shape.scale,
        window, k_scale=oks, v_scale=ovs, bf16=fmt == "bf16", num_threads=8, lib=orc)
    assert torch.isfinite(out).all()
    assert max_abs_err(out, ref) <= TOL[fmt]


@pytest.mark.parametrize("fmt,hq,hkv,d,bs", [("f16", 8, 2, 128, 16), ("f32", 4, 2, 64, 4),
                                             ("fp8", 8, 2, 128, 16)])
def test_window_ignores_freed_blocks(fmt, hq, hkv, d, bs):
    """Blocks wholly before the window freed: -1 table entries and NaN rows
    change no bit of the output."""
    ctx = [700, 1029, 64, 2048]
    window = 300
    shape, lay, case, kc, vc, ks, vs, *_ = setup(fmt, hq, hkv, d, bs, ctx, 8)
    ref = run(case, lay, kc, vc, ks, vs, shape.scale, window)
    bt = lay.block_tables.clone()
    kc2, vc2 = kc.clone(), vc.clone()
    for s, c in enumerate(ctx):
        first = max(0, c - window)
        for j in range(first // bs):
            blk = int(bt[s, j])
            if fmt not in W.QUANTIZED:
                kc2[blk] = float("nan")
                vc2[blk] = float("nan")
            bt[s, j] = -1
    got = run(case, lay, kc2, vc2, ks, vs, shape.scale, window, bt.to(dev()))
    assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))


def test_window_argument_checks():
    q = torch.zeros((1, 2, 64), dtype=torch.float16, device=dev())
    kc = torch.zeros((4, 2, 16, 64), dtype=torch.float16, device=dev())
    bt = torch.zeros((1, 4), dtype=torch.int32, device=dev())
    ctx = torch.ones(1, dtype=torch.int32, device=dev())
    with pytest.raises(pa.PagedAttnError, match="window"):
        pa.paged_decode_attention_window(q, kc, kc, bt, ctx, 0.1, -1, q.clone())


def test_window_full_size_sampled(orc):
    """Llama-3-8B layer shape, 16 sequences of 16384 positions, a 4096-token
    window, fp16, the library's plan; sampled (sequence, head) rows."""
    ctx = [16384] * 16
    shape, lay, case = make("f16", 32, 8, 128, 16, ctx, seed=9, spare_blocks=0)
    kc, vc = case.k_cache.to(dev()), case.v_cache.to(dev())
    out = run(case, lay, kc, vc, None, None, shape.scale, 4096)
    rng = np.random.default_rng(12)
    pairs = [(int(rng.integers(16)), int(rng.integers(32))) for _ in range(24)]
    ref = oracle.paged_decode_attention_window(
        host(case.q), host(case.k_cache), host(case.v_cache), host(lay.block_tables),
        host(lay.context_lens), shape.scale, 4096, pairs=pairs, num_threads=8, lib=orc)
    assert torch.isfinite(out).all()
    assert max_abs_err(out, ref, pairs) <= TOL["f16"]
