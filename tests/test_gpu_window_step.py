"""The sliding-window decode step on the GPU against the oracle (needs an
MI355X): pa_decode_step_window stores (fp32 / fp16 / bf16) or quantizes
(int8, fp8, int4) each sequence's new K/V rows at ctx - 1 inside the
windowed attention launch.  The pool after the step equals, bit for bit,
the oracle's append at the decode slots of the same starting pool (new rows
poisoned first); the output is within tolerance of the oracle's windowed
attention over that pool."""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
from gpu_cases import TOL, dev, host, max_abs_err
from test_gpu_kernels import make, to_dev
import test_gpu_quant_step as QS

pytestmark = pytest.mark.gpu

CASES = [("f32", 4, 2, 64, 4), ("f16", 8, 2, 128, 16), ("f16", 32, 32, 128, 16),
         ("bf16", 16, 2, 128, 32), ("bf16", 32, 8, 128, 16), ("i8", 8, 2, 128, 16),
         ("i8", 32, 8, 128, 16), ("fp8", 8, 2, 64, 16), ("i4", 8, 4, 128, 16),
         ("i4", 64, 8, 128, 16)]


def setup_float(fmt, hq, hkv, d, bs, ctx, seed):
    shape, lay, case = make(fmt, hq, hkv, d, bs, ctx, seed=seed, spare_blocks=2,
                            poison_new=True)
    start = [host(case.k_cache).copy(), host(case.v_cache).copy()]
    slots = oracle.decode_slot_mapping(host(lay.block_tables), host(lay.context_lens), bs)
    want = [a.copy() for a in start]
    oracle.kv_append(host(case.k_new), host(case.v_new), slots, *want, bf16=fmt == "bf16")
    return shape, lay, case, start, want


@pytest.mark.parametrize("fmt,hq,hkv,d,bs", CASES)
@pytest.mark.parametrize("window", [1, 37, 1000, 0])
def test_decode_step_window_matches_oracle(fmt, hq, hkv, d, bs, window, orc):
    ctx = [1, 5, 40, 300, 1029, 2048]
    print(f"decode_step_window {fmt} hq={hq} hkv={hkv} d={d} bs={bs} w={window}", flush=True)
    quant = fmt in ("i8", "fp8", "i4")
    int4 = fmt == "i4"
    if quant:
        shape, lay, case, start, want = QS.setup(fmt, hq, hkv, d, bs, ctx, seed=9)
        pools = [QS.to_gpu(fmt, a) for a in start]
        scales = dict(k_scale=pools[2], v_scale=pools[3])
        oscales = dict(k_scale=want[2], v_scale=want[3])
    else:
        shape, lay, case, start, want = setup_float(fmt, hq, hkv, d, bs, ctx, seed=9)
        if fmt == "bf16":   # host copies hold the bf16 bit patterns as uint16
            pools = [torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
                     for a in start]
        else:
            pools = [torch.from_numpy(a).to(dev()) for a in start]
        scales, oscales = {}, {}
    q, kn, vn, bt, ctx_t = to_dev(case.q, case.k_new, case.v_new, lay.block_tables,
                                  lay.context_lens)
    out = torch.full_like(q, float("nan"))
    pa.decode_step_window(q, kn, vn, pools[0], pools[1], bt, ctx_t, shape.scale, window, out,
                          int4=int4, **scales)
    torch.cuda.synchronize()
    for got, exp in zip(pools, want):
        assert host(got).tobytes() == np.ascontiguousarray(exp).tobytes()
    ref = oracle.paged_decode_attention_window(
        host(case.q), want[0], want[1], host(lay.block_tables), host(lay.context_lens),
        shape.scale, window, bf16=fmt == "bf16", int4=int4, num_threads=8, lib=orc, **oscales)
    assert torch.isfinite(out).all()
    assert max_abs_err(out, ref) <= TOL["i8" if int4 else fmt]


def test_decode_step_window_full_size(orc):
    """The benchmark's windowed step at full size: Llama-3-8B layer shape
    (32 q / 8 KV heads, fp16, block 16), 16 sequences of 16384 positions, a
    4096-token window, the library's plan; the new rows bit-exact, sampled
    outputs within tolerance."""
    ctx = [16384] * 16
    bs = 16
    print("decode_step_window full size", flush=True)
    shape, lay, case = make("f16", 32, 8, 128, bs, ctx, seed=19, spare_blocks=0,
                            poison_new=True)
    kh, vh = host(case.k_cache).copy(), host(case.v_cache).copy()
    q, kc, vc, kn, vn, bt, ctx_t = to_dev(case.q, case.k_cache, case.v_cache, case.k_new,
                                          case.v_new, lay.block_tables, lay.context_lens)
    out = torch.empty_like(q)
    pa.decode_step_window(q, kn, vn, kc, vc, bt, ctx_t, shape.scale, 4096, out)
    torch.cuda.synchronize()
    slots = oracle.decode_slot_mapping(host(lay.block_tables), host(lay.context_lens), bs)
    oracle.kv_append(host(case.k_new), host(case.v_new), slots, kh, vh)
    b, o = torch.as_tensor(slots // bs), torch.as_tensor(slots % bs)
    assert np.array_equal(host(kc[b.to(dev()), :, o.to(dev())]), kh[slots // bs, :, slots % bs])
    assert np.array_equal(host(vc[b.to(dev()), :, o.to(dev())]), vh[slots // bs, :, slots % bs])
    rng = np.random.default_rng(13)
    pairs = [(s, 0) for s in range(16)] + [(int(rng.integers(16)), int(rng.integers(32)))
                                           for _ in range(16)]
    ref = oracle.paged_decode_attention_window(
        host(case.q), kh, vh, host(lay.block_tables), host(lay.context_lens), shape.scale, 4096,
        pairs=pairs, num_threads=8, lib=orc)
    assert torch.isfinite(out).all()
    assert max_abs_err(out, ref, pairs) <= TOL["f16"]
