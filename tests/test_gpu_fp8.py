"""fp8 (OCP E4M3) caches on the GPU against the oracle (needs an MI355X):
the quantizing append bit-exact (codes and scales, ties included), and
decode attention over the same codes and scales within tolerance, in the
vector-ALU kernel (one or two query heads per KV head) and the matrix-core
kernel (four or more), at test sizes and at the full Llama-3-8B shape."""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
import workloads as W
from gpu_cases import (TOL, decode_gpu, dev, host, max_abs_err, quantize_blocks_oracle,
                       quantize_pool_gpu, tile_tokens)
from test_gpu_kernels import make, to_dev

pytestmark = pytest.mark.gpu

E4M3 = torch.float8_e4m3fn


def tie_row(d):
    """A row whose scale is exactly 2^-4 (max 28 = 448 * 2^-4), so that x / s
    = 16 x is exact and lands on every E4M3 midpoint: each must round to the
    code with an even last bit."""
    table = torch.arange(127, dtype=torch.uint8).view(E4M3).double().numpy()
    mids = (table[:-1] + table[1:]) / 2 / 16
    row = np.concatenate([[28.0], mids, -mids])[:d]
    return torch.from_numpy(row).to(torch.float16)


@pytest.mark.parametrize("d", [64, 128])
def test_kv_append_fp8_bit_exact(d):
    nb, hkv, bs = 10, 2, 16
    t = 40
    k_new = (torch.randn((t, hkv, d), generator=W.generator(19)) *
             torch.logspace(-4, 4, t)[:, None, None]).to(torch.float16)
    v_new = W.randn((t, hkv, d), "f16", 20)
    k_new[3] = 0                       # all-zero rows: scale 0, codes 0
    k_new[4, 0, :5] = torch.tensor([65504, -65504, 1e-7, 6e-8, -3.0])
    k_new[6, 1] = tie_row(d)
    v_new[7, 0] = tie_row(d)
    v_new[8, 1, 2] = float("nan")      # a NaN input encodes as 0
    slots = torch.randperm(nb * bs, generator=W.generator(21))[:t].to(torch.int64)
    slots[5] = -1
    slots[9] = nb * bs                 # outside the pool: skipped
    kq = torch.full((nb, hkv, bs, d), 0x7F, dtype=torch.uint8).view(E4M3)
    vq = kq.clone()
    ks = torch.full((nb, hkv, bs), float("nan"), dtype=torch.float16)
    vs = ks.clone()
    dk = to_dev(k_new, v_new, slots, kq, vq, ks, vs)
    print(f"kv_append_fp8 d={d}", flush=True)
    pa.kv_append_fp8(*dk)
    torch.cuda.synchronize()
    hq_, hv_, hks, hvs = host(kq).copy(), host(vq).copy(), host(ks).copy(), host(vs).copy()
    ok = slots.clone()
    ok[ok >= nb * bs] = -1
    oracle.kv_append_fp8(host(k_new), host(v_new), ok.numpy(), hq_, hv_, hks, hvs)
    assert host(dk[3]).tobytes() == hq_.tobytes()
    assert host(dk[4]).tobytes() == hv_.tobytes()
    assert host(dk[5]).view(np.uint16).tobytes() == hks.view(np.uint16).tobytes()
    assert host(dk[6]).view(np.uint16).tobytes() == hvs.view(np.uint16).tobytes()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [4, 16, 32])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (16, 2)])
def test_fp8_decode_matches_oracle(d, bs, hq, hkv):
    ctx = [1, bs + 3, 200, 513]
    shape, lay, case = make("fp8", hq, hkv, d, bs, ctx, seed=4, spare_blocks=2)
    src_k = case.k_cache.nan_to_num(0.0).to(dev())
    src_v = case.v_cache.nan_to_num(0.0).to(dev())
    print(f"fp8 decode d={d} bs={bs} hq={hq} hkv={hkv}", flush=True)
    kq, vq, ks, vs = quantize_pool_gpu(src_k, src_v, None, "fp8")
    okq, ovq, oks, ovs, _ = quantize_blocks_oracle(src_k, src_v, range(lay.num_blocks), "fp8")
    assert host(kq).tobytes() == okq.tobytes() and host(vq).tobytes() == ovq.tobytes()
    assert host(ks).tobytes() == oks.tobytes() and host(vs).tobytes() == ovs.tobytes()
    q, bt, ctx_t = to_dev(case.q, lay.block_tables, lay.context_lens)
    ref = oracle.paged_decode_attention(host(case.q), okq, ovq, host(lay.block_tables),
                                        host(lay.context_lens), shape.scale, k_scale=oks,
                                        v_scale=ovs)
    tile = tile_tokens("fp8", d, bs)
    for part in (None, tile, -(-lay.max_blocks * bs // tile) * tile):
        out = decode_gpu(q, kq, vq, bt, ctx_t, shape.scale, part, ks, vs)
        assert torch.isfinite(out).all()
        assert max_abs_err(out, ref) <= TOL["fp8"], part


def test_fp8_full_size():
    """Llama-3-8B layer, 64 sequences x 8192 positions in fp8, the library's
    own plan: the whole pool bit-exact against the oracle's quantizer and
    every (sequence, head) output within tolerance of the oracle."""
    shape = W.LLAMA3_8B_FP8
    lay = W.layout_for(shape)
    case = W.make_case(shape, lay, device=dev(), poison=False)
    print("fp8 full size", flush=True)
    kq, vq, ks, vs = quantize_pool_gpu(case.k_cache, case.v_cache, None, "fp8")
    okq, ovq, oks, ovs, _ = quantize_blocks_oracle(case.k_cache, case.v_cache,
                                                   range(lay.num_blocks), "fp8")
    assert host(kq).tobytes() == okq.tobytes() and host(vq).tobytes() == ovq.tobytes()
    assert host(ks).tobytes() == oks.tobytes() and host(vs).tobytes() == ovs.tobytes()
    bt, ctx = lay.block_tables.to(dev()), lay.context_lens.to(dev())
    out = decode_gpu(case.q, kq, vq, bt, ctx, shape.scale, None, ks, vs)
    ref = oracle.paged_decode_attention(host(case.q), okq, ovq, host(lay.block_tables),
                                        host(lay.context_lens), shape.scale, k_scale=oks,
                                        v_scale=ovs)
    assert torch.isfinite(out).all()
    assert max_abs_err(out, ref) <= TOL["fp8"]
