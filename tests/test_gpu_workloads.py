"""Parity at the full sizes of the benchmark workloads (one layer each), in the
launch configuration the benchmark times (the library's own plan): every
(sequence, head) output element-wise against the fp64 oracle (run on all host
cores), and bit-exact on the slots, the appended rows and, for the int8
cache, every code and scale of the pool (needs an MI355X)."""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
import workloads as W
from gpu_cases import (TOL, decode_gpu, dev, host, max_abs_err, quantize_blocks_oracle,
                       quantize_pool_gpu)

pytestmark = pytest.mark.gpu


def same_bytes(a: np.ndarray, b: np.ndarray) -> bool:
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


def append_then_decode(shape, layer_seed=0):
    lay = W.layout_for(shape)
    case = W.make_case(shape, lay, device=dev(), seed=layer_seed, poison=True,
                       poison_new_slot=True)
    kh, vh = host(case.k_cache).copy(), host(case.v_cache).copy()   # before the append
    bt, ctx = lay.block_tables.to(dev()), lay.context_lens.to(dev())
    slots = pa.decode_slot_mapping(bt, ctx, shape.block_size)
    pa.kv_append(case.k_new, case.v_new, slots, case.k_cache, case.v_cache)
    out = decode_gpu(case.q, case.k_cache, case.v_cache, bt, ctx, shape.scale)
    # oracle: its own slots and append on the host copy, then attention
    oslots = oracle.decode_slot_mapping(host(lay.block_tables), host(lay.context_lens),
                                        shape.block_size)
    assert (slots.cpu().numpy() == oslots).all()
    oracle.kv_append(host(case.k_new), host(case.v_new), oslots, kh, vh,
                     bf16=shape.cache_dtype == "bf16")
    assert same_bytes(host(case.k_cache), kh) and same_bytes(host(case.v_cache), vh)
    ref = oracle.paged_decode_attention(host(case.q), kh, vh, host(lay.block_tables),
                                        host(lay.context_lens), shape.scale,
                                        bf16=shape.cache_dtype == "bf16")
    return max_abs_err(out, ref), out


def test_llama3_8b_fp16_append_and_decode():
    err, out = append_then_decode(W.LLAMA3_8B)
    assert err <= TOL["f16"], err
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("layer", [0, 31])
def test_llama2_7b_fp16_append_and_decode(layer):
    err, out = append_then_decode(W.LLAMA2_7B, layer_seed=layer)
    assert err <= TOL["f16"], err
    assert torch.isfinite(out).all()


def test_llama2_70b_bf16_shared_prefix_decode():
    shape = W.LLAMA2_70B
    lay = W.layout_for(shape)
    assert int(lay.owners.max()) == W.PREFIX_GROUP        # prefix blocks serve 8 tables
    case = W.make_case(shape, lay, device=dev(), poison=True, poison_new_slot=False)
    bt, ctx = lay.block_tables.to(dev()), lay.context_lens.to(dev())
    out = decode_gpu(case.q, case.k_cache, case.v_cache, bt, ctx, shape.scale)
    assert torch.isfinite(out).all()
    ref = oracle.paged_decode_attention(host(case.q), host(case.k_cache), host(case.v_cache),
                                        host(lay.block_tables), host(lay.context_lens),
                                        shape.scale, bf16=True)
    assert max_abs_err(out, ref) <= TOL["bf16"]


def test_llama3_8b_int8_quantized_decode():
    shape = W.LLAMA3_8B_I8
    lay = W.layout_for(shape)
    case = W.make_case(shape, lay, device=dev(), poison=False)
    kq, vq, ks, vs = quantize_pool_gpu(case.k_cache, case.v_cache, None)
    blocks = lay.block_tables.flatten()
    okq, ovq, oks, ovs, used = quantize_blocks_oracle(case.k_cache, case.v_cache, blocks[blocks >= 0])
    assert len(used) == lay.num_blocks                  # every pool block is some sequence's
    assert same_bytes(host(kq), okq) and same_bytes(host(vq), ovq)
    assert same_bytes(host(ks), oks) and same_bytes(host(vs), ovs)
    bt, ctx = lay.block_tables.to(dev()), lay.context_lens.to(dev())
    out = decode_gpu(case.q, kq, vq, bt, ctx, shape.scale, None, ks, vs)
    ref = oracle.paged_decode_attention(host(case.q), okq, ovq, host(lay.block_tables),
                                        host(lay.context_lens), shape.scale, k_scale=oks,
                                        v_scale=ovs)
    assert max_abs_err(out, ref) <= TOL["i8"]


@pytest.mark.parametrize("shape", [W.LLAMA2_7B, W.LLAMA3_8B], ids=lambda s: s.name)
def test_decode_step_full_size(shape):
    """The benchmark's step at full size: append fused into the attention
    launch (library plan), then the merge launch."""
    lay = W.layout_for(shape)
    case = W.make_case(shape, lay, device=dev(), seed=3, poison=True, poison_new_slot=True)
    kh, vh = host(case.k_cache).copy(), host(case.v_cache).copy()
    bt, ctx = lay.block_tables.to(dev()), lay.context_lens.to(dev())
    out = torch.empty_like(case.q)
    pa.decode_step(case.q, case.k_new, case.v_new, case.k_cache, case.v_cache, bt, ctx,
                   shape.scale, out)
    torch.cuda.synchronize()
    oslots = oracle.decode_slot_mapping(host(lay.block_tables), host(lay.context_lens),
                                        shape.block_size)
    oracle.kv_append(host(case.k_new), host(case.v_new), oslots, kh, vh)
    assert same_bytes(host(case.k_cache), kh) and same_bytes(host(case.v_cache), vh)
    ref = oracle.paged_decode_attention(host(case.q), kh, vh, host(lay.block_tables),
                                        host(lay.context_lens), shape.scale)
    assert max_abs_err(out, ref) <= TOL["f16"]
