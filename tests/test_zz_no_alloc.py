"""pa_decode_step_noalloc (no workspace: the partials go to the library's
static device scratch) against pa_decode_step with a caller workspace, called
through the C ABI: two calls in a row on each kernel family, the second with
a smaller input than the first (the scratch then still holds the first
call's partials), each bit-equal to the workspace path in output and pool and
within tolerance of the oracle (needs an MI355X)."""
import ctypes

import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
import workloads as W
from gpu_cases import TOL, dev, host

pytestmark = pytest.mark.gpu

# (format, q heads, KV heads, head_dim, block, contexts of call 1, contexts of call 2):
# vector ALU (G = 1, 2) and matrix cores (G = 4, 8), every call multi-partition
CASES = [
    ("f16", 32, 32, 128, 16, [4096, 3000, 1, 2500, 4096, 17, 999, 4000], [700, 5, 1200]),
    ("bf16", 16, 8, 64, 8, [3000, 2047, 64, 5000], [900, 333]),
    ("f16", 32, 8, 128, 16, [4096] * 16, [2048, 1500, 777]),
    ("bf16", 64, 8, 128, 32, [9000, 20000, 128, 4096], [3000, 100]),
    ("f32", 8, 2, 64, 16, [1500, 4000, 3], [600]),
]


def make(fmt, hq, hkv, d, bs, ctx, seed):
    shape = W.Shape(f"noalloc-{fmt}", fmt, len(ctx), hq, hkv, d, bs)
    need = sum(W.blocks_needed(c, bs) for c in ctx)
    lay = W.carve_layout(ctx, bs, num_blocks=need + 4, seed=seed + 1)
    case = W.make_case(shape, lay, seed=seed, poison=True, poison_new_slot=True)
    return shape, lay, case


def c_step_noalloc(q, kn, vn, kc, vc, bt, ctx, scale, out):
    """The entry point called directly through ctypes (no binding checks)."""
    lib = pa.library()
    desc = pa.CacheDesc.of(kc)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    return lib.pa_decode_step_noalloc(
        q.data_ptr(), kn.data_ptr(), vn.data_ptr(), kc.data_ptr(), vc.data_ptr(),
        bt.data_ptr(), bt.shape[1], ctx.data_ptr(), q.shape[0], q.shape[1], float(scale),
        out.data_ptr(), ctypes.byref(desc), stream)


@pytest.mark.parametrize("case_i", range(len(CASES)))
def test_noalloc_step_equals_workspace_step(case_i, orc):
    fmt, hq, hkv, d, bs, ctx1, ctx2 = CASES[case_i]
    for call, ctx in enumerate((ctx1, ctx2)):
        print(f"noalloc {fmt} hq={hq} hkv={hkv} d={d} bs={bs} call={call} ctx={ctx}", flush=True)
        shape, lay, case = make(fmt, hq, hkv, d, bs, ctx, seed=10 * case_i + call)
        s = len(ctx)
        maxb = lay.max_blocks
        desc = pa.CacheDesc.of(case.k_cache)
        assert pa.decode_workspace_bytes(desc, s, hq, maxb) > 0     # multi-partition: scratch used
        q, kn, vn, bt, ctx_t = (t.to(dev()).contiguous() for t in (
            case.q, case.k_new, case.v_new, lay.block_tables, lay.context_lens))
        kc_a, vc_a = case.k_cache.to(dev()), case.v_cache.to(dev())
        kc_b, vc_b = kc_a.clone(), vc_a.clone()
        ref = torch.empty_like(q)
        pa.decode_step(q, kn, vn, kc_a, vc_a, bt, ctx_t, shape.scale, ref)
        got = torch.full_like(q, float("nan"))
        assert c_step_noalloc(q, kn, vn, kc_b, vc_b, bt, ctx_t, shape.scale, got) == 0, \
            pa.library().pa_last_error()
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert torch.equal(kc_b.view(torch.uint8), kc_a.view(torch.uint8))
        assert torch.equal(vc_b.view(torch.uint8), vc_a.view(torch.uint8))
        # and the oracle: its own slots and append, then attention
        kh, vh = host(case.k_cache).copy(), host(case.v_cache).copy()
        slots = oracle.decode_slot_mapping(host(lay.block_tables), host(lay.context_lens), bs)
        oracle.kv_append(host(case.k_new), host(case.v_new), slots, kh, vh, bf16=fmt == "bf16")
        want = oracle.paged_decode_attention(host(case.q), kh, vh, host(lay.block_tables),
                                             host(lay.context_lens), shape.scale,
                                             bf16=fmt == "bf16", lib=orc)
        err = float(np.max(np.abs(got.double().cpu().numpy() - want)))
        assert err <= TOL[fmt], err


def test_noalloc_rejects_quantized_cache():
    kc = torch.zeros((4, 2, 16, 64), dtype=torch.int8, device=dev())
    q = torch.zeros((1, 4, 64), dtype=torch.float16, device=dev())
    bt = torch.zeros((1, 4), dtype=torch.int32, device=dev())
    ctx = torch.ones(1, dtype=torch.int32, device=dev())
    kn = torch.zeros((1, 2, 64), dtype=torch.float16, device=dev())
    status = c_step_noalloc(q, kn, kn, kc, kc, bt, ctx, 0.1, q.clone())
    assert status == 2 and b"quantized" in pa.library().pa_last_error()    # PA_ERR_UNSUPPORTED
