"""The Python binding rejects mismatched pools and scales with ValueError
before any pointer reaches the library (no GPU needed: the checks run on the
tensors' shapes and dtypes, ahead of the device check).  The library sizes
both pools from one descriptor built from k_cache, so a V pool or a scale
tensor that is smaller than the K pool would otherwise be read or written
past its end on the GPU."""
import os

import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa

NB, HKV, BS, D, S, HQ = 6, 2, 16, 64, 2, 4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(pa.LIBRARY_PATH):
        pytest.fail("libpagedattn.so not built (python -m decode_attention_paged_append_amd.build)")


def pools(dtype, int4=False, nb=NB):
    w = D // 2 if int4 else D
    k = torch.zeros((nb, HKV, BS, w), dtype=dtype)
    return k, k.clone()


def scales(int4=False, nb=NB):
    shape = (nb, HKV, BS, D // 32) if int4 else (nb, HKV, BS)
    s = torch.zeros(shape, dtype=torch.float16)
    return s, s.clone()


def batch(qdtype=torch.float16):
    q = torch.zeros((S, HQ, D), dtype=qdtype)
    bt = torch.zeros((S, 3), dtype=torch.int32)
    ctx = torch.ones(S, dtype=torch.int32)
    return q, bt, ctx, torch.zeros_like(q)


class rejects:
    """pytest.raises(ValueError, match=what) that also fails when the error is
    the device check's (every tensor here is on the host), so a pass means the
    shape / dtype check fired first."""

    def __init__(self, what):
        self.ctx = pytest.raises(ValueError, match=what)

    def __enter__(self):
        self.info = self.ctx.__enter__()
        return self.info

    def __exit__(self, *exc):
        handled = self.ctx.__exit__(*exc)
        assert "GPU tensor" not in str(self.info.value), self.info.value
        return handled


QUANT = [(torch.int8, False), (torch.float8_e4m3fn, False), (torch.uint8, True)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_plain_calls_reject_a_smaller_or_other_v_pool(dtype):
    q, bt, ctx, out = batch(dtype)
    k, _ = pools(dtype)
    for v, what in ((pools(dtype, nb=NB - 1)[1], "v_cache"),
                    (torch.zeros_like(k, dtype=torch.float32 if dtype != torch.float32
                                      else torch.float16), "v_cache")):
        with rejects(what):
            pa.paged_decode_attention(q, k, v, bt, ctx, 0.1, out)
        with rejects(what):
            pa.decode_step(q, q[:, :HKV], q[:, :HKV], k, v, bt, ctx, 0.1, out)
        with rejects(what):
            pa.decode_partitions(q, k, v, bt, ctx, 0.1, out, 64, None)
        with rejects(what):
            pa.decode_step_partitions(q, q[:, :HKV], q[:, :HKV], k, v, bt, ctx, 0.1, out, 64,
                                      None)
        with rejects(what):
            pa.paged_decode_attention_window(q, k, v, bt, ctx, 0.1, 8, out)
        with rejects(what):
            pa.decode_step_window(q, q[:, :HKV], q[:, :HKV], k, v, bt, ctx, 0.1, 8, out)
        with rejects(what):
            pa.kv_append(q[:, :HKV], q[:, :HKV], torch.zeros(S, dtype=torch.int64), k, v)
        with rejects(what):
            pa.copy_blocks(k, v, np.array([[0, 1]], np.int32))
        with rejects(what):
            pa.gather_kv(k, v, bt, ctx, torch.zeros((S, 48, HKV, D), dtype=dtype),
                         torch.zeros((S, 48, HKV, D), dtype=dtype))
        if dtype != torch.float32:
            with rejects(what):
                pa.paged_prefill_attention(q, k, v, bt, torch.tensor([0, 1, 2], dtype=torch.int32),
                                           ctx, 0.1, out, max_query_len=1)


@pytest.mark.parametrize("dtype,int4", QUANT)
def test_quantized_calls_reject_bad_pools_and_scales(dtype, int4):
    q, bt, ctx, out = batch()
    k, v = pools(dtype, int4)
    ks, vs = scales(int4)
    kn = torch.zeros((S, HKV, D), dtype=torch.float16)
    short_v = pools(dtype, int4, nb=NB - 1)[1]
    short_s = scales(int4, nb=NB - 1)[1]
    other = scales(not int4)[1]            # per-row scales for int4, per-group for int8 / fp8
    cases = [(short_v, ks, vs, "v_cache"), (k, ks, short_s, "v_scale"), (k, short_s, vs, "k_scale"),
             (k, other, vs, "k_scale"), (k, ks, vs.to(torch.float32), "v_scale"),
             (k, None, vs, "k_scale"), (k, ks, None, "v_scale")]
    attend = {torch.int8: pa.paged_decode_attention_int8,
              torch.float8_e4m3fn: pa.paged_decode_attention_fp8,
              torch.uint8: pa.paged_decode_attention_int4}[dtype]
    append = {torch.int8: pa.kv_append_int8, torch.float8_e4m3fn: pa.kv_append_fp8,
              torch.uint8: pa.kv_append_int4}[dtype]
    for vv, a, b, what in cases:
        with rejects(what):
            attend(q, k, vv, a, b, bt, ctx, 0.1, out)
        with rejects(what):
            append(kn, kn, torch.zeros(S, dtype=torch.int64), k, vv, a, b)
        with rejects(what):
            pa.decode_step_quant(q, kn, kn, k, vv, a, b, bt, ctx, 0.1, out, int4=int4)
        with rejects(what):
            pa.decode_step_partitions_quant(q, kn, kn, k, vv, a, b, bt, ctx, 0.1, out, 64, None,
                                            int4=int4)
        with rejects(what):
            pa.decode_partitions(q, k, vv, bt, ctx, 0.1, out, 64, None, a, b, int4=int4)
        with rejects(what):
            pa.paged_decode_attention_window(q, k, vv, bt, ctx, 0.1, 8, out, a, b, int4=int4)
        with rejects(what):
            pa.decode_step_window(q, kn, kn, k, vv, bt, ctx, 0.1, 8, out, a, b, int4=int4)
        with rejects(what):
            pa.copy_blocks(k, vv, np.array([[0, 1]], np.int32), a, b, int4=int4)


@pytest.mark.parametrize("dtype,int4", QUANT)
def test_gather_checks_scale_outputs(dtype, int4):
    k, v = pools(dtype, int4)
    ks, vs = scales(int4)
    _, bt, ctx, _ = batch()
    w = k.shape[3]
    ko, vo = torch.zeros((S, 48, HKV, w), dtype=dtype), torch.zeros((S, 48, HKV, w), dtype=dtype)
    good = (S, 48, HKV) + ((D // 32,) if int4 else ())
    bad = torch.zeros((S, 47) + good[2:], dtype=torch.float16)
    with rejects("k_scale_out"):
        pa.gather_kv(k, v, bt, ctx, ko, vo, ks, vs, bad, torch.zeros(good, dtype=torch.float16),
                     int4=int4)
    with rejects("go together"):
        pa.gather_kv(k, v, bt, ctx, ko, vo, ks, vs, torch.zeros(good, dtype=torch.float16), None,
                     int4=int4)


def test_workspace_size_is_passed_in_bytes():
    """A workspace of any dtype is sized by its bytes, not its element count."""
    assert pa._nbytes(torch.zeros(10, dtype=torch.float32)) == 40
    assert pa._nbytes(torch.zeros(10, dtype=torch.uint8)) == 10
    assert pa._nbytes(None) == 0
