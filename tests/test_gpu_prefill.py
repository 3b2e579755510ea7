"""Prefill / chunked-prefill attention on the GPU against the fp64 oracle
(needs an MI355X).  Pools are built on the host (random N(0,1) rows placed at
random blocks, everything else NaN) and copied to the GPU, so the oracle's
inputs never come from the HIP path."""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
from gpu_cases import TOL, dev

pytestmark = pytest.mark.gpu

NP = {"f16": np.float16, "bf16": np.uint16}
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def to_fmt(x: np.ndarray, fmt: str) -> np.ndarray:
    """float32 -> the format's host array (bf16 as uint16 bits, RNE)."""
    if fmt == "f16":
        return x.astype(np.float16)
    b = x.astype(np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def to_gpu(a: np.ndarray, fmt: str):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if fmt == "bf16" else t).to(dev())


def make_batch(rng, fmt, ctx, tq, hq, hkv, d, bs, spare_blocks=8):
    """Host pool with each sequence's ctx rows at random blocks; q for the
    last tq positions of each."""
    need = [-(-c // bs) for c in ctx]
    nb = sum(need) + spare_blocks
    maxb = max(need)
    poison = np.float16(np.nan) if fmt == "f16" else np.uint16(0x7FC0)
    kp = np.full((nb, hkv, bs, d), poison, dtype=NP[fmt])
    vp = np.full_like(kp, poison)
    bt = np.full((len(ctx), maxb), -1, np.int32)
    perm = rng.permutation(nb)
    cur = 0
    for s, c in enumerate(ctx):
        k = to_fmt(rng.standard_normal((c, hkv, d)).astype(np.float32), fmt)
        v = to_fmt(rng.standard_normal((c, hkv, d)).astype(np.float32), fmt)
        for j in range(need[s]):
            b = perm[cur]
            cur += 1
            bt[s, j] = b
            lo, hi = j * bs, min((j + 1) * bs, c)
            kp[b, :, :hi - lo] = np.transpose(k[lo:hi], (1, 0, 2))
            vp[b, :, :hi - lo] = np.transpose(v[lo:hi], (1, 0, 2))
    qs = np.concatenate([[0], np.cumsum(tq)]).astype(np.int32)
    q = to_fmt(rng.standard_normal((int(qs[-1]), hq, d)).astype(np.float32), fmt)
    return kp, vp, bt, qs, np.array(ctx, np.int32), q


# Unit roundoff of the operand/output format.  A prefill row near the start of
# a prompt averages few value rows, so |out| is close to |v| rather than the
# ~sqrt(e/ctx) of a long decode context that the absolute tolerances assume;
# rounding the output (<= u |out|) and the softmax weights fed to the matrix
# cores (<= u sum_i w_i |v_i| <= u max|v|) then add a relative term.
UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def within(got, ref, fmt, vmax):
    """Max-abs tolerance plus twice the format's rounding of out and weights."""
    bound = TOL[fmt] + 2 * UNIT[fmt] * (np.abs(ref) + vmax)
    return bool(np.all(np.abs(got - ref) <= bound)), float(np.max(np.abs(got - ref)))


def vmax_of(vp, fmt):
    v = vp.astype(np.float32) if fmt == "f16" else (vp.astype(np.uint32) << 16).view(np.float32)
    return float(np.nanmax(np.abs(v)))


def run_gpu(fmt, kp, vp, bt, qs, ctx, q, scale, max_query_len=None):
    qg = to_gpu(q, fmt)
    out = torch.full_like(qg, float("nan"))
    pa.paged_prefill_attention(qg, to_gpu(kp, fmt), to_gpu(vp, fmt),
                               torch.from_numpy(bt).to(dev()), torch.from_numpy(qs).to(dev()),
                               torch.from_numpy(ctx).to(dev()), scale, out, max_query_len)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


CASES = [  # (ctx, chunk lengths): whole prompts, chunks after a cached prefix, mixed
    ([1, 5, 17, 64, 130], [1, 5, 17, 64, 130]),
    ([300, 40, 97], [300, 12, 33]),
    ([33, 160, 7, 260], [1, 160, 7, 100]),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [4, 16, 32])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (16, 2)])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_matches_oracle(fmt, d, bs, hq, hkv, case, orc):
    ctx, tq = CASES[case]
    rng = np.random.default_rng(1000 * case + 10 * hq + bs + d)
    kp, vp, bt, qs, ctx_a, q = make_batch(rng, fmt, ctx, tq, hq, hkv, d, bs)
    scale = 1.0 / np.sqrt(d)
    print(f"prefill {fmt} d={d} bs={bs} hq={hq} hkv={hkv} case={case}", flush=True)
    got = run_gpu(fmt, kp, vp, bt, qs, ctx_a, q, scale)
    ref = oracle.paged_prefill_attention(q, kp, vp, bt, qs, ctx_a, scale, bf16=fmt == "bf16",
                                         num_threads=8, lib=orc)
    assert np.isfinite(got).all()
    ok, err = within(got, ref, fmt, vmax_of(vp, fmt))
    assert ok, err


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_chunked_equals_whole_prompt_bit_exact(fmt):
    """A prompt taken in chunks gives the rows of one whole prefill bit for
    bit: a row's arithmetic depends only on its position."""
    rng = np.random.default_rng(7)
    hq, hkv, d, bs, n = 32, 8, 128, 16, 600
    kp, vp, bt, _, _, q = make_batch(rng, fmt, [n], [n], hq, hkv, d, bs)
    scale = 1.0 / np.sqrt(d)
    whole = run_gpu(fmt, kp, vp, bt, np.array([0, n], np.int32), np.array([n], np.int32), q,
                    scale)
    done = 0
    for t in (100, 260, 1, 239):
        part = run_gpu(fmt, kp, vp, bt, np.array([0, t], np.int32),
                       np.array([done + t], np.int32), q[done:done + t], scale)
        assert np.array_equal(part, whole[done:done + t])
        done += t
    assert done == n


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_one_token_chunks_match_decode(fmt):
    """T = 1 is a decode step: same rows as the decode kernel, within tolerance."""
    rng = np.random.default_rng(8)
    hq, hkv, d, bs = 32, 8, 128, 16
    ctx = [1, 17, 500, 2049]
    kp, vp, bt, qs, ctx_a, q = make_batch(rng, fmt, ctx, [1] * 4, hq, hkv, d, bs)
    scale = 1.0 / np.sqrt(d)
    got = run_gpu(fmt, kp, vp, bt, qs, ctx_a, q, scale)
    out = torch.empty((4, hq, d), dtype=TORCH[fmt], device=dev())
    pa.paged_decode_attention(to_gpu(q, fmt), to_gpu(kp, fmt), to_gpu(vp, fmt),
                              torch.from_numpy(bt).to(dev()), torch.from_numpy(ctx_a).to(dev()),
                              scale, out)
    torch.cuda.synchronize()
    dec = out.double().cpu().numpy()
    ok, err = within(got, dec, fmt, 2 * vmax_of(vp, fmt))
    assert ok, err


def test_bad_context_gives_nan_rows():
    rng = np.random.default_rng(9)
    kp, vp, bt, qs, ctx_a, q = make_batch(rng, "f16", [40, 40], [10, 10], 8, 2, 64, 16)
    ctx_a[1] = 5                                   # shorter than its chunk
    got = run_gpu("f16", kp, vp, bt, qs, ctx_a, q, 0.125)
    assert np.isfinite(got[:10]).all() and np.isnan(got[10:]).all()


def test_prefill_argument_checks():
    f = torch.zeros((4, 8, 64), dtype=torch.float16, device=dev())
    kc = torch.zeros((8, 2, 16, 64), dtype=torch.float16, device=dev())
    bt = torch.zeros((1, 4), dtype=torch.int32, device=dev())
    qs = torch.tensor([0, 4], dtype=torch.int32, device=dev())
    ctx = torch.tensor([4], dtype=torch.int32, device=dev())
    with pytest.raises(pa.PagedAttnError, match="fp16 or bf16"):
        pa.paged_prefill_attention(f.float(), kc.float(), kc.float(), bt, qs, ctx, 0.1,
                                   f.float(), 4)
    with pytest.raises(pa.PagedAttnError, match="divide"):
        pa.paged_prefill_attention(f[:, :3].contiguous(), kc, kc, bt, qs, ctx, 0.1,
                                   f[:, :3].contiguous(), 4)
    pa.paged_prefill_attention(f, kc, kc, bt, qs, ctx, 0.1, f, 0)   # nothing to do


def test_full_size_sampled_rows(orc):
    """Llama-3-8B layer shape: 4 prompts of 2048 tokens plus a 512-token chunk
    after 3584 cached positions, checked on sampled rows."""
    rng = np.random.default_rng(10)
    hq, hkv, d, bs = 32, 8, 128, 16
    ctx, tq = [2048, 2048, 2048, 2048, 4096], [2048, 2048, 2048, 2048, 512]
    kp, vp, bt, qs, ctx_a, q = make_batch(rng, "f16", ctx, tq, hq, hkv, d, bs)
    scale = 1.0 / np.sqrt(d)
    got = run_gpu("f16", kp, vp, bt, qs, ctx_a, q, scale)
    total = int(qs[-1])
    rows = [(t, h) for t in (0, 1, 2047, 2048, total - 512, total - 1) for h in (0, hq - 1)]
    rows += [(int(rng.integers(total)), int(rng.integers(hq))) for _ in range(40)]
    ref = oracle.paged_prefill_attention(q, kp, vp, bt, qs, ctx_a, scale, rows=rows,
                                         num_threads=8, lib=orc)
    g = np.stack([got[t, h] for t, h in rows])
    assert np.isfinite(got).all()
    ok, err = within(g, ref, "f16", vmax_of(vp, "f16"))
    assert ok, err


def test_tokens_past_max_query_len_are_not_written():
    """max_query_len bounds the grid: a longer chunk's first max_query_len
    tokens are computed exactly as in a full call, the rest of its rows keep
    what out held (the documented contract)."""
    rng = np.random.default_rng(11)
    kp, vp, bt, qs, ctx_a, q = make_batch(rng, "f16", [300, 70], [40, 10], 16, 2, 128, 16)
    full = run_gpu("f16", kp, vp, bt, qs, ctx_a, q, 0.1)
    part = run_gpu("f16", kp, vp, bt, qs, ctx_a, q, 0.1, max_query_len=16)
    assert np.array_equal(part[:16], full[:16])          # sequence 0, tokens 0..15
    assert np.isnan(part[16:40]).all()                   # past the bound: untouched (NaN fill)
    assert np.array_equal(part[40:], full[40:])          # sequence 1 fits the bound
