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


# Unit roundoff of the operand/output format.
UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
LONG_ROW = 128      # rows that see at least this many positions meet the plain tolerance


def abs_pool(vp, fmt):
    """|V| in the pool's own format (clearing the sign bit is exact; NaN stays NaN)."""
    return np.abs(vp) if fmt == "f16" else (vp & np.uint16(0x7FFF))


def visible(qs, ctx):
    """Positions each query row attends to: token i of a chunk of T tokens of
    a context of c sits at position c - T + i and sees c - T + i + 1 rows."""
    n = [c - (qs[s + 1] - qs[s]) + 1 + np.arange(qs[s + 1] - qs[s])
         for s, c in enumerate(ctx)]
    return np.concatenate(n) if n else np.zeros(0, np.int64)


def within(got, ref, ref_abs_v, vis, fmt):
    """Per-element bound of the GPU output against the fp64 oracle.

    The kernel rounds each softmax weight w_i to the operand format before the
    value product (relative error <= u) and normalises by the sum of those
    same rounded weights, so the result is an exact weighted mean of V with
    perturbed weights: |error| <= u * sum_i wbar_i |v_i - out| <=
    u * (sum_i wbar_i |v_i| + |out|).  Rounding the output adds <= u |out|.
    sum_i wbar_i |v_i| is the oracle run once more on |V| (ref_abs_v).  The
    brief's max-abs tolerance covers the fp32 accumulation and exp; a row
    near the start of a prompt averages few value rows, so the relative
    terms are what matter there.  Rows that see LONG_ROW or more positions
    must meet the plain tolerance."""
    bound = TOL[fmt] + UNIT[fmt] * (2.0 * np.abs(ref) + ref_abs_v)
    long_rows = np.broadcast_to((vis >= LONG_ROW).reshape(vis.shape + (1,) * (ref.ndim - 1)),
                                bound.shape)
    bound = np.where(long_rows, TOL[fmt], bound)
    err = np.abs(got - ref)
    worst_long = float(err[long_rows].max()) if long_rows.any() else 0.0
    return bool(np.all(err <= bound)), float(err.max()), worst_long


def oracle_pair(q, kp, vp, bt, qs, ctx, scale, fmt, orc, rows=None):
    """The oracle's output and its output over |V| (same weights)."""
    kw = dict(bf16=fmt == "bf16", num_threads=0, lib=orc)
    if rows is not None:
        kw["rows"] = rows
    ref = oracle.paged_prefill_attention(q, kp, vp, bt, qs, ctx, scale, **kw)
    ref_abs = oracle.paged_prefill_attention(q, kp, abs_pool(vp, fmt), bt, qs, ctx, scale, **kw)
    return ref, ref_abs


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
    ref, ref_abs = oracle_pair(q, kp, vp, bt, qs, ctx_a, scale, fmt, orc)
    assert np.isfinite(got).all()
    ok, err, err_long = within(got, ref, ref_abs, visible(qs, ctx_a), fmt)
    assert ok, (err, err_long)


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
def test_one_token_chunks_match_decode(fmt, orc):
    """T = 1 is a decode step: the prefill rows and the decode kernel's rows
    each within their bound of the oracle."""
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
    ref, ref_abs = oracle_pair(q, kp, vp, bt, qs, ctx_a, scale, fmt, orc)
    ok, err, err_long = within(got, ref, ref_abs, visible(qs, ctx_a), fmt)
    assert ok, (err, err_long)
    assert np.max(np.abs(dec - ref)) <= TOL[fmt]


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
    after 3584 cached positions.  Every query head of 100 tokens (the first,
    second and last of each prompt and of the chunk, and 80 drawn at random)
    against the oracle: all rows would take the fp64 oracle minutes."""
    rng = np.random.default_rng(10)
    hq, hkv, d, bs = 32, 8, 128, 16
    ctx, tq = [2048, 2048, 2048, 2048, 4096], [2048, 2048, 2048, 2048, 512]
    kp, vp, bt, qs, ctx_a, q = make_batch(rng, "f16", ctx, tq, hq, hkv, d, bs)
    scale = 1.0 / np.sqrt(d)
    got = run_gpu("f16", kp, vp, bt, qs, ctx_a, q, scale)
    total = int(qs[-1])
    toks = {int(qs[s]) + i for s in range(len(ctx)) for i in (0, 1)} | {int(t) - 1 for t in qs[1:]}
    toks |= {int(t) for t in rng.choice(total, 100 - len(toks), replace=False)}
    toks = sorted(toks)[:100]
    rows = [(t, h) for t in toks for h in range(hq)]
    ref, ref_abs = oracle_pair(q, kp, vp, bt, qs, ctx_a, scale, "f16", orc, rows=rows)
    g = np.stack([got[t, h] for t, h in rows])
    vis = visible(qs, ctx_a)[[t for t, _ in rows]]
    assert np.isfinite(got).all()
    ok, err, err_long = within(g, ref, ref_abs, vis, "f16")
    assert ok, (err, err_long)


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
