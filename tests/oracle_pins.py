"""Checks that tie the CPU oracle to facts fixed outside itself.

Each ``pin_*`` function takes an oracle library handle and raises
AssertionError when the oracle disagrees with what the pages or the
mathematics fix:
  - values the pages print (tests/golden/*.json, each with its citation),
  - closed forms and special cases of softmax attention,
  - library routines (numpy / torch float64) on tiny inputs,
  - invariances the pages state in words (blocks may sit anywhere in the pool;
    the cache changes the cost, never the result; GQA shares KV heads).
The same functions run against deliberately broken copies of the oracle in
test_oracle_mutations.py, which checks that every planted mistake is caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa64(q, K, V, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU (one query)."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).reshape(1, 1, 1, -1)
    Kt = torch.from_numpy(np.asarray(K, np.float64)).reshape(1, 1, K.shape[0], -1)
    Vt = torch.from_numpy(np.asarray(V, np.float64)).reshape(1, 1, V.shape[0], -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return o.reshape(-1).numpy()


def _scatter_pool(dense_k, dense_v, block_size, num_blocks, rng, dtype):
    """Place per-sequence dense rows into a pool at random blocks (test-side
    numpy indexing).  dense_*: list over seqs of [ctx, Hkv, D] float arrays.
    Returns pools [NB, Hkv, BS, D], block tables, context lengths."""
    hkv, d = dense_k[0].shape[1], dense_k[0].shape[2]
    need = [(-(-k.shape[0] // block_size)) for k in dense_k]
    maxb = max(max(need), 1)
    perm = rng.permutation(num_blocks)
    poison = 0x7FC0 if dtype == np.uint16 else np.nan     # bfloat16 bits travel as uint16
    kp = np.full((num_blocks, hkv, block_size, d), poison, dtype=dtype)
    vp = np.full_like(kp, poison)
    bt = np.full((len(dense_k), maxb), -1, np.int32)
    cur = 0
    for s, (k, v) in enumerate(zip(dense_k, dense_v)):
        for j in range(need[s]):
            b = perm[cur]
            cur += 1
            bt[s, j] = b
            rows = slice(j * block_size, min((j + 1) * block_size, k.shape[0]))
            n = rows.stop - rows.start
            kp[b, :, :n, :] = np.transpose(k[rows], (1, 0, 2))
            vp[b, :, :n, :] = np.transpose(v[rows], (1, 0, 2))
    ctx = np.array([k.shape[0] for k in dense_k], np.int32)
    return kp, vp, bt, ctx


# ---------------------------------------------------------------- formats

def pin_f16_decode_exhaustive(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([lib.oracle_f16_to_double(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"binary16 decode differs at {np.flatnonzero(~same)[:5]}"


def pin_bf16_decode_exhaustive(lib):
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([lib.oracle_bf16_to_double(int(b) & 0xFFFF) for b in bits.tolist()])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), "bfloat16 decode differs"


def pin_f16_encode(lib):
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        rng.uniform(0, 1e-4, 2000), rng.uniform(0, 1, 2000), rng.uniform(0, 70000, 2000),
        np.exp(rng.uniform(-20, 11, 2000)),
        # exact ties between two binary16 neighbours, half of them toward odd
        [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -24 * 1.5, 2.0 ** -24 * 2.5, 65504 + 8,
         2.0 ** -25, 2.0 ** -26, 0.0, 65519.99, 65520.0],
    ])
    ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([lib.oracle_double_to_f16_bits(float(x)) for x in xs], dtype=np.uint16)
    assert (got == ref).all(), f"binary16 rounding differs for {xs[got != ref][:5]}"


# ---------------------------------------------------------------- slots / append / gather

def pin_slot_mapping(lib):
    rng = np.random.default_rng(3)
    for bs in (1, 4, 16):
        s, maxb = 5, 6
        bt = rng.integers(0, 100, size=(s, maxb)).astype(np.int32)
        seq = rng.integers(0, s, size=40).astype(np.int32)
        pos = rng.integers(0, maxb * bs, size=40).astype(np.int32)
        got = oracle.slot_mapping(bt, seq, pos, bs, lib=lib)
        for t in range(40):
            blk, off = divmod(int(pos[t]), bs)
            assert got[t] == int(bt[seq[t], blk]) * bs + off
        ctx = rng.integers(0, maxb * bs + 1, size=s).astype(np.int32)
        ctx[0] = 0
        got = oracle.decode_slot_mapping(bt, ctx, bs, lib=lib)
        for i in range(s):
            if ctx[i] == 0:
                assert got[i] == -1
            else:
                blk, off = divmod(int(ctx[i]) - 1, bs)
                assert got[i] == int(bt[i, blk]) * bs + off


def pin_kv_append(lib):
    rng = np.random.default_rng(4)
    nb, hkv, bs, d = 6, 3, 4, 8
    for dt in (np.float32, np.float16):
        kc = rng.standard_normal((nb, hkv, bs, d)).astype(dt)
        vc = rng.standard_normal((nb, hkv, bs, d)).astype(dt)
        kc0, vc0 = kc.copy(), vc.copy()
        slots = np.array([5, -1, 23, 0, 9], np.int64)
        kn = rng.standard_normal((5, hkv, d)).astype(dt)
        vn = rng.standard_normal((5, hkv, d)).astype(dt)
        oracle.kv_append(kn, vn, slots, kc, vc, lib=lib)
        for t, sl in enumerate(slots):
            if sl < 0:
                continue
            b, o = divmod(int(sl), bs)
            kc0[b, :, o, :] = kn[t]
            vc0[b, :, o, :] = vn[t]
        assert kc.tobytes() == kc0.tobytes() and vc.tobytes() == vc0.tobytes()
    for bad in ([1, 1], [nb * bs]):
        sl = np.array(bad, np.int64)
        kn = np.zeros((len(bad), hkv, d), np.float32)
        try:
            oracle.kv_append(kn, kn, sl, np.zeros((nb, hkv, bs, d), np.float32),
                             np.zeros((nb, hkv, bs, d), np.float32), lib=lib)
        except oracle.OracleError:
            continue
        raise AssertionError(f"kv_append accepted slots {bad}")


def pin_gather(lib):
    rng = np.random.default_rng(5)
    nb, hkv, bs, d = 20, 2, 4, 8
    kc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    bt = rng.permutation(nb)[:12].reshape(3, 4).astype(np.int32)
    ctx = np.array([0, 9, 16], np.int32)
    ko = np.full((3, 16, hkv, d), -7.0, np.float32)
    vo = np.full_like(ko, -7.0)
    oracle.gather_kv(kc, vc, bt, ctx, ko, vo, lib=lib)
    for s in range(3):
        for i in range(16):
            if i < ctx[s]:
                b, o = divmod(i, bs)
                assert (ko[s, i] == kc[bt[s, b], :, o]).all()
                assert (vo[s, i] == vc[bt[s, b], :, o]).all()
            else:
                assert (ko[s, i] == -7.0).all() and (vo[s, i] == -7.0).all()


# ---------------------------------------------------------------- attention

def pin_attention_vs_library(lib):
    rng = np.random.default_rng(6)
    for n in (1, 2, 5, 33, 100):
        for d in (8, 64):
            q = rng.standard_normal(d)
            K = rng.standard_normal((n, d))
            V = rng.standard_normal((n, d))
            sc = 1 / math.sqrt(d)
            got, w = oracle.attention_dense(q, K, V, sc, lib=lib)
            ref = _sdpa64(q, K, V, sc)
            assert np.max(np.abs(got - ref)) < 1e-12, (n, d)
            z = sc * (K @ q)
            e = np.exp(z - z.max())
            assert np.max(np.abs(w - e / e.sum())) < 1e-13


def pin_attention_special_cases(lib):
    rng = np.random.default_rng(8)
    d = 16
    K = rng.standard_normal((9, d))
    V = rng.standard_normal((9, d))
    q = rng.standard_normal(d)
    # a single cached row: its weight is 1 and the output is that row exactly
    got, w = oracle.attention_dense(q, K[:1], V[:1], 0.25, lib=lib)
    assert (got == V[0]).all() and w[0] == 1.0
    # zero query, or identical keys: uniform weights, the mean of V
    for qq, KK in ((np.zeros(d), K), (q, np.repeat(K[:1], 9, axis=0))):
        got, w = oracle.attention_dense(qq, KK, V, 0.25, lib=lib)
        assert np.max(np.abs(got - V.mean(axis=0))) < 1e-14
        assert np.max(np.abs(w - 1 / 9)) < 1e-15
    # V == 1 gives 1, and the weights sum to 1
    got, w = oracle.attention_dense(q, K, np.ones((9, d)), 0.25, lib=lib)
    assert np.max(np.abs(got - 1)) < 1e-14 and abs(w.sum() - 1) < 1e-14
    # one-hot values expose the weights; they follow the softmax of the scores
    got, w = oracle.attention_dense(q, K, np.eye(9, d), 0.25, lib=lib)
    z = 0.25 * (K @ q)
    ref = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    assert np.max(np.abs(got[:9] - ref)) < 1e-14 and np.all(got[9:] == 0)
    # a huge scale with distinct scores selects the best-scoring row
    got, _ = oracle.attention_dense(q, K, V, 1e3, lib=lib)
    assert np.max(np.abs(got - V[np.argmax(K @ q)])) < 1e-9
    # nothing cached: zero output
    got, _ = oracle.attention_dense(q, K[:0], V[:0], 0.25, lib=lib)
    assert (got == 0).all()


def _random_batch(rng, ctx, hkv, d, bs, nb, dt):
    dk = [rng.standard_normal((c, hkv, d)).astype(dt) for c in ctx]
    dv = [rng.standard_normal((c, hkv, d)).astype(dt) for c in ctx]
    kp, vp, bt, ctxa = _scatter_pool(dk, dv, bs, nb, rng, dt)
    return dk, dv, kp, vp, bt, ctxa


def pin_paged_equals_dense_library(lib):
    """Paging changes where rows live, not the result: oracle over a randomly
    placed pool equals torch float64 attention on the contiguous rows."""
    rng = np.random.default_rng(9)
    for (hq, hkv, d, bs, ctx, dt) in ((4, 2, 64, 4, [3, 7, 16, 33], np.float32),
                                       (6, 3, 32, 8, [1, 8, 9, 40], np.float16),
                                       (4, 1, 16, 16, [0, 17, 31], np.float32)):
        dk, dv, kp, vp, bt, ctxa = _random_batch(rng, ctx, hkv, d, bs, 64, dt)
        q = rng.standard_normal((len(ctx), hq, d)).astype(dt)
        sc = 1 / math.sqrt(d)
        got = oracle.paged_decode_attention(q, kp, vp, bt, ctxa, sc, lib=lib)
        g = hq // hkv
        for s in range(len(ctx)):
            for h in range(hq):
                if ctx[s] == 0:
                    assert (got[s, h] == 0).all()
                    continue
                ref = _sdpa64(q[s, h].astype(np.float64), dk[s][:, h // g].astype(np.float64),
                              dv[s][:, h // g].astype(np.float64), sc)
                assert np.max(np.abs(got[s, h] - ref)) < 1e-12, (s, h)


def pin_bf16_paged(lib):
    rng = np.random.default_rng(10)
    hq, hkv, d, bs = 4, 2, 32, 4
    ctx = [5, 12]
    dk = [torch.from_numpy(rng.standard_normal((c, hkv, d))).to(torch.bfloat16) for c in ctx]
    dv = [torch.from_numpy(rng.standard_normal((c, hkv, d))).to(torch.bfloat16) for c in ctx]
    bits = [[t.view(torch.int16).numpy().view(np.uint16) for t in x] for x in (dk, dv)]
    kp, vp, bt, ctxa = _scatter_pool(bits[0], bits[1], bs, 16, rng, np.uint16)
    q = torch.from_numpy(rng.standard_normal((2, hq, d))).to(torch.bfloat16)
    qb = q.view(torch.int16).numpy().view(np.uint16)
    got = oracle.paged_decode_attention(qb, kp, vp, bt, ctxa, 0.2, bf16=True, lib=lib)
    for s in range(2):
        for h in range(hq):
            ref = _sdpa64(q[s, h].double().numpy(), dk[s][:, h // 2].double().numpy(),
                          dv[s][:, h // 2].double().numpy(), 0.2)
            assert np.max(np.abs(got[s, h] - ref)) < 1e-12


def pin_permutation_invariance(lib):
    """Blocks may sit anywhere in the pool: renumbering them changes nothing."""
    rng = np.random.default_rng(11)
    dk, dv, kp, vp, bt, ctx = _random_batch(rng, [3, 7, 16, 33], 2, 64, 4, 64, np.float32)
    q = rng.standard_normal((4, 4, 64)).astype(np.float32)
    a = oracle.paged_decode_attention(q, kp, vp, bt, ctx, 0.125, lib=lib)
    perm = rng.permutation(64)                     # new id of old block b is perm[b]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    b = oracle.paged_decode_attention(q, kp2, vp2, bt2, ctx, 0.125, lib=lib)
    assert a.tobytes() == b.tobytes()


def pin_gqa_equals_repeated_mha(lib):
    rng = np.random.default_rng(12)
    hq, hkv = 8, 2
    g = hq // hkv
    dk, dv, kp, vp, bt, ctx = _random_batch(rng, [5, 20, 1], hkv, 32, 8, 16, np.float32)
    q = rng.standard_normal((3, hq, 32)).astype(np.float32)
    a = oracle.paged_decode_attention(q, kp, vp, bt, ctx, 0.17, lib=lib)
    kx = np.ascontiguousarray(np.repeat(kp, g, axis=1))
    vx = np.ascontiguousarray(np.repeat(vp, g, axis=1))
    b = oracle.paged_decode_attention(q, kx, vx, bt, ctx, 0.17, lib=lib)
    assert a.tobytes() == b.tobytes()
    # multi-query: one KV head serves every query head
    dk, dv, kp, vp, bt, ctx = _random_batch(rng, [6, 9], 1, 16, 4, 8, np.float32)
    q = rng.standard_normal((2, 4, 16)).astype(np.float32)
    got = oracle.paged_decode_attention(q, kp, vp, bt, ctx, 0.25, lib=lib)
    for s in range(2):
        for h in range(4):
            ref = _sdpa64(q[s, h], dk[s][:, 0], dv[s][:, 0], 0.25)
            assert np.max(np.abs(got[s, h] - ref)) < 1e-12


def pin_shared_prefix(lib):
    """Two tables naming the same blocks read the same rows: same query, same
    output; and sharing a prefix equals keeping private copies of it."""
    rng = np.random.default_rng(13)
    nb, hkv, bs, d = 12, 2, 4, 16
    kp = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vp = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    bt = np.array([[0, 1, 2, -1], [0, 1, 3, 4]], np.int32)   # blocks 0,1 shared
    ctx = np.array([10, 15], np.int32)
    q = rng.standard_normal((2, 2, d)).astype(np.float32)
    a = oracle.paged_decode_attention(q, kp, vp, bt, ctx, 0.3, lib=lib)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[[5, 6]], vp2[[5, 6]] = kp[[0, 1]], vp[[0, 1]]         # private copies for seq 1
    bt2 = np.array([[0, 1, 2, -1], [5, 6, 3, 4]], np.int32)
    b = oracle.paged_decode_attention(q, kp2, vp2, bt2, ctx, 0.3, lib=lib)
    assert a.tobytes() == b.tobytes()
    q2 = np.repeat(q[:1], 2, axis=0)
    c = oracle.paged_decode_attention(q2, kp, vp, np.repeat(bt[:1], 2, axis=0),
                                      np.array([10, 10], np.int32), 0.3, lib=lib)
    assert c[0].tobytes() == c[1].tobytes()


# ---------------------------------------------------------------- the pages' worked numbers

def pin_decode_loop_rows(lib):
    """3-token prompt + 4 decode steps: 25 K,V rows without a cache, 7 with,
    and identical attention outputs in both lanes."""
    from oracle import decode_loop
    gold = _golden("kv_rows_prompt3_decode4.json")
    rng = np.random.default_rng(14)
    hq, hkv, d, dm, bs = 4, 2, 64, 64, 4
    n_tok = len(gold["prompt"]) + len(gold["decoded"])
    x = rng.standard_normal((n_tok, dm))
    Wq = rng.standard_normal((dm, hq * d)) / 8
    Wk = rng.standard_normal((dm, hkv * d)) / 8
    Wv = rng.standard_normal((dm, hkv * d)) / 8
    table = [5, 2, 9]
    r = decode_loop.run(x, Wq, Wk, Wv, len(gold["prompt"]), hq, hkv, d, bs, table, 16,
                        0.125, lib=lib)
    assert r["rows_no_cache"] == gold["rows_without_cache"]
    assert r["rows_cache"] == gold["rows_with_cache"]
    assert sum(r["rows_no_cache"]) == gold["total_without_cache"]
    assert sum(r["rows_cache"]) == gold["total_with_cache"]
    assert r["out_cache"].tobytes() == r["out_no_cache"].tobytes()
    # and both equal float64 attention computed from the same rows by torch
    k = (x @ Wk).astype(np.float32).reshape(n_tok, hkv, d).astype(np.float64)
    v = (x @ Wv).astype(np.float32).reshape(n_tok, hkv, d).astype(np.float64)
    q = (x @ Wq).astype(np.float32).reshape(n_tok, hq, d).astype(np.float64)
    for i, n in enumerate(r["prefix_lengths"]):
        for h in range(hq):
            ref = _sdpa64(q[n - 1, h], k[:n, h // 2], v[:n, h // 2], 0.125)
            assert np.max(np.abs(r["out_cache"][i, h] - ref)) < 1e-5


def pin_rows_closed_form(lib):
    """Prompt p then n decode steps: sum_{t=0..n} (p+t) rows without a cache,
    p+n with it; for p=1 that is n(n+1)/2-ish growth against linear."""
    gold = _golden("kv_rows_prompt3_decode4.json")
    p, n = len(gold["prompt"]), len(gold["decoded"])
    assert sum(p + t for t in range(n + 1)) == gold["total_without_cache"]
    assert p + n == gold["total_with_cache"]
    for N in (10, 100, 1000):
        assert sum(range(1, N + 1)) == N * (N + 1) // 2


def pin_bytes_per_token(lib):
    gold = _golden("kv_memory_table.json")
    bpn = gold["bytes_per_number"]
    for m in gold["models"]:
        b = oracle.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], bpn, lib=lib)
        assert b == m["per_token_kib"] * 1024, m["model"]
        if "at_4096_bytes" in m:
            assert b * 4096 == m["at_4096_bytes"]
        else:
            # printed to one decimal, rounding half up: exactly 1.25 GiB shows as 1.3
            assert math.floor(b * 4096 / 2 ** 30 * 10 + 0.5) / 10 == m["at_4096_gib_printed"]
    ex = gold["batch_example"]
    llama2 = [m for m in gold["models"] if m["model"] == ex["model"]][0]
    b = oracle.kv_bytes_per_token(llama2["layers"], llama2["kv_heads"], llama2["head_dim"], bpn,
                                  lib=lib)
    assert b * ex["tokens"] * ex["requests"] == ex["cache_gib"] * 2 ** 30
    assert b * ex["tokens"] * ex["requests"] > ex["weights_gb_about"] * 1e9
    g = gold["guide_example"]
    b = oracle.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["bytes_per_number"],
                                  lib=lib) * g["tokens"]
    assert abs(b / 2 ** 30 - g["about_gb"]) < 0.01
    gq = gold["gqa_example"]
    a = oracle.kv_bytes_per_token(32, gq["kv_heads"], 128, bpn, lib=lib)
    c = oracle.kv_bytes_per_token(32, gq["instead_of"], 128, bpn, lib=lib)
    assert c == gq["saving_factor"] * a
    # int8 codes plus one fp16 scale per (token, head) row: about half of fp16
    d = 128
    ratio = (oracle.kv_bytes_per_token(32, 8, d, 1, lib=lib) + 2 * 32 * 8 * 2) / \
        oracle.kv_bytes_per_token(32, 8, d, 2, lib=lib)
    assert abs(ratio - (d + 2) / (2 * d)) < 1e-12 and 0.45 < ratio < 0.55


# ---------------------------------------------------------------- int8 reading (ours)

def pin_int8_quantizer(lib):
    # worked by hand: 1/127 = 0.0078740..., which lies in [2^-7, 2^-6) where
    # binary16 steps by 2^-17; 0.0078740 / 2^-17 = 1032.06 -> 1032, so
    # s = 1032 * 2^-17 = 0.00787353515625; 1/s = 127.0085 -> 127,
    # -0.5/s = -63.504 -> -64, 0.25/s = 31.752 -> 32, 0.001/s = 0.127 -> 0.
    x = np.array([1.0, -0.5, 0.25, 0.001] + [0.0] * 4, np.float16)
    q, s = oracle.quantize_row_int8(x, lib=lib)
    assert float(s) == 1032 * 2.0 ** -17
    assert q.tolist() == [127, -64, 32, 0, 0, 0, 0, 0]
    # an all-zero row: zero scale, zero codes
    q, s = oracle.quantize_row_int8(np.zeros(16, np.float16), lib=lib)
    assert float(s) == 0 and (q == 0).all()
    rng = np.random.default_rng(15)
    for _ in range(200):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float16)
        q, s = oracle.quantize_row_int8(x, lib=lib)
        s = float(s)
        xf = x.astype(np.float64)
        assert np.abs(q).max() == 127 and q.min() >= -127
        # within half a step, plus the rounding of the scale itself
        assert np.all(np.abs(xf - s * q) <= s / 2 * (1 + 1e-6) + np.abs(xf) * 2.0 ** -10)
        qn, sn = oracle.quantize_row_int8(-x, lib=lib)
        assert float(sn) == s and (qn == -q).all()


def pin_int8_attention_dequantizes_exactly(lib):
    """The int8 path equals the float path on the dequantized values, which
    code * scale gives exactly in binary32."""
    rng = np.random.default_rng(16)
    nb, hkv, bs, d, hq = 10, 2, 4, 32, 4
    src_k = rng.standard_normal((nb * bs, hkv, d)).astype(np.float16)
    src_v = rng.standard_normal((nb * bs, hkv, d)).astype(np.float16)
    kq = np.zeros((nb, hkv, bs, d), np.int8)
    vq = np.zeros_like(kq)
    ks = np.zeros((nb, hkv, bs), np.float16)
    vs = np.zeros_like(ks)
    oracle.kv_append_int8(src_k, src_v, np.arange(nb * bs, dtype=np.int64), kq, vq, ks, vs,
                          lib=lib)
    kf = (kq.astype(np.float32) * ks[..., None].astype(np.float32)).astype(np.float32)
    vf = (vq.astype(np.float32) * vs[..., None].astype(np.float32)).astype(np.float32)
    assert np.all(np.abs(kf.transpose(0, 2, 1, 3).reshape(-1, hkv, d) - src_k.astype(np.float32))
                  <= ks.transpose(0, 2, 1).reshape(-1, hkv)[..., None].astype(np.float32) * 0.51)
    bt = rng.permutation(nb)[:8].reshape(2, 4).astype(np.int32)
    ctx = np.array([13, 16], np.int32)
    q = rng.standard_normal((2, hq, d)).astype(np.float16)
    a = oracle.paged_decode_attention(q, kq, vq, bt, ctx, 0.2, k_scale=ks, v_scale=vs, lib=lib)
    b = oracle.paged_decode_attention(q, kf, vf, bt, ctx, 0.2, lib=lib)
    assert a.tobytes() == b.tobytes()


# ---------------------------------------------------------------- sliding window

def _window_batch(rng, ctx, bs=4, hkv=2, d=16, nb=96):
    K = [rng.standard_normal((c, hkv, d)).astype(np.float32) for c in ctx]
    V = [rng.standard_normal((c, hkv, d)).astype(np.float32) for c in ctx]
    kp, vp, bt, ctx_a = _scatter_pool(K, V, bs, nb, rng, np.float32)
    return K, V, kp, vp, bt, ctx_a


def pin_window_whole_context(lib):
    """No window, or one at least as long as the context, is plain decode."""
    rng = np.random.default_rng(31)
    _, _, kp, vp, bt, ctx = _window_batch(rng, [1, 7, 23, 40])
    q = rng.standard_normal((4, 4, 16)).astype(np.float32)
    full = oracle.paged_decode_attention(q, kp, vp, bt, ctx, 0.3, lib=lib)
    for w in (0, -5, 40, 41, 1000):
        got = oracle.paged_decode_attention_window(q, kp, vp, bt, ctx, 0.3, w, lib=lib)
        assert got.tobytes() == full.tobytes(), w


def pin_window_is_attention_over_last_rows(lib):
    """torch's float64 SDPA over the last `window` rows of each sequence; a
    window of one row returns that row."""
    rng = np.random.default_rng(32)
    K, V, kp, vp, bt, ctx = _window_batch(rng, [5, 23, 40, 17])
    q = rng.standard_normal((4, 4, 16)).astype(np.float32)
    for w in (1, 3, 4, 9, 16, 22):
        got = oracle.paged_decode_attention_window(q, kp, vp, bt, ctx, 0.3, w, lib=lib)
        for s in range(4):
            lo = max(0, int(ctx[s]) - w)
            for h in range(4):
                ref = _sdpa64(q[s, h], K[s][lo:, h // 2], V[s][lo:, h // 2], 0.3)
                assert np.max(np.abs(got[s, h] - ref)) < 1e-12, (w, s, h)
                if w == 1:
                    assert np.array_equal(got[s, h], V[s][-1, h // 2].astype(np.float64))


def pin_window_reads_nothing_before_it(lib):
    """Blocks wholly before the window may be freed: NaN in their rows and -1
    in their table entries change nothing; a block-aligned window equals the
    whole-context attention of the table that starts at the window's block."""
    rng = np.random.default_rng(33)
    _, _, kp, vp, bt, ctx = _window_batch(rng, [40, 37, 16])
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    w = 12
    ref = oracle.paged_decode_attention_window(q, kp, vp, bt, ctx, 0.3, w, lib=lib)
    kp2, vp2, bt2 = kp.copy(), vp.copy(), bt.copy()
    for s in range(3):
        first = max(0, int(ctx[s]) - w)
        for j in range(first // 4):
            kp2[bt[s, j]] = np.nan
            vp2[bt[s, j]] = np.nan
            bt2[s, j] = -1
    got = oracle.paged_decode_attention_window(q, kp2, vp2, bt2, ctx, 0.3, w, lib=lib)
    assert got.tobytes() == ref.tobytes()
    # sequence 0: ctx 40, window 12 -> positions 28..39 = blocks 7..9, aligned
    shifted = np.full((1, bt.shape[1]), -1, np.int32)
    shifted[0, :3] = bt[0, 7:10]
    whole = oracle.paged_decode_attention(q[:1], kp, vp, shifted, np.array([12], np.int32),
                                          0.3, lib=lib)
    assert whole.tobytes() == ref[:1].tobytes()


# ---------------------------------------------------------------- fp8 (E4M3)

def _e4m3_table():
    """torch's float8_e4m3fn decoding of every code (library routine)."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def pin_fp8_e4m3_decode_exhaustive(lib):
    ref = _e4m3_table()
    got = np.array([oracle.fp8_e4m3_to_double(c, lib) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def pin_fp8_e4m3_encode(lib):
    """Every finite code round-trips; a value halfway between two neighbours
    goes to the one with the even code (as torch's cast does); a hair off the
    midpoint goes to the nearer; above 448 saturates (this project's reading:
    torch rounds magnitudes past 464 to NaN); NaN encodes as 0."""
    enc = lambda x: oracle.double_to_fp8_e4m3(float(x), lib)
    vals = _e4m3_table()[:127]            # 0 .. 448, increasing
    for c in range(127):
        assert enc(vals[c]) == c
        if c:
            assert enc(-vals[c]) == c | 0x80
    for c in range(126):
        a, b = vals[c], vals[c + 1]
        mid = (a + b) / 2
        even = c if c % 2 == 0 else c + 1
        assert enc(mid) == even
        assert enc(mid) == torch.tensor(mid, dtype=torch.float64).to(
            torch.float8_e4m3fn).view(torch.uint8).item()
        assert enc(mid + (b - a) * 1e-6) == c + 1 and enc(mid - (b - a) * 1e-6) == c
    assert enc(449.0) == 0x7E and enc(1e6) == 0x7E and enc(-1e6) == 0xFE
    assert enc(float("nan")) == 0


def pin_fp8_quantizer(lib):
    # worked by hand: 1/448 = 0.0022321... lies in [2^-9, 2^-8) where binary16
    # steps by 2^-19; 0.0022321 / 2^-19 = 1170.3 -> 1170, s = 1170 * 2^-19.
    # 1/s = 448.11 saturates to 448 (0x7E); -0.5/s = -224.05 -> -224 = -1.75*2^7
    # (0xF6); 0.25/s = 112.03 -> 112 = 1.75*2^6 (0x6E); 0.001/s = 0.4483 ->
    # 0.4375 = 1.75*2^-2 (0x2E), the E4M3 step in [0.25, 0.5) being 2^-5.
    x = np.array([1.0, -0.5, 0.25, 0.001] + [0.0] * 4, np.float16)
    q, s = oracle.quantize_row_fp8(x, lib=lib)
    assert float(s) == 1170 * 2.0 ** -19
    assert q.tolist() == [0x7E, 0xF6, 0x6E, 0x2E, 0, 0, 0, 0]
    q, s = oracle.quantize_row_fp8(np.zeros(16, np.float16), lib=lib)
    assert float(s) == 0 and (q == 0).all()
    table = _e4m3_table()
    rng = np.random.default_rng(17)
    for _ in range(200):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float16)
        q, s = oracle.quantize_row_fp8(x, lib=lib)
        s = float(s)
        xf = x.astype(np.float64)
        deq = s * table[q]
        # half an E4M3 step (2^-4 relative, or 2^-10 absolute among the
        # subnormals) plus the rounding of the scale
        assert np.all(np.abs(xf - deq) <= np.abs(xf) * (2.0 ** -4 + 2.0 ** -10)
                      + s * 2.0 ** -10 * 1.0001)
        qn, sn = oracle.quantize_row_fp8(-x, lib=lib)
        assert float(sn) == s and np.array_equal(qn, np.where(q == 0, 0, q ^ 0x80))


def pin_fp8_attention_dequantizes_exactly(lib):
    """The fp8 path equals the float path on code * scale, exact in binary32
    (4 significant bits times 11)."""
    rng = np.random.default_rng(18)
    nb, hkv, bs, d, hq = 10, 2, 4, 32, 4
    src_k = rng.standard_normal((nb * bs, hkv, d)).astype(np.float16)
    src_v = rng.standard_normal((nb * bs, hkv, d)).astype(np.float16)
    kq = np.zeros((nb, hkv, bs, d), np.uint8)
    vq = np.zeros_like(kq)
    ks = np.zeros((nb, hkv, bs), np.float16)
    vs = np.zeros_like(ks)
    oracle.kv_append_fp8(src_k, src_v, np.arange(nb * bs, dtype=np.int64), kq, vq, ks, vs,
                         lib=lib)
    table = _e4m3_table().astype(np.float32)
    kf = (table[kq] * ks[..., None].astype(np.float32)).astype(np.float32)
    vf = (table[vq] * vs[..., None].astype(np.float32)).astype(np.float32)
    bt = rng.permutation(nb)[:8].reshape(2, 4).astype(np.int32)
    ctx = np.array([13, 16], np.int32)
    q = rng.standard_normal((2, hq, d)).astype(np.float16)
    a = oracle.paged_decode_attention(q, kq, vq, bt, ctx, 0.2, k_scale=ks, v_scale=vs, lib=lib)
    b = oracle.paged_decode_attention(q, kf, vf, bt, ctx, 0.2, lib=lib)
    assert a.tobytes() == b.tobytes()


# ---------------------------------------------------------------- int4

def _int4_unpack(packed):
    """Codes of packed int4 rows: dim 2i low nibble of byte i, 2i+1 high,
    stored as code + 8 (test-side numpy, from the documented layout)."""
    lo = (packed & 15).astype(np.int16) - 8
    hi = (packed >> 4).astype(np.int16) - 8
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


def pin_int4_quantizer(lib):
    # worked by hand, group 0: max 7 -> s = fp16(7 / 7) = 1 exactly, so the
    # codes are the values rounded half to even and clamped: 7, -3.5 -> -4,
    # 2.5 -> 2, 0.4 -> 0, -0.6 -> -1, 6.5 -> 6, -7, 0; nibbles (+8) 15, 4, 10,
    # 8, 7, 14, 1, 8 pack as bytes 0x4F, 0x8A, 0xE7, 0x81.  Group 1 is zero:
    # scale 0, every nibble 8 (byte 0x88).  Group 2 holds a NaN: it codes as 0.
    x = np.zeros(96, np.float16)
    x[:8] = [7, -3.5, 2.5, 0.4, -0.6, 6.5, -7, 0]
    x[64:72] = [1, 2, 3, float("nan"), -4, 0.5, 0, 0]
    q, sc = oracle.quantize_row_int4(x, lib=lib)
    assert q[:4].tolist() == [0x4F, 0x8A, 0xE7, 0x81] and (q[4:16] == 0x88).all()
    assert float(sc[0]) == 1.0 and float(sc[1]) == 0.0
    assert (q[16:32] == 0x88).all()            # group 1: dims 32..63 are zero
    codes = _int4_unpack(q)
    assert codes[67] == 0 and codes[68] == -7 and codes[64:67].tolist() == [2, 4, 5]
    rng = np.random.default_rng(41)
    for _ in range(200):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float16)
        q, sc = oracle.quantize_row_int4(x, lib=lib)
        c = _int4_unpack(q).astype(np.float64)
        s = np.repeat(sc.astype(np.float64), 32)
        xf = x.astype(np.float64)
        assert np.abs(c).max() == 7 and np.abs(c).min() >= 0
        assert np.all(np.abs(xf - s * c) <= s / 2 * (1 + 1e-6) + np.abs(xf) * 2.0 ** -10)
        qn, sn = oracle.quantize_row_int4(-x, lib=lib)
        assert np.array_equal(sn, sc) and np.array_equal(_int4_unpack(qn), -_int4_unpack(q))


def pin_int4_attention_dequantizes_exactly(lib):
    """The int4 path equals the float path on code * group scale (exact in
    binary32), and the gather copies packed rows and their group scales."""
    rng = np.random.default_rng(42)
    nb, hkv, bs, d, hq = 10, 2, 4, 64, 4
    src_k = (rng.standard_normal((nb * bs, hkv, d)) *
             np.repeat(rng.uniform(0.1, 10, (1, 1, d // 32)), 32, axis=2)).astype(np.float16)
    src_v = rng.standard_normal((nb * bs, hkv, d)).astype(np.float16)
    kq = np.zeros((nb, hkv, bs, d // 2), np.uint8)
    vq = np.zeros_like(kq)
    ks = np.zeros((nb, hkv, bs, d // 32), np.float16)
    vs = np.zeros_like(ks)
    oracle.kv_append_int4(src_k, src_v, np.arange(nb * bs, dtype=np.int64), kq, vq, ks, vs,
                          lib=lib)
    kf = (_int4_unpack(kq) * np.repeat(ks.astype(np.float32), 32, axis=3)).astype(np.float32)
    vf = (_int4_unpack(vq) * np.repeat(vs.astype(np.float32), 32, axis=3)).astype(np.float32)
    bt = rng.permutation(nb)[:8].reshape(2, 4).astype(np.int32)
    ctx = np.array([13, 16], np.int32)
    q = rng.standard_normal((2, hq, d)).astype(np.float16)
    a = oracle.paged_decode_attention(q, kq, vq, bt, ctx, 0.2, k_scale=ks, v_scale=vs,
                                      int4=True, lib=lib)
    b = oracle.paged_decode_attention(q, kf, vf, bt, ctx, 0.2, lib=lib)
    assert a.tobytes() == b.tobytes()
    ko = np.zeros((2, 16, hkv, d // 2), np.uint8)
    vo = np.zeros_like(ko)
    kso = np.zeros((2, 16, hkv, d // 32), np.float16)
    vso = np.zeros_like(kso)
    oracle.gather_kv(kq, vq, bt, ctx, ko, vo, k_scale=ks, v_scale=vs, k_scale_out=kso,
                     v_scale_out=vso, int4=True, lib=lib)
    for s_ in range(2):
        for i in range(int(ctx[s_])):
            b_, o = divmod(i, bs)
            assert np.array_equal(ko[s_, i], kq[bt[s_, b_], :, o])
            assert np.array_equal(kso[s_, i], ks[bt[s_, b_], :, o])


# ---------------------------------------------------------------- quantizing appends: placement

def _dequant_rows(kind, codes, scales):
    """Test-side numpy decoding of stored rows: codes [..., D] (int4: [..., D/2]
    packed) times their scales ([...] or, for int4, [..., D/32]), in float64."""
    if kind == "int8":
        return codes.astype(np.float64) * scales.astype(np.float64)[..., None]
    if kind == "fp8":
        return _e4m3_table()[codes] * scales.astype(np.float64)[..., None]
    return _int4_unpack(codes).astype(np.float64) * np.repeat(scales.astype(np.float64), 32,
                                                              axis=-1)


def _within_quantizer_bound(kind, x, deq, scales):
    """Each quantizer's stated error bound (the pins above): half a code step,
    plus the binary16 rounding of the scale (fp8: half an E4M3 step relative,
    or half a subnormal step)."""
    x = x.astype(np.float64)
    if kind == "fp8":
        s = scales.astype(np.float64)[..., None]
        return np.all(np.abs(x - deq) <= np.abs(x) * (2.0 ** -4 + 2.0 ** -10) + s * 2.0 ** -10 *
                      1.0001)
    s = scales.astype(np.float64)
    s = s[..., None] if kind == "int8" else np.repeat(s, 32, axis=-1)
    return np.all(np.abs(x - deq) <= s / 2 * (1 + 1e-6) + np.abs(x) * 2.0 ** -10)


def pin_quantizing_appends_place_source_rows(lib):
    """Every quantizing append stores token t's K row in the K pool and its V
    row in the V pool at (slot // block_size, slot % block_size), for every KV
    head ([viz] "PagedAttention: the cache in blocks": a slot names one
    position of one block; [notes] "Quantized KV cache": the cache holds the
    rows in fewer bits).  Slots are a seeded permutation with -1 pads, K and V
    are drawn at different magnitudes, and decoding each stored row must land
    within the quantizer's bound of the row it came from.  A slot of -1 and
    every slot the call does not name keep their bytes."""
    rng = np.random.default_rng(61)
    nb, hkv, bs, d = 12, 3, 4, 64
    for kind in ("int8", "fp8", "int4"):
        t_real = 17
        slots = rng.permutation(nb * bs)[:t_real].astype(np.int64)
        slots = np.insert(slots, [0, 5, t_real], -1)      # pads at the front, middle and end
        t = slots.shape[0]
        k_new = (rng.standard_normal((t, hkv, d)) * 3.0).astype(np.float16)
        v_new = (rng.standard_normal((t, hkv, d)) * 0.25 + 0.5).astype(np.float16)
        cdt, cw = (np.int8, d) if kind == "int8" else (np.uint8, d if kind == "fp8" else d // 2)
        sshape = (nb, hkv, bs) if kind != "int4" else (nb, hkv, bs, d // 32)
        kq = rng.integers(-100, 100, (nb, hkv, bs, cw)).astype(cdt)
        vq = rng.integers(-100, 100, (nb, hkv, bs, cw)).astype(cdt)
        ks = rng.uniform(1, 2, sshape).astype(np.float16)
        vs = rng.uniform(3, 4, sshape).astype(np.float16)
        before = [a.copy() for a in (kq, vq, ks, vs)]
        fn = {"int8": oracle.kv_append_int8, "fp8": oracle.kv_append_fp8,
              "int4": oracle.kv_append_int4}[kind]
        fn(k_new, v_new, slots, kq, vq, ks, vs, lib=lib)
        written = np.zeros((nb, bs), bool)
        for i, slot in enumerate(slots):
            if slot < 0:
                continue
            b, o = divmod(int(slot), bs)
            written[b, o] = True
            for src, codes, sc in ((k_new, kq, ks), (v_new, vq, vs)):
                deq = _dequant_rows(kind, codes[b, :, o], sc[b, :, o])
                assert _within_quantizer_bound(kind, src[i], deq, sc[b, :, o]), (kind, i, slot)
        for now, old in zip((kq, vq, ks, vs), before):
            keep = np.broadcast_to(~written[:, None, :].reshape(nb, 1, bs, *([1] * (now.ndim - 3))),
                                   now.shape)
            assert np.array_equal(now[keep], old[keep]), kind


# ---------------------------------------------------------------- prefill

def _sdpa64_rows(q, K, V, scale, mask):
    """torch float64 SDPA for several queries with a boolean mask (True = seen)."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    Kt = torch.from_numpy(np.asarray(K, np.float64))[None, None]
    Vt = torch.from_numpy(np.asarray(V, np.float64))[None, None]
    m = torch.from_numpy(np.asarray(mask, bool))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m,
                                                            scale=scale)[0, 0].numpy()


def pin_prefill_is_causal_attention(lib):
    """Whole prompts (T = context): torch's causal SDPA on the dense rows;
    chunks (T < context, earlier positions cached): SDPA with the mask 'key
    position <= query position', the query positions being the last T."""
    rng = np.random.default_rng(21)
    hq, hkv, d, bs = 4, 2, 16, 4
    ctx = [1, 5, 19, 23, 9]
    tq = [1, 5, 19, 7, 3]                       # the last two are chunks
    K = [rng.standard_normal((c, hkv, d)).astype(np.float32) for c in ctx]
    V = [rng.standard_normal((c, hkv, d)).astype(np.float32) for c in ctx]
    kp, vp, bt, ctx_a = _scatter_pool(K, V, bs, 64, rng, np.float32)
    qs = np.concatenate([[0], np.cumsum(tq)]).astype(np.int32)
    q = rng.standard_normal((qs[-1], hq, d)).astype(np.float32)
    out = oracle.paged_prefill_attention(q, kp, vp, bt, qs, ctx_a, 0.25, lib=lib)
    for s, (c, t) in enumerate(zip(ctx, tq)):
        for h in range(hq):
            qq = q[qs[s]:qs[s + 1], h].astype(np.float64)
            kk, vv = K[s][:, h // 2].astype(np.float64), V[s][:, h // 2].astype(np.float64)
            if t == c:
                qt = torch.from_numpy(qq)[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qt, torch.from_numpy(kk)[None, None], torch.from_numpy(vv)[None, None],
                    is_causal=True, scale=0.25)[0, 0].numpy()
            else:
                mask = np.arange(c)[None, :] <= (c - t + np.arange(t))[:, None]
                ref = _sdpa64_rows(qq, kk, vv, 0.25, mask)
            assert np.max(np.abs(out[qs[s]:qs[s + 1], h] - ref)) < 1e-12


def pin_prefill_matches_decode_loop(lib):
    """The pages' loop (3-token prompt, 4 decode steps): one causal prefill
    over all 7 tokens gives, at every position, exactly the output the loop
    produced when that position was the newest ("the attention itself is the
    same in both lanes")."""
    from oracle import decode_loop
    rng = np.random.default_rng(14)
    hq, hkv, d, dm, bs = 4, 2, 64, 64, 4
    n_tok = 7
    x = rng.standard_normal((n_tok, dm))
    Wq = rng.standard_normal((dm, hq * d)) / 8
    Wk = rng.standard_normal((dm, hkv * d)) / 8
    Wv = rng.standard_normal((dm, hkv * d)) / 8
    table = [5, 2, 9]
    r = decode_loop.run(x, Wq, Wk, Wv, 3, hq, hkv, d, bs, table, 16, 0.125, lib=lib)
    rows = lambda W, h: np.stack([oracle.project_row(x[t], W, lib).astype(np.float32)
                                  .reshape(h, d) for t in range(n_tok)])
    q, k, v = rows(Wq, hq), rows(Wk, hkv), rows(Wv, hkv)
    kc = np.full((16, hkv, bs, d), np.nan, np.float32)
    vc = np.full_like(kc, np.nan)
    bt = np.array([table], np.int32)
    slots = oracle.slot_mapping(bt, np.zeros(n_tok, np.int32), np.arange(n_tok, dtype=np.int32),
                                bs, lib=lib)
    oracle.kv_append(k, v, slots, kc, vc, lib=lib)
    out = oracle.paged_prefill_attention(q, kc, vc, bt, np.array([0, n_tok], np.int32),
                                         np.array([n_tok], np.int32), 0.125, lib=lib)
    for i, n in enumerate(r["prefix_lengths"]):
        assert out[n - 1].tobytes() == r["out_cache"][i].tobytes()


def pin_prefill_chunking_invariance(lib):
    """A prompt taken in chunks (each attending over the positions cached so
    far plus itself) gives the same rows as one whole prefill, bit for bit."""
    rng = np.random.default_rng(22)
    hq, hkv, d, bs, n = 2, 1, 8, 4, 12
    K = [rng.standard_normal((n, hkv, d)).astype(np.float32)]
    V = [rng.standard_normal((n, hkv, d)).astype(np.float32)]
    kp, vp, bt, _ = _scatter_pool(K, V, bs, 16, rng, np.float32)
    q = rng.standard_normal((n, hq, d)).astype(np.float32)
    whole = oracle.paged_prefill_attention(q, kp, vp, bt, np.array([0, n], np.int32),
                                           np.array([n], np.int32), 0.3, lib=lib)
    done = 0
    for t in (5, 4, 3):
        part = oracle.paged_prefill_attention(q[done:done + t], kp, vp, bt,
                                              np.array([0, t], np.int32),
                                              np.array([done + t], np.int32), 0.3, lib=lib)
        assert part.tobytes() == whole[done:done + t].tobytes()
        done += t


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
