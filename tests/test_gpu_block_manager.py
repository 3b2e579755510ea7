"""The block pool on the GPU (needs an MI355X):
  - pa_copy_blocks moves whole blocks bit-exactly and skips pairs outside the
    pool;
  - a seeded serving script -- prompts prefilled, prefixes forked, decode
    rounds, requests finished -- run by the native manager on GPU pools
    (copy-on-write copies, appends and attention all through the library)
    keeps every live sequence's rows equal to the rows appended to it, and
    its attention output within tolerance of the fp64 oracle over those rows.
"""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
from gpu_cases import ELEM, TOL, dev, host
from oracle import block_manager as bm

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8,
         "fp8": torch.float8_e4m3fn}


def random_pool(rng, nb, hkv, bs, d, fmt):
    raw = rng.integers(0, 256, size=(nb, hkv, bs, d * ELEM[fmt]), dtype=np.uint8)
    return torch.from_numpy(raw).to(dev()).view(TORCH[fmt])


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16", "i8", "fp8"])
@pytest.mark.parametrize("d,bs,hkv", [(64, 4, 3), (128, 16, 8), (128, 32, 1)])
def test_copy_blocks_bit_exact(fmt, d, bs, hkv):
    rng = np.random.default_rng(d + bs + hkv)
    nb = 64
    kc, vc = random_pool(rng, nb, hkv, bs, d, fmt), random_pool(rng, nb, hkv, bs, d, fmt)
    ks = vs = None
    if fmt in ("i8", "fp8"):
        ks = torch.from_numpy(rng.integers(0, 1 << 16, (nb, hkv, bs), dtype=np.uint16)
                              .view(np.float16)).to(dev())
        vs = torch.from_numpy(rng.integers(0, 1 << 16, (nb, hkv, bs), dtype=np.uint16)
                              .view(np.float16)).to(dev())
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:12], perm[12:24]], 1)
    bad = np.array([[-1, perm[30]], [perm[31], nb], [nb + 5, -3]])
    all_pairs = np.concatenate([pairs[:6], bad, pairs[6:]]).astype(np.int32)
    want = [host(t).copy() for t in (kc, vc) + ((ks, vs) if ks is not None else ())]
    for w in want:
        w[pairs[:, 1]] = w[pairs[:, 0]]
    print(f"copy_blocks {fmt} d={d} bs={bs} hkv={hkv}", flush=True)
    pa.copy_blocks(kc, vc, all_pairs, ks, vs)
    torch.cuda.synchronize()
    got = [host(t) for t in (kc, vc) + ((ks, vs) if ks is not None else ())]
    for g, w in zip(got, want):
        assert np.array_equal(g.view(np.uint8), w.view(np.uint8))


def test_copy_blocks_empty_and_checks():
    kc = torch.zeros((4, 1, 16, 64), dtype=torch.float16, device=dev())
    pa.copy_blocks(kc, kc.clone(), np.zeros((0, 2), np.int32))
    with pytest.raises(ValueError, match="k_scale"):      # the library's own NULL check: test_abi
        pa.copy_blocks(kc.to(torch.int8), kc.to(torch.int8), np.array([[0, 1]], np.int32))


CONFIGS = {  # fmt: (head_dim, block_size, q heads, kv heads, pool blocks)
    "f32": (64, 8, 4, 2, 160),
    "f16": (128, 16, 8, 2, 96),
    "bf16": (128, 32, 16, 2, 64),
    "i8": (128, 16, 8, 2, 96),
}


def _rows(rng, t, hkv, d, fmt):
    x = torch.from_numpy(rng.standard_normal((t, hkv, d)).astype(np.float32)).to(dev())
    return x.to(torch.float16 if fmt == "i8" else TORCH[fmt])


def _dense_kv(dense, sid, fmt, lib):
    """fp64 K, V [n, Hkv, D] of a sequence as the cache holds them (int8:
    the oracle's quantization of the appended fp16 rows, dequantized)."""
    k, v = dense.kv(sid)
    if fmt == "bf16":
        to64 = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return to64(k), to64(v)
    if fmt != "i8":
        return k.astype(np.float64), v.astype(np.float64)
    out = []
    for a in (k, v):
        deq = np.empty(a.shape, np.float64)
        for i in range(a.shape[0]):
            for h in range(a.shape[1]):
                codes, s = oracle.quantize_row_int8(a[i, h], lib=lib)
                deq[i, h] = codes.astype(np.float64) * float(s)
        out.append(deq)
    return out


@pytest.mark.parametrize("fmt", sorted(CONFIGS))
def test_serving_script(fmt, orc):
    d, bs, hq, hkv, nb = CONFIGS[fmt]
    g = hq // hkv
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng({"f32": 1, "f16": 2, "bf16": 3, "i8": 4}[fmt])
    i8 = fmt == "i8"
    cdt = TORCH[fmt]
    if i8:
        kc = torch.zeros((nb, hkv, bs, d), dtype=torch.int8, device=dev())
        vc = torch.zeros_like(kc)
        ks = torch.full((nb, hkv, bs), float("nan"), dtype=torch.float16, device=dev())
        vs = ks.clone()
    else:
        kc = torch.full((nb, hkv, bs, d), float("nan"), dtype=cdt, device=dev())
        vc = kc.clone()
        ks = vs = None
    mgr = pa.BlockManager(nb, bs)
    dense = bm.DenseRows()
    live = []
    copies_seen = 0
    rounds = 0

    def append(reqs):
        nonlocal copies_seen
        slots, copies = mgr.append(reqs)
        copies_seen += len(copies)
        if len(copies):
            pa.copy_blocks(kc, vc, copies, ks, vs)
        t = slots.size
        kn, vn = _rows(rng, t, hkv, d, fmt), _rows(rng, t, hkv, d, fmt)
        sl = torch.from_numpy(slots).to(dev())
        if i8:
            pa.kv_append_int8(kn, vn, sl, kc, vc, ks, vs)
        else:
            pa.kv_append(kn, vn, sl, kc, vc)
        khost, vhost = host(kn), host(vn)
        i = 0
        for sid, n in reqs:
            for _ in range(n):
                dense.append(sid, khost[i], vhost[i])
                i += 1

    def decode_round(fused):
        """Every live sequence appends one token and attends."""
        nonlocal rounds, copies_seen
        rounds += 1
        q = _rows(rng, len(live), hq, d, fmt)
        out = torch.empty_like(q)
        if fused:
            # the fused step computes its own slots from the tables: reserve
            # the positions (and copy shared blocks) first, then append+attend
            slots, copies = mgr.append([(s, 1) for s in live])
            copies_seen += len(copies)
            if len(copies):
                pa.copy_blocks(kc, vc, copies, ks, vs)
            kn, vn = _rows(rng, len(live), hkv, d, fmt), _rows(rng, len(live), hkv, d, fmt)
            for i, s in enumerate(live):
                dense.append(s, host(kn)[i], host(vn)[i])
        else:
            append([(s, 1) for s in live])
        maxb = max(-(-mgr.length(s) // bs) for s in live)
        tables, lens = mgr.block_tables(live, maxb)
        bt, ctx = torch.from_numpy(tables).to(dev()), torch.from_numpy(lens).to(dev())
        print(f"{fmt} round {rounds}: {len(live)} seqs, ctx max {int(lens.max())}, "
              f"fused={fused}", flush=True)
        if fused:
            pa.decode_step(q.contiguous(), kn, vn, kc, vc, bt, ctx, scale, out)
        elif i8:
            pa.paged_decode_attention_int8(q, kc, vc, ks, vs, bt, ctx, scale, out)
        else:
            pa.paged_decode_attention(q, kc, vc, bt, ctx, scale, out)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()
        qh = q.double().cpu().numpy()
        err = 0.0
        for i, s in enumerate(live):
            K, V = _dense_kv(dense, s, fmt, orc)
            for h in range(hq):
                ref, _ = oracle.attention_dense(qh[i, h], K[:, h // g], V[:, h // g], scale,
                                                lib=orc)
                err = max(err, float(np.max(np.abs(got[i, h] - ref))))
        assert err <= TOL[fmt], (rounds, err)
        # every live sequence un-pages to exactly its rows
        nk = torch.empty((len(live), maxb * bs, hkv, d), dtype=cdt, device=dev())
        nv = torch.empty_like(nk)
        sk = sv = None
        if i8:
            sk = torch.empty((len(live), maxb * bs, hkv), dtype=torch.float16, device=dev())
            sv = torch.empty_like(sk)
        pa.gather_kv(kc, vc, bt, ctx, nk, nv, ks, vs, sk, sv)
        gk, gv = host(nk), host(nv)
        for i, s in enumerate(live):
            k, v = dense.kv(s)
            n = k.shape[0]
            if i8:
                for (rows, codes, scales) in ((k, gk, host(sk)), (v, gv, host(sv))):
                    for j in range(n):
                        for h in range(hkv):
                            c, sc = oracle.quantize_row_int8(rows[j, h], lib=orc)
                            assert np.array_equal(codes[i, j, h], c)
                            assert scales[i, j, h].view(np.uint16) == np.float16(sc).view(np.uint16)
            else:
                assert np.array_equal(gk[i, :n].view(np.uint8), k.view(np.uint8))
                assert np.array_equal(gv[i, :n].view(np.uint8), v.view(np.uint8))

    for step in range(40):
        op = rng.integers(5)
        if op == 0 or len(live) < 2:
            s = mgr.add()
            dense.add(s)
            live.append(s)
            try:
                append([(s, int(rng.integers(1, 70)))])
            except pa.OutOfBlocks:
                live.pop()
                mgr.free(s)
                dense.free(s)
        elif op == 1 and len(live) < 8:
            p = live[int(rng.integers(len(live)))]
            pre = int(rng.integers(0, mgr.length(p) + 1))
            s = mgr.fork(p, pre)
            dense.fork(p, s, pre)
            live.append(s)
        elif op == 2 and len(live) > 2:
            s = live.pop(int(rng.integers(len(live))))
            mgr.free(s)
            dense.free(s)
        else:
            try:
                decode_round(fused=not i8 and step % 2 == 0)
            except pa.OutOfBlocks:
                s = live.pop(0)
                mgr.free(s)
                dense.free(s)
    assert rounds >= 10 and copies_seen >= 1
