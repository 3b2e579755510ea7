"""Checks that tie the block-pool model (oracle/block_manager.py) to the
paging rules of the pages, and to the plain definition of a sequence's cache.

Each ``pin_*`` function takes the model module and raises AssertionError when
the model breaks a rule fixed outside itself:
  - the visualization page's rules ("PagedAttention: the cache in blocks"):
    a new block only when the last one is full, hence at most one partly
    filled block; slot = table[pos // BS] * BS + pos % BS; a prefix shared by
    reference; a shared block copied only when written;
  - the guide's "Paging": blocks come back as soon as a request finishes;
  - the definition: paging changes where rows sit, never what a sequence
    holds -- un-paging a sequence through the model's tables (with the oracle's
    own append and gather on a host pool) gives back exactly the rows appended
    to it, in order (DenseRows).
test_block_manager_oracle.py runs them against the model and against copies
of it with planted mistakes, each of which some pin must catch.
"""
from __future__ import annotations

import numpy as np

import oracle


def _ceil(a, b):
    return -(-a // b)


def _refs_match_tables(m):
    counts = [0] * m.num_blocks
    for s in m.seqs:
        for b in m.table(s):
            counts[b] += 1
    assert counts == m.ref, "reference counts differ from the table entries"


def pin_block_count_and_waste(bm):
    for bs in (4, 16):
        for n in range(0, 3 * bs + 2):
            one = bm.BlockManager(16, bs)
            a = one.add()
            slots, copies = one.append([(a, n)])
            assert copies == []
            assert len(one.table(a)) == _ceil(n, bs)
            waste = len(one.table(a)) * bs - n
            assert 0 <= waste < bs or n == 0
            step = bm.BlockManager(16, bs)
            b = step.add()
            for i in range(n):
                step.append([(b, 1)])
                assert len(step.table(b)) == _ceil(i + 1, bs), "block taken before the last was full"
            assert step.length(b) == one.length(a) == n


def pin_slots_follow_table(bm):
    rng = np.random.default_rng(11)
    m = bm.BlockManager(64, 4)
    seqs = [m.add() for _ in range(3)]
    written = {}
    for _ in range(12):
        reqs = [(s, int(rng.integers(0, 6))) for s in seqs]
        start = {s: m.length(s) for s in seqs}
        slots, _ = m.append(reqs)
        flat = [x for row in slots for x in row]
        assert len(set(flat)) == len(flat), "two tokens of one append share a slot"
        for (s, n), row in zip(reqs, slots):
            t = m.table(s)
            for i, slot in enumerate(row):
                pos = start[s] + i
                assert slot == t[pos // 4] * 4 + pos % 4
                written[(s, pos)] = slot
    # distinct live positions never share a slot (no sharing without a fork)
    assert len(set(written.values())) == len(written)


def pin_prefix_sharing(bm):
    bs = 16
    m = bm.BlockManager(32, bs)
    a = m.add()
    m.append([(a, 64)])
    b = m.fork(a)
    assert m.table(b) == m.table(a)
    assert m.num_free() == 32 - 4, "a shared 64-token prompt must use 4 blocks, not 8"
    _, copies = m.append([(a, 1), (b, 1)])
    assert copies == [], "appending past a full shared block copies nothing"
    assert m.num_free() == 32 - 6 and m.table(a)[:4] == m.table(b)[:4]
    # a prefix that ends inside a block: the first writer copies it, the
    # second writes in place
    c = m.add()
    m.append([(c, 70)])
    d = m.fork(c, 70)
    shared = m.table(c)[4]
    assert m.ref[shared] == 2
    _, copies = m.append([(d, 1)])
    assert len(copies) == 1 and copies[0][0] == shared
    assert m.table(d)[4] == copies[0][1] != shared and m.ref[shared] == 1
    _, copies = m.append([(c, 1)])
    assert copies == [] and m.table(c)[4] == shared
    _refs_match_tables(m)


def pin_fork_prefix_lengths(bm):
    m = bm.BlockManager(64, 4)
    a = m.add()
    m.append([(a, 13)])
    for p in range(0, 14):
        c = m.fork(a, p)
        assert m.length(c) == p and m.table(c) == m.table(a)[:_ceil(p, 4)]
        m.free(c)
    _refs_match_tables(m)


def pin_copy_only_on_write(bm):
    m = bm.BlockManager(16, 4)
    a = m.add()
    m.append([(a, 6)])
    before = m.num_free()
    b = m.fork(a)
    assert m.num_free() == before, "a fork takes no blocks"
    m.free(b)
    assert m.num_free() == before
    c = m.fork(a)
    _, copies = m.append([(a, 1)])
    assert len(copies) == 1, "writing a shared block copies it once"
    _, copies = m.append([(a, 1), (c, 1)])
    assert copies == [], "blocks no longer shared are written in place"
    _refs_match_tables(m)


def pin_reclaim(bm):
    rng = np.random.default_rng(5)
    m = bm.BlockManager(40, 4)
    live = []
    for _ in range(200):
        op = rng.integers(4)
        if op == 0 or not live:
            live.append(m.add())
        elif op == 1:
            p = live[int(rng.integers(len(live)))]
            live.append(m.fork(p, int(rng.integers(0, m.length(p) + 1))))
        elif op == 2:
            reqs = [(s, int(rng.integers(0, 4))) for s in live if rng.random() < 0.5]
            try:
                m.append(reqs)
            except bm.OutOfBlocks:
                pass
        else:
            m.free(live.pop(int(rng.integers(len(live)))))
        _refs_match_tables(m)
        for s in live:
            assert len(m.table(s)) == _ceil(m.length(s), 4)
    for s in live:
        m.free(s)
    assert m.num_free() == 40 and sum(m.ref) == 0, "finished requests must return every block"


def pin_out_of_blocks_all_or_nothing(bm):
    m = bm.BlockManager(2, 4)
    a = m.add()
    m.append([(a, 2)])
    b = m.fork(a)
    snap = (m.table(a), m.table(b), list(m.ref), m.length(a), m.length(b))
    # a copy of the shared block plus one block boundary: 2 blocks, 1 free
    assert m.blocks_needed(a, 3) == 2
    try:
        m.append([(a, 3)])
        raise AssertionError("append beyond the pool succeeded")
    except bm.OutOfBlocks:
        pass
    assert snap == (m.table(a), m.table(b), list(m.ref), m.length(a), m.length(b)), \
        "a failed append changed the state"
    m.append([(a, 1), (b, 1)])                    # one copy fits
    assert m.num_free() == 0


def pin_dense_equivalence(bm, lib=None, steps=160, seed=3):
    """Drive the model with a seeded script and a host pool written by the
    oracle's append; every live sequence must un-page to its dense rows."""
    rng = np.random.default_rng(seed)
    nb, bs, hkv, d = 48, 4, 2, 8
    m = bm.BlockManager(nb, bs)
    dense = bm.DenseRows()
    kc = np.full((nb, hkv, bs, d), np.nan, np.float32)
    vc = np.full((nb, hkv, bs, d), np.nan, np.float32)
    live = []
    for _ in range(steps):
        op = rng.integers(5)
        if op == 0 or not live:
            s = m.add()
            dense.add(s)
            live.append(s)
        elif op == 1:
            p = live[int(rng.integers(len(live)))]
            pre = int(rng.integers(0, m.length(p) + 1))
            s = m.fork(p, pre)
            dense.fork(p, s, pre)
            live.append(s)
        elif op == 4 and len(live) > 1:
            s = live.pop(int(rng.integers(len(live))))
            m.free(s)
            dense.free(s)
        else:
            reqs = [(s, int(rng.choice([0, 1, 1, 2, 3, 7]))) for s in live if rng.random() < 0.7]
            try:
                slots, copies = m.append(reqs)
            except bm.OutOfBlocks:
                continue
            bm.copy_block_rows(kc, copies)
            bm.copy_block_rows(vc, copies)
            flat = np.array([x for row in slots for x in row], np.int64)
            kn = rng.standard_normal((flat.size, hkv, d)).astype(np.float32)
            vn = rng.standard_normal((flat.size, hkv, d)).astype(np.float32)
            if flat.size:
                oracle.kv_append(kn, vn, flat, kc, vc, lib=lib)
            t = 0
            for (s, n) in reqs:
                for _ in range(n):
                    dense.append(s, kn[t], vn[t])
                    t += 1
        # un-page every live sequence and compare with its dense rows
        for s in live:
            n = m.length(s)
            assert n == len(dense.rows[s]), "sequence length differs from its rows"
            if n == 0:
                continue
            table = np.array([m.table(s) + [-1] * (64 - len(m.table(s)))], np.int32)
            ko = np.zeros((1, 64 * bs, hkv, d), np.float32)
            vo = np.zeros_like(ko)
            oracle.gather_kv(kc, vc, table, np.array([n], np.int32), ko, vo, lib=lib)
            k_ref, v_ref = dense.kv(s)
            assert np.array_equal(ko[0, :n], k_ref) and np.array_equal(vo[0, :n], v_ref), \
                f"sequence {s} un-pages to other rows than were appended to it"
    for s in live:
        m.free(s)
    assert m.num_free() == nb


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
