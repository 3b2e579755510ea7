"""The library's native block manager (pa_bm_*) against the block-pool oracle
model, on the host (no GPU).  Block numbers are the managers' own choice, so
the two are compared on what is unique: lengths, which table entries alias
one block, free counts, reference counts, which requests copied a block,
and which requests fail; slots must follow each manager's own tables."""
import ctypes

import numpy as np
import pytest

import block_manager_pins as pins
import decode_attention_paged_append_amd as pa
import oracle
from oracle import block_manager as bm


class Lockstep:
    def __init__(self, nb, bs):
        self.nat = pa.BlockManager(nb, bs)
        self.ora = bm.BlockManager(nb, bs)
        self.bs = bs
        self.handles = []           # [(native id, oracle id)] of live sequences

    def check(self):
        nat_tabs = [self.nat.block_tables([n], 1 + self.nat.length(n) // self.bs)[0][0]
                    for n, _ in self.handles]
        nat_tabs = [[int(b) for b in t if b >= 0] for t in nat_tabs]
        ora_tabs = [self.ora.table(o) for _, o in self.handles]
        assert bm.aliasing(nat_tabs) == bm.aliasing(ora_tabs)
        for (n, o), nt, ot in zip(self.handles, nat_tabs, ora_tabs):
            assert self.nat.length(n) == self.ora.length(o)
            assert len(nt) == -(-self.nat.length(n) // self.bs)
            for a, b in zip(nt, ot):
                assert self.nat.ref_count(a) == self.ora.ref[b]
        assert self.nat.num_free() == self.ora.num_free()

    def add(self):
        self.handles.append((self.nat.add(), self.ora.add()))

    def fork(self, i, prefix):
        n, o = self.handles[i]
        self.handles.append((self.nat.fork(n, prefix), self.ora.fork(o, prefix)))

    def free(self, i):
        n, o = self.handles.pop(i)
        self.nat.free(n)
        self.ora.free(o)

    def append(self, reqs):
        """reqs: [(handle index, n)].  Returns True if both accepted it."""
        nat_err = ora_err = None
        try:
            slots, copies = self.nat.append([(self.handles[i][0], n) for i, n in reqs])
        except pa.OutOfBlocks as e:
            nat_err = e
        try:
            oslots, ocopies = self.ora.append([(self.handles[i][1], n) for i, n in reqs])
        except bm.OutOfBlocks as e:
            ora_err = e
        assert (nat_err is None) == (ora_err is None), (nat_err, ora_err)
        if nat_err is not None:
            return False
        # slots follow the native tables, position by position
        t = 0
        for i, n in reqs:
            sid = self.handles[i][0]
            tab = self.nat.block_tables([sid], 1 + self.nat.length(sid) // self.bs)[0][0]
            start = self.nat.length(sid) - n
            for p in range(start, start + n):
                assert slots[t] == tab[p // self.bs] * self.bs + p % self.bs
                t += 1
        assert t == slots.size == sum(len(r) for r in oslots)
        # the same requests copied, each its own last block before the append
        def copiers(copies, table_of):
            who = []
            for src, dst in copies:
                who.append([i for i, _ in reqs if dst in table_of(i)])
            return who
        nat_who = copiers(copies.tolist(), lambda i: list(self.nat.block_tables(
            [self.handles[i][0]], 1 + self.nat.length(self.handles[i][0]) // self.bs)[0][0]))
        ora_who = copiers(ocopies, lambda i: self.ora.table(self.handles[i][1]))
        assert nat_who == ora_who
        return True


def random_script(ls, rng, steps, max_live=8, sizes=(0, 1, 1, 1, 2, 3, 9, 17)):
    for _ in range(steps):
        op = rng.integers(6)
        if op == 0 and len(ls.handles) < max_live or not ls.handles:
            ls.add()
        elif op == 1 and len(ls.handles) < max_live:
            i = int(rng.integers(len(ls.handles)))
            ls.fork(i, int(rng.integers(0, ls.ora.length(ls.handles[i][1]) + 1)))
        elif op == 2 and len(ls.handles) > 1:
            ls.free(int(rng.integers(len(ls.handles))))
        else:
            idx = [i for i in range(len(ls.handles)) if rng.random() < 0.6]
            ls.append([(i, int(rng.choice(sizes))) for i in idx])
        ls.check()


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("nb,bs", [(64, 4), (24, 4), (40, 16), (512, 8)])
def test_lockstep_with_oracle(seed, nb, bs):
    ls = Lockstep(nb, bs)
    random_script(ls, np.random.default_rng(seed), 300)
    while ls.handles:
        ls.free(0)
        ls.check()
    assert ls.nat.num_free() == nb


def test_pool_exhaustion_changes_nothing():
    ls = Lockstep(3, 4)
    ls.add()
    assert ls.append([(0, 5)])
    ls.fork(0, 5)
    before = (ls.nat.num_free(), ls.nat.block_tables([0, 1], 3))
    assert not ls.append([(0, 8)])          # copy + 2 new blocks > 1 free
    after = (ls.nat.num_free(), ls.nat.block_tables([0, 1], 3))
    assert before[0] == after[0] and all(np.array_equal(a, b) for a, b in zip(before[1], after[1]))
    ls.check()
    assert ls.append([(0, 1), (1, 1)])      # one copy; the second holder writes in place
    ls.check()


class NativeAsModel:
    """The native manager behind the oracle model's interface, so the dense
    equivalence pin can drive it directly."""
    OutOfBlocks = pa.OutOfBlocks
    DenseRows = bm.DenseRows
    copy_block_rows = staticmethod(bm.copy_block_rows)

    class BlockManager:
        def __init__(self, nb, bs):
            self.m = pa.BlockManager(nb, bs)
            self.bs = bs

        def add(self):
            return self.m.add()

        def fork(self, p, prefix=None):
            return self.m.fork(p, prefix)

        def free(self, s):
            self.m.free(s)

        def length(self, s):
            return self.m.length(s)

        def num_free(self):
            return self.m.num_free()

        def table(self, s):
            t = self.m.block_tables([s], 1 + self.m.length(s) // self.bs)[0][0]
            return [int(b) for b in t if b >= 0]

        def append(self, reqs):
            slots, copies = self.m.append(reqs)
            out, t = [], 0
            for _, n in reqs:
                out.append(slots[t:t + n].tolist())
                t += n
            return out, [tuple(c) for c in copies.tolist()]


@pytest.mark.parametrize("seed", range(4))
def test_native_manager_unpages_to_dense_rows(seed, orc):
    pins.pin_dense_equivalence(NativeAsModel, lib=orc, steps=200, seed=seed)


def test_argument_checks():
    m = pa.BlockManager(8, 4)
    a = m.add()
    with pytest.raises(pa.PagedAttnError, match="not live"):
        m.append([(a + 5, 1)])
    with pytest.raises(pa.PagedAttnError, match="twice"):
        m.append([(a, 1), (a, 2)])
    with pytest.raises(pa.PagedAttnError, match="tokens"):
        m.append([(a, -1)])
    m.append([(a, 3)])
    with pytest.raises(pa.PagedAttnError, match="longer"):
        m.fork(a, 4)
    with pytest.raises(pa.OutOfBlocks):
        m.append([(a, 8 * 4)])
    m.free(a)
    with pytest.raises(pa.PagedAttnError, match="not live"):
        m.free(a)
    with pytest.raises(pa.PagedAttnError, match="block_size"):
        pa.BlockManager(8, 12)
    with pytest.raises(pa.PagedAttnError, match="positive"):
        pa.BlockManager(0, 4)
    # buffers too small, through the C ABI directly: nothing may change
    lib = pa.library()
    b = m.add()
    m.append([(b, 2)])
    c = m.fork(b)
    seqs = (ctypes.c_int32 * 1)(b)
    ntok = (ctypes.c_int32 * 1)(3)
    slots = (ctypes.c_int64 * 2)()
    copies = (ctypes.c_int32 * 2)()
    n = ctypes.c_int32()
    assert lib.pa_bm_append(m._h, seqs, ntok, 1, slots, 2, copies, 1, ctypes.byref(n)) == 1
    assert b"slots buffer" in lib.pa_last_error()
    slots3 = (ctypes.c_int64 * 3)()
    assert lib.pa_bm_append(m._h, seqs, ntok, 1, slots3, 3, copies, 0, ctypes.byref(n)) == 1
    assert b"copies buffer" in lib.pa_last_error()
    assert m.length(b) == 2 and m.num_free() == 7 and m.ref_count(m.block_tables([b], 1)[0][0, 0]) == 2
    assert lib.pa_bm_append(m._h, seqs, ntok, 1, slots3, 3, copies, 1, ctypes.byref(n)) == 0
    assert n.value == 1 and m.length(b) == 5 and m.length(c) == 2
    with pytest.raises(pa.PagedAttnError, match="holds"):
        m.block_tables([b], 1)
    assert m.ref_count(-1) == -1 and m.ref_count(8) == -1 and m.length(99) == -1


def test_ids_are_reused_after_free():
    m = pa.BlockManager(8, 4)
    a, b = m.add(), m.add()
    m.free(a)
    c = m.add()
    assert c == a and m.length(c) == 0 and m.block_tables([c], 2)[0].tolist() == [[-1, -1]]
    assert m.length(b) == 0
