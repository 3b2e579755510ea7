"""Plain model of the block pool that feeds the paged cache.

TEST INFRASTRUCTURE ONLY: the tests use it to check the library's native
block manager.  Nothing in the product path imports it.

The rules are those of the KV-cache visualization page, "PagedAttention: the
cache in blocks", with one step from the jovanaeducation guide, "Paging":
  - the cache is cut into blocks of a fixed number of token slots, all drawn
    from one shared pool;
  - every request keeps a block table: its block numbers, in order, so that
    position pos lives in slot table[pos // BS] * BS + pos % BS;
  - a request takes a new block only when its last block is full, so at most
    one of its blocks is partly filled;
  - a finished request gives its blocks back at once (guide, "Paging");
  - two requests with a common prefix point at the same blocks for it, and a
    shared block is copied only when one of them writes into it.

Readings where the pages stop short:
  - A block is shared by reference count.  Writing into a block whose count is
    above one first moves the writer onto a fresh copy of it (the count of the
    old block drops by one); the last holder writes in place.
  - A fork shares the first ceil(prefix / BS) blocks of the parent.  When the
    prefix ends inside a block, that block is shared too, and the first write
    of either side into it copies it.
  - Which free block is handed out is not fixed by the pages.  The model takes
    the lowest-numbered free block; results are compared on what is unique (the
    contents a sequence sees, which table entries alias one block, counts),
    never on block numbers.
  - An append that would need more blocks than are free changes nothing and
    fails (the pages leave eviction out).

DenseRows is the plainest statement of what a sequence's cache holds: the K
and V rows appended to it, in order, with a fork starting from a copy of its
parent's first rows.  No blocks at all.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


@dataclass
class _Seq:
    table: list[int] = field(default_factory=list)
    length: int = 0


class BlockManager:
    """Pool of num_blocks blocks of block_size slots, shared by sequences."""

    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("pool sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.seqs: dict[int, _Seq] = {}
        self._next_id = 0

    # -- pool
    def free_blocks(self) -> list[int]:
        return [b for b in range(self.num_blocks) if self.ref[b] == 0]

    def num_free(self) -> int:
        return len(self.free_blocks())

    def _take(self) -> int:
        free = self.free_blocks()
        if not free:
            raise OutOfBlocks("pool exhausted")
        self.ref[free[0]] = 1
        return free[0]

    def _drop(self, block: int) -> None:
        assert self.ref[block] > 0
        self.ref[block] -= 1

    # -- sequences
    def add(self) -> int:
        sid = self._next_id
        self._next_id += 1
        self.seqs[sid] = _Seq()
        return sid

    def fork(self, parent: int, prefix: int | None = None) -> int:
        p = self.seqs[parent]
        n = p.length if prefix is None else prefix
        if not 0 <= n <= p.length:
            raise ValueError("prefix longer than the parent")
        nblocks = -(-n // self.block_size)
        sid = self.add()
        child = self.seqs[sid]
        child.table = list(p.table[:nblocks])
        child.length = n
        for b in child.table:
            self.ref[b] += 1
        return sid

    def free(self, sid: int) -> None:
        s = self.seqs.pop(sid)
        for b in s.table:
            self._drop(b)

    def blocks_needed(self, sid: int, n: int) -> int:
        """Fresh blocks an append of n tokens takes: one per block boundary
        crossed, plus one copy when the first write lands in a shared block."""
        s = self.seqs[sid]
        if n == 0:
            return 0
        bs = self.block_size
        new = -(-(s.length + n) // bs) - (-(-s.length // bs))
        cow = 1 if s.length % bs and self.ref[s.table[-1]] > 1 else 0
        return new + cow

    def batch_blocks_needed(self, requests) -> int:
        """Fresh blocks a batch of appends takes, in request order: once one
        sharer of a block has copied it away, the next holder may be its
        only one and writes in place."""
        ref = list(self.ref)
        bs = self.block_size
        need = 0
        for sid, n in requests:
            s = self.seqs[sid]
            if n == 0:
                continue
            need += -(-(s.length + n) // bs) - (-(-s.length // bs))
            if s.length % bs and ref[s.table[-1]] > 1:
                need += 1
                ref[s.table[-1]] -= 1
        return need

    def append(self, requests: list[tuple[int, int]]):
        """Reserve slots for requests [(seq, n_tokens)], all or nothing.

        Returns (slots, copies): slots[i] lists the slots of request i in
        position order; copies lists (source, destination) block pairs whose
        contents must be copied before anything is written to the slots."""
        sids = [sid for sid, _ in requests]
        if len(set(sids)) != len(sids):
            raise ValueError("a sequence appears twice")
        if any(n < 0 for _, n in requests):
            raise ValueError("negative token count")
        need = self.batch_blocks_needed(requests)
        if need > self.num_free():
            raise OutOfBlocks(f"need {need} blocks, {self.num_free()} free")
        slots, copies = [], []
        bs = self.block_size
        for sid, n in requests:
            s = self.seqs[sid]
            mine = []
            for _ in range(n):
                pos = s.length
                if pos % bs == 0:
                    s.table.append(self._take())
                else:
                    last = s.table[-1]
                    if self.ref[last] > 1:            # first write into a shared block
                        fresh = self._take()
                        copies.append((last, fresh))
                        self._drop(last)
                        s.table[-1] = fresh
                mine.append(s.table[pos // bs] * bs + pos % bs)
                s.length += 1
            slots.append(mine)
        return slots, copies

    def table(self, sid: int) -> list[int]:
        return list(self.seqs[sid].table)

    def length(self, sid: int) -> int:
        return self.seqs[sid].length


class DenseRows:
    """Each sequence's K and V rows in append order (no paging)."""

    def __init__(self):
        self.rows: dict[int, list[tuple[np.ndarray, np.ndarray]]] = {}

    def add(self, sid: int) -> None:
        self.rows[sid] = []

    def fork(self, parent: int, child: int, prefix: int | None = None) -> None:
        src = self.rows[parent]
        n = len(src) if prefix is None else prefix
        self.rows[child] = [(k.copy(), v.copy()) for k, v in src[:n]]

    def free(self, sid: int) -> None:
        del self.rows[sid]

    def append(self, sid: int, k: np.ndarray, v: np.ndarray) -> None:
        self.rows[sid].append((k.copy(), v.copy()))

    def kv(self, sid: int) -> tuple[np.ndarray, np.ndarray]:
        """[len, ...] arrays of the sequence's K and V rows."""
        ks = [k for k, _ in self.rows[sid]]
        vs = [v for _, v in self.rows[sid]]
        return np.stack(ks), np.stack(vs)


def copy_block_rows(cache: np.ndarray, copies) -> None:
    """Carry out a list of (source, destination) block copies on a host pool
    laid out [num_blocks][...]."""
    for src, dst in copies:
        cache[dst] = cache[src]


def aliasing(tables: list[list[int]]) -> list[list[int]]:
    """Rename block numbers by first appearance over the tables in order, so
    two managers that share and copy the same way give equal results."""
    names: dict[int, int] = {}
    out = []
    for t in tables:
        out.append([names.setdefault(b, len(names)) for b in t])
    return out
