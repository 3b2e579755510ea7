"""The block-pool model against its pins, and planted mistakes in copies of
the model, each of which some pin must catch (no GPU)."""
import sys
import types

import pytest

import block_manager_pins as pins
import oracle
from oracle import block_manager as bm

SOURCE = bm.__file__


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, orc):
    if pin is pins.pin_dense_equivalence:
        pin(bm, lib=orc)
    else:
        pin(bm)


MUTANTS = {
    "no copy before writing a shared block": ("if self.ref[last] > 1:", "if False:"),
    "copy on every write": ("if self.ref[last] > 1:", "if self.ref[last] >= 1:"),
    "copy direction reversed": ("copies.append((last, fresh))", "copies.append((fresh, last))"),
    "source keeps its count after a copy": (
        "copies.append((last, fresh))\n                        self._drop(last)",
        "copies.append((last, fresh))"),
    "fork shares whole blocks only": ("nblocks = -(-n // self.block_size)",
                                      "nblocks = n // self.block_size"),
    "fork takes the whole parent": ("n = p.length if prefix is None else prefix", "n = p.length"),
    "finished request keeps its blocks": ("for b in s.table:\n            self._drop(b)",
                                          "for b in s.table:\n            pass"),
    "copy not counted before an append": (
        "need += 1\n                ref[s.table[-1]] -= 1", "ref[s.table[-1]] -= 1"),
    "every sharer counted as copying": (
        "need += 1\n                ref[s.table[-1]] -= 1", "need += 1"),
    "new block one slot early": ("if pos % bs == 0:", "if pos % bs == 0 or pos % bs == bs - 1:"),
    "slot offset from the block index": ("mine.append(s.table[pos // bs] * bs + pos % bs)",
                                         "mine.append(s.table[pos // bs] * bs + pos // bs % bs)"),
    "dense fork copies the whole parent": ("n = len(src) if prefix is None else prefix",
                                           "n = len(src)"),
    "block copy ignores its list": ("cache[dst] = cache[src]", "pass"),
}


def _load_mutant(old, new):
    src = open(SOURCE).read()
    assert src.count(old) == 1, f"mutation site not found exactly once: {old!r}"
    mod = types.ModuleType("block_manager_mutant")
    mod.__file__ = "<mutant>"
    sys.modules[mod.__name__] = mod          # dataclasses look the module up
    try:
        exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    finally:
        del sys.modules[mod.__name__]
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, orc):
    mod = _load_mutant(*MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            if pin is pins.pin_dense_equivalence:
                pin(mod, lib=orc)
            else:
                pin(mod)
        except (AssertionError, IndexError, KeyError, ValueError, mod.OutOfBlocks,
                oracle.OracleError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant '{name}'"
