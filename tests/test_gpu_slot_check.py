"""pa_check_slot_mapping on the GPU (needs an MI355X): its flags against the
oracle's own validation of an append (which rejects a slot used twice and a
slot outside the pool) and against a count of the slots on the host, on
seeded mappings that span several 256-slot tiles, with pads, and on the
decode slots of real layouts -- including two sequences whose tables share
a block they would both append into (a missing copy-on-write)."""
import numpy as np
import pytest
import torch

import decode_attention_paged_append_amd as pa
import oracle
import workloads as W
from gpu_cases import dev

pytestmark = pytest.mark.gpu


def host_flags(slots, pool_slots):
    """The two properties counted on the host (test-side numpy)."""
    live = slots[slots >= 0]
    repeated = np.unique(live).size != live.size
    outside = bool((slots >= pool_slots).any())
    return (pa.SLOT_REPEATED if repeated else 0) | (pa.SLOT_OUTSIDE_POOL if outside else 0)


def oracle_status(slots, pool_slots, block_size=16):
    """The oracle append's status on these slots: 0, -2 (outside) or -3 (repeated)."""
    nb = pool_slots // block_size
    t = slots.shape[0]
    kc = np.zeros((nb, 1, block_size, 4), np.float32)
    kn = np.zeros((t, 1, 4), np.float32)
    try:
        oracle.kv_append(kn, kn, slots, kc, kc.copy())
        return 0
    except oracle.OracleError as e:
        return {"slot outside the pool": -2, "slot used twice": -3}[str(e)]


def gpu_flags(slots, pool_slots):
    f = pa.check_slot_mapping(torch.from_numpy(slots).to(dev()), pool_slots)
    torch.cuda.synchronize()
    return int(f.item())


@pytest.mark.parametrize("t", [1, 2, 255, 256, 257, 1000, 4099])
def test_flags_match_oracle_and_host(t):
    rng = np.random.default_rng(t)
    pool_slots = 16 * (t + 50)
    base = rng.permutation(pool_slots)[:t].astype(np.int64)
    base[rng.random(t) < 0.1] = -1                       # pads
    print(f"slot check t={t}", flush=True)
    assert gpu_flags(base, pool_slots) == 0 == host_flags(base, pool_slots)
    assert oracle_status(base, pool_slots) == 0
    if t >= 2:
        # a repeat: the last token takes an earlier live slot (same or earlier tile)
        live = np.flatnonzero(base >= 0)
        dup = base.copy()
        i, j = live[0], t - 1
        dup[j] = base[i]
        assert gpu_flags(dup, pool_slots) == pa.SLOT_REPEATED == host_flags(dup, pool_slots)
        assert oracle_status(dup, pool_slots) == -3
        # a repeat inside the last tile only
        dup2 = base.copy()
        dup2[t - 1] = 5
        dup2[max(0, t - 2)] = 5
        if t - 2 >= 0 and t >= 2:
            assert gpu_flags(dup2, pool_slots) & pa.SLOT_REPEATED
    out = base.copy()
    out[t // 2] = pool_slots + 3
    assert gpu_flags(out, pool_slots) == pa.SLOT_OUTSIDE_POOL == host_flags(out, pool_slots)
    assert oracle_status(out, pool_slots) == -2
    if t >= 4:          # the repeated pair does not overwrite the outside slot
        both = out.copy()
        k = (t // 2 + 1) % t
        both[k] = both[(k + 1) % t] = 7
        assert gpu_flags(both, pool_slots) == host_flags(both, pool_slots) == 3


def test_pads_never_compare_and_empty_is_clean():
    pads = np.full(300, -1, np.int64)
    assert gpu_flags(pads, 64) == 0
    assert gpu_flags(np.zeros(0, np.int64), 64) == 0


def test_decode_slots_of_a_layout_are_clean_and_a_shared_block_is_caught():
    """The decode slots of a carved layout never repeat; two sequences whose
    tables share their last block (a fork whose copy-on-write was skipped)
    would append into one slot, and the check says so."""
    bs = 16
    lay = W.carve_layout([17, 40, 1, 32, 100], bs, num_blocks=64, seed=4)
    bt, ctx = lay.block_tables.to(dev()), lay.context_lens.to(dev())
    slots = pa.decode_slot_mapping(bt, ctx, bs)
    f = pa.check_slot_mapping(slots, 64 * bs)
    torch.cuda.synchronize()
    assert int(f.item()) == 0
    tables = lay.block_tables.clone()
    lens = lay.context_lens.clone()
    lens[1] = lens[0]                                    # same position ...
    tables[1, :2] = tables[0, :2]                        # ... in the same blocks
    slots = pa.decode_slot_mapping(tables.to(dev()), lens.to(dev()), bs)
    f = pa.check_slot_mapping(slots, 64 * bs)
    torch.cuda.synchronize()
    assert int(f.item()) == pa.SLOT_REPEATED
