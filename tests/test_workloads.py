"""Byte counts the bench reports, on hand-made layouts, and its one-GPU guard
(CPU only)."""
import os

import workloads as W


def _shape(dtype="f16"):
    return W.Shape("t", dtype, 2, 4, 2, 64, 16)


def test_unique_bytes_equal_logical_without_sharing():
    sh = _shape()
    lay = W.carve_layout([40, 7, 33], 16, seed=4)
    assert int(lay.owners.max()) == 1
    assert (W.unique_kv_bytes_per_layer_step(sh, lay)
            == W.kv_bytes_per_layer_step(sh, lay.context_lens.tolist()))


def test_unique_bytes_count_a_shared_prefix_once():
    # two sequences share a 32-token prefix (two blocks of 16); the second
    # uses 4 rows of the second shared block, the first all 16 and 8 more
    sh = _shape()
    lay = W.carve_layout([40, 20], 16, prefix_group=2, prefix_tokens=32, seed=4)
    assert int(lay.owners.max()) == 2
    per_row = sh.num_kv_heads * sh.head_dim * 2 * 2
    assert W.kv_bytes_per_layer_step(sh, [40, 20]) == 60 * per_row
    assert W.unique_kv_bytes_per_layer_step(sh, lay) == (16 + 16 + 8) * per_row


def test_unique_bytes_of_quantized_caches_carry_scales():
    lay = W.carve_layout([40, 20], 16, prefix_group=2, prefix_tokens=32, seed=4)
    i8 = W.unique_kv_bytes_per_layer_step(_shape("i8"), lay)
    assert i8 == 40 * 2 * 2 * (64 + 2)
    i4 = W.unique_kv_bytes_per_layer_step(_shape("i4"), lay)
    assert i4 == 40 * 2 * 2 * (32 + 2 * 2)


def test_bench_rejects_more_than_one_gpu():
    """bench.py measures one GPU; --gpus above 1 exits with a message before
    touching a device."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
