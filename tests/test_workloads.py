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


def test_traffic_record_from_counter_csvs(tmp_path):
    """bench.py --traffic-from: each counter's mean per dispatch (a dispatch's
    rows summed), scaled by the 1 GiB copy's reading of the same counter."""
    import importlib.util
    import json

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    k = "void pa::decode_partition_kernel<(pa::Fmt)1, 128, 16, 1, 4>(pa::DecodeParams)"
    rows = {
        "pmc_fetch": [(1, k, "FETCH_SIZE", 300.0), (1, k, "FETCH_SIZE", 100.0),
                      (2, k, "FETCH_SIZE", 600.0), (3, "other", "FETCH_SIZE", 9e9)],
        "pmc_write": [(1, k, "WRITE_SIZE", 10.0), (2, k, "WRITE_SIZE", 30.0)],
        "pmc_copy_fetch": [(7, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)],
        "pmc_copy_write": [(7, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)],
    }
    for sub, rr in rows.items():
        (tmp_path / sub).mkdir()
        with open(tmp_path / sub / "run_counter_collection.csv", "w") as f:
            f.write(head + "".join(f'{d},"{n}",{c},{v}\n' for d, n, c, v in rr))
    out = tmp_path / "traffic.json"
    rec = bench.write_traffic_record(str(tmp_path), str(out))
    # fetch: dispatches 400 and 600 KiB -> 500 KiB, x2 (the copy's fetch reads half);
    # write: 20 KiB, x1
    assert rec["fetch_kib_per_dispatch"] == 500.0 and rec["write_kib_per_dispatch"] == 20.0
    assert rec["copy_fetch_factor"] == 2.0 and rec["copy_write_factor"] == 1.0
    assert rec["traffic_bytes_per_launch"] == 500 * 1024 * 2 + 20 * 1024
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
    assert json.loads(out.read_text()) == rec
