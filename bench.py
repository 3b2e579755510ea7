"""Benchmark: decode steps of paged KV-cache attention on one MI355X.

Default workload (the headline): Llama-2-7B layer shape, fp16, multi-head
(32 query / 32 KV heads, head_dim 128), 16 sequences x 4096 cached
positions, block size 16, all 32 layers' pools resident (32 GiB).  One step
= for every layer in order: store the new token's K/V rows at its slot and
attend over the paged cache (pa_decode_step: slots, append and partitioned
attention in one launch, then the log-sum-exp merge).  --separate runs the
same step as separate launches (slots, append, partitions, merge).

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line.  value = logical KV bytes read per step / step time
(GB/s); the roofline block times the dominant kernel (the partitioned
attention) with HIP events around a back-to-back batch of its launches;
cpu_baseline times the CPU oracle on the host cores over a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import decode_attention_paged_append_amd as pa  # noqa: E402
import workloads as W  # noqa: E402

METRIC = ("decode-attention KV-read GB/s (% of HBM peak) + seq-steps/s, "
          "Llama-2-7B 16×4096")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, 8 TB/s
KERNEL_SOURCES = ["decode_attention_paged_append_amd/csrc/decode_kernel.h",
                  "decode_attention_paged_append_amd/csrc/device.h",
                  "decode_attention_paged_append_amd/csrc/quant.h",
                  "decode_attention_paged_append_amd/csrc/decode_dispatch.h",
                  "decode_attention_paged_append_amd/csrc/decode_plan.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


class Bench:
    """All layers' inputs resident on the GPU, and the step that runs them."""

    def __init__(self, shape: W.Shape, layers: int, dev, partition_tokens: int = 0,
                 separate: bool = False):
        self.shape, self.layers, self.dev = shape, layers, dev
        self.separate = separate
        self.layout = W.layout_for(shape)
        lay = self.layout
        self.bt = lay.block_tables.to(dev)
        self.ctx = lay.context_lens.to(dev)
        # quantized caches (int8, fp8): codes + fp16 scales, appended by the
        # quantizing append; attention reads them through the partitions call
        self.quant = shape.cache_dtype in W.QUANTIZED
        self.int4 = shape.cache_dtype == "i4"
        self.window = shape.window
        self.append = shape.name != W.LLAMA2_70B.name   # shared-prefix blocks are not appended
        self.cases = []
        for layer in range(layers):
            c = W.make_case(shape, lay, device=dev, seed=layer, poison=False)
            if self.quant:
                c = self._quantize(c)
            self.cases.append(c)
        s, hq, d = shape.num_seqs, shape.num_q_heads, shape.head_dim
        desc = pa.CacheDesc(lay.num_blocks, shape.num_kv_heads, shape.block_size, d,
                            pa.INT4 if self.int4 else
                            pa.DTYPE_CODE[W.TORCH_DTYPE[shape.cache_dtype]])
        self.part = partition_tokens or pa.decode_partition_tokens(desc, s, hq, lay.max_blocks)
        if self.window:
            # the library plans a windowed call itself (partitions + merge)
            self.wws = torch.empty(max(pa.decode_window_workspace_bytes(
                desc, s, hq, lay.max_blocks, self.window), 256), dtype=torch.uint8, device=dev)
        # the library routes >= 4 query heads per KV head with 16/32 blocks to
        # matrix cores (int4: at head_dim 128)
        self.mfma = (shape.cache_dtype != "f32" and shape.block_size in (16, 32)
                     and shape.group % 4 == 0
                     and (shape.cache_dtype != "i4" or shape.head_dim == 128))
        self.nparts = -(-lay.max_blocks * shape.block_size // self.part)
        nbytes = pa.decode_workspace_bytes(desc, s, hq, lay.max_blocks, self.part)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.outs = [torch.empty_like(c.q) for c in self.cases]
        self.slots = torch.empty(s, dtype=torch.int64, device=dev)

    def quant_append(self, *args):
        {"i8": pa.kv_append_int8, "fp8": pa.kv_append_fp8,
         "i4": pa.kv_append_int4}[self.shape.cache_dtype](*args)

    def _quantize(self, c):
        nb, hkv, bs, d = c.k_cache.shape
        rows = lambda x: x.permute(0, 2, 1, 3).reshape(nb * bs, hkv, d).contiguous()
        slots = torch.arange(nb * bs, dtype=torch.int64, device=self.dev)
        kq = torch.empty((nb, hkv, bs, d // 2 if self.int4 else d),
                         dtype=W.TORCH_DTYPE[self.shape.cache_dtype], device=self.dev)
        vq = torch.empty_like(kq)
        ks = torch.empty((nb, hkv, bs) + ((d // W.INT4_GROUP,) if self.int4 else ()),
                         dtype=torch.float16, device=self.dev)
        vs = torch.empty_like(ks)
        self.quant_append(rows(c.k_cache), rows(c.v_cache), slots, kq, vq, ks, vs)
        torch.cuda.synchronize()
        c.k_cache, c.v_cache = kq, vq
        c.k_scale, c.v_scale = ks, vs
        return c

    def step(self):
        """One decode step over every layer."""
        sh = self.shape
        fused_append = self.fused_append
        if self.append and not fused_append:
            pa.decode_slot_mapping(self.bt, self.ctx, sh.block_size, out=self.slots)
        for layer, c in enumerate(self.cases):
            if self.append and not fused_append:
                if self.quant:
                    self.quant_append(c.k_new, c.v_new, self.slots, c.k_cache, c.v_cache,
                                      c.k_scale, c.v_scale)
                else:
                    pa.kv_append(c.k_new, c.v_new, self.slots, c.k_cache, c.v_cache)
            self.attend(layer)
            if self.nparts > 1 and not self.window:
                pa.lse_merge(self.ws, self.ctx, sh.num_q_heads, sh.head_dim,
                             self.layout.max_blocks, sh.block_size, self.part, self.outs[layer])

    def attend(self, layer):
        """The dominant kernel: one layer's attention-partition launch (with
        the append fused into it for 16/32-bit caches)."""
        c, sh = self.cases[layer], self.shape
        out = self.outs[layer]
        if self.window and self.fused_append:
            pa.decode_step_window(c.q, c.k_new, c.v_new, c.k_cache, c.v_cache, self.bt, self.ctx,
                                  sh.scale, self.window, out, getattr(c, "k_scale", None),
                                  getattr(c, "v_scale", None), self.wws, int4=self.int4)
        elif self.window:
            pa.paged_decode_attention_window(c.q, c.k_cache, c.v_cache, self.bt, self.ctx,
                                             sh.scale, self.window, out, workspace=self.wws)
        elif self.fused_append and self.quant:
            pa.decode_step_partitions_quant(c.q, c.k_new, c.v_new, c.k_cache, c.v_cache,
                                            c.k_scale, c.v_scale, self.bt, self.ctx, sh.scale,
                                            out, self.part, self.ws, int4=self.int4)
        elif self.fused_append:
            pa.decode_step_partitions(c.q, c.k_new, c.v_new, c.k_cache, c.v_cache, self.bt,
                                      self.ctx, sh.scale, out, self.part, self.ws)
        else:
            pa.decode_partitions(c.q, c.k_cache, c.v_cache, self.bt, self.ctx, sh.scale, out,
                                 self.part, self.ws, getattr(c, "k_scale", None),
                                 getattr(c, "v_scale", None), int4=self.int4)

    @property
    def fused_append(self) -> bool:
        return self.append and not self.separate

    def kv_bytes_per_layer(self) -> int:
        return W.kv_bytes_per_layer_step(self.shape, self.layout.context_lens.tolist())

    def io_bytes_per_layer(self) -> int:
        """Algorithmic bytes of one layer's attention launch: cached K/V
        (+ scales), q and out, the block-table entries read, and with a fused
        append the new rows read and written."""
        sh = self.shape
        qo = 2 * sh.num_seqs * sh.num_q_heads * sh.head_dim * W.ELEM_BYTES[sh.q_dtype]
        bs = sh.block_size
        first = [max(0, int(c) - sh.window) // bs if sh.window else 0
                 for c in self.layout.context_lens]
        tables = sum(W.blocks_needed(int(c), bs) - f
                     for c, f in zip(self.layout.context_lens, first)) * 4
        new_rows = 0
        if self.fused_append:
            rows = 2 * sh.num_seqs * sh.num_kv_heads     # K and V rows of the new tokens
            if self.int4:       # fp16 read, packed codes + group scales written
                new_rows = rows * (2 * sh.head_dim + sh.head_dim // 2 +
                                   2 * (sh.head_dim // W.INT4_GROUP))
            elif self.quant:    # fp16 read, codes + one scale written
                new_rows = rows * (2 * sh.head_dim + sh.head_dim + 2)
            else:               # read and written in the cache's format
                new_rows = rows * 2 * sh.head_dim * W.ELEM_BYTES[sh.cache_dtype]
        return self.kv_bytes_per_layer() + qo + tables + new_rows


READ_PROBE_BYTES = 4 << 30   # 16x the 256 MiB last-level cache


def read_probe(dev, launches: int = 10, groups=()) -> dict:
    """The library's HBM read-rate probe (pa_hbm_read_probe) over a 4 GiB
    buffer, timed between HIP events: 4 KiB chunks read in sequence, and in a
    seeded random order (the access pattern of the attention kernels' block
    gather).  These are the practical read bandwidths the attention kernels'
    rates are compared with.  groups: also random orders of runs of n
    adjacent chunks (n waves of one workgroup read 4n contiguous KiB), the
    rate a kernel that read bigger contiguous pieces could reach."""
    src = torch.empty(READ_PROBE_BYTES // 4, dtype=torch.int32, device=dev)
    src.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    chunks = READ_PROBE_BYTES // 4096
    gen = torch.Generator().manual_seed(3)

    def runs_of(n):
        perm = torch.randperm(chunks // n, generator=gen)
        return (perm[:, None] * n + torch.arange(n)[None, :]).reshape(-1).to(torch.int32).to(dev)

    orders = [("sequential", None), ("random_chunks", runs_of(1))]
    orders += [(f"random_{4 * n}KiB_runs", runs_of(n)) for n in groups]
    result = {"bytes": READ_PROBE_BYTES, "chunk_bytes": 4096}
    for name, o in orders:
        for _ in range(2):
            pa.hbm_read_probe(src, sink, o)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(launches):
            pa.hbm_read_probe(src, sink, o)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        result[name + "_GB/s"] = round(READ_PROBE_BYTES / (ms / 1e3) / 1e9, 1)
    del src, orders
    return result


def cpu_baseline(b: Bench, min_seconds: float = 10.0) -> dict:
    """The CPU oracle, as it stands, over layer 0 of the same workload."""
    import oracle

    c = b.cases[0]
    lay = b.layout
    host = W.to_numpy_bits
    args = dict(k_scale=host(c.k_scale) if b.quant else None,
                v_scale=host(c.v_scale) if b.quant else None,
                bf16=b.shape.cache_dtype == "bf16", int4=b.int4)
    q, kc, vc = host(c.q), host(c.k_cache), host(c.v_cache)
    bt, ctx = host(lay.block_tables), host(lay.context_lens)
    threads = oracle.max_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        if b.window:
            oracle.paged_decode_attention_window(q, kc, vc, bt, ctx, b.shape.scale, b.window,
                                                 num_threads=threads, **args)
        else:
            oracle.paged_decode_attention(q, kc, vc, bt, ctx, b.shape.scale,
                                          num_threads=threads, **args)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    # one thread over every head of sequence 0 (at least 3 s)
    pairs = [(0, h) for h in range(b.shape.num_q_heads)]
    one = W.kv_bytes_per_layer_step(b.shape, [int(lay.context_lens[0])])
    reps1, t1 = 0, time.perf_counter()
    while True:
        if b.window:
            oracle.paged_decode_attention_window(q, kc, vc, bt, ctx, b.shape.scale, b.window,
                                                 pairs=pairs, num_threads=1, **args)
        else:
            oracle.paged_decode_attention(q, kc, vc, bt, ctx, b.shape.scale, pairs=pairs,
                                          num_threads=1, **args)
        reps1 += 1
        if time.perf_counter() - t1 >= 3.0:
            break
    dt1 = time.perf_counter() - t1
    return {"value": round(b.kv_bytes_per_layer() * reps / dt / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"layer 0 of {b.layers}: all {b.shape.num_seqs} seqs x "
                      f"{b.shape.num_q_heads} heads, fp64 oracle run {reps} time(s) in "
                      f"{dt:.1f} s on {threads} threads",
            "single_thread": {"value": round(one * reps1 / dt1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"layer 0, sequence 0 (all {b.shape.num_q_heads} "
                                        f"heads), {reps1} time(s) in {dt1:.1f} s"},
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def write_traffic_record(counter_dir: str, out_path: str = TRAFFIC_FILE) -> dict:
    """Rebuild the traffic record from the four rocprofv3 --pmc runs listed in
    the headline counters summary: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of the headline attention kernel, each scaled by what the same
    counter reads for a 1 GiB device copy (2^30 bytes read and written).
    counter_dir holds pmc_fetch/, pmc_write/, pmc_copy_fetch/ and
    pmc_copy_write/ as rocprofv3 wrote them.  The record carries the hash of
    the kernel sources it was taken on."""
    import csv
    import glob

    def mean_per_dispatch(sub, counter, kernel):
        files = glob.glob(os.path.join(counter_dir, sub, "**", "*counter_collection.csv"),
                          recursive=True)
        if not files:
            raise FileNotFoundError(f"no counter CSV under {os.path.join(counter_dir, sub)}")
        per = {}
        with open(files[0]) as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        if not per:
            raise ValueError(f"no {counter} samples of {kernel} in {files[0]}")
        return sum(per.values()) / len(per)

    fetch = mean_per_dispatch("pmc_fetch", "FETCH_SIZE", "decode_partition_kernel")
    write = mean_per_dispatch("pmc_write", "WRITE_SIZE", "decode_partition_kernel")
    cf = mean_per_dispatch("pmc_copy_fetch", "FETCH_SIZE", "copy")
    cw = mean_per_dispatch("pmc_copy_write", "WRITE_SIZE", "copy")
    ff, fw = 2**30 / (cf * 1024), 2**30 / (cw * 1024)
    rec = {"kernel": "decode_partition_kernel<F16,128,16,1,4>",
           "workload": "llama2-7b-f16 16x4096, fused append",
           "bench_workload": "llama2-7b-f16",
           "kernel_source_sha256": kernel_source_hash(),
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "copy_fetch_factor": ff, "copy_write_factor": fw,
           "traffic_bytes_per_launch": round(fetch * 1024 * ff) + round(write * 1024 * fw)}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def traffic_block(workload: str, default_launch: bool):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on this workload's default launch and the current kernel sources (else
    null)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (not default_launch or t.get("bench_workload") != workload
            or t.get("kernel_source_sha256") != kernel_source_hash()):
        return None
    return t.get("traffic_bytes_per_launch")


def block_pool_bench(dev, steps: int, warmup: int, cpu: bool) -> dict:
    """The block pool at the Llama-3-8B layer shape (8 KV heads x 128, fp16,
    block size 16): the copy-on-write kernel's bandwidth over a batch of
    whole-block copies, and the native manager's host time per decode round
    of 256 sequences (256 appends of one token, then the table export)."""
    import numpy as np

    hkv, bs, d, nb = 8, 16, 128, 8192
    kc = torch.randn((nb, hkv, bs, d), device=dev).to(torch.float16)
    vc = torch.randn_like(kc)
    g = torch.Generator().manual_seed(1)
    perm = torch.randperm(nb, generator=g)
    results = {}
    for npairs in (2048, 64):
        pairs = torch.stack([perm[:npairs], perm[nb // 2:nb // 2 + npairs]], 1).to(
            torch.int32).to(dev).contiguous()
        for _ in range(warmup):
            pa.copy_blocks(kc, vc, pairs)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = steps * 10
        torch.cuda.synchronize()
        pa.copy_blocks(kc, vc, pairs)   # lead call, untimed (see timed_steps)
        e0.record()
        for _ in range(reps):
            pa.copy_blocks(kc, vc, pairs)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        moved = 2 * npairs * 2 * hkv * bs * d * 2          # K and V, read + write
        results[npairs] = (ms, moved)

    # host: 256 sequences prefilled to 4096 tokens, then decode rounds
    seqs_n, ctx0, rounds = 256, 4096, 2048
    pool = seqs_n * (ctx0 + rounds) // bs + 64
    m = pa.BlockManager(pool, bs)
    seqs = [m.add() for _ in range(seqs_n)]
    m.append([(s, ctx0) for s in seqs])
    maxb = (ctx0 + rounds) // bs + 1
    ids = np.array(seqs, np.int32)
    ones = np.ones(seqs_n, np.int32)
    t0 = time.perf_counter()
    for _ in range(rounds):
        m.append_arrays(ids, ones)
        m.block_tables(ids, maxb)
    host_us = (time.perf_counter() - t0) / rounds * 1e6
    # forks: 32 prompts of 1000 tokens, 8 requests each sharing the prompt;
    # the first decode round copies the 32 x 7 shared partial blocks
    m2 = pa.BlockManager(32 * 8 * 80, bs)
    roots = [m2.add() for _ in range(32)]
    m2.append([(r, 1000) for r in roots])
    kids = [m2.fork(r) for r in roots for _ in range(7)]
    t0 = time.perf_counter()
    _, copies = m2.append([(s, 1) for s in roots + kids])
    fork_round_us = (time.perf_counter() - t0) * 1e6

    cpu_block = None
    if cpu:
        from oracle import block_manager as obm
        om = obm.BlockManager(pool, bs)
        oseqs = [om.add() for _ in range(seqs_n)]
        om.append([(s, ctx0) for s in oseqs])
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0 and n < rounds:
            om.append([(s, 1) for s in oseqs])
            n += 1
        dt = time.perf_counter() - t0
        cpu_block = {"value": round(dt / n * 1e6, 1), "unit": "us per decode round",
                     "cores": 1, "kind": "oracle",
                     "sample": f"the plain block-pool model, {n} decode rounds of 256 "
                               f"sequences at 4096+ tokens, {dt:.1f} s"}
    ms, moved = results[2048]
    ms64, moved64 = results[64]
    gbs = moved / (ms / 1e3) / 1e9
    return {
        "metric": "block pool: copy-on-write block copy GB/s (read + write) + host us per "
                  "decode round",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "block pool at the Llama-3-8B layer shape (8 KV heads x 128, "
                               "fp16, block 16); step = pa_copy_blocks of 2048 block pairs "
                               "(K and V, 64 KiB per pair)", "pairs": 2048},
        "copy_64_pairs": {"us": round(ms64 * 1e3, 2),
                          "GB/s": round(moved64 / (ms64 / 1e3) / 1e9, 2)},
        "host_us_per_decode_round": round(host_us, 2),
        "host_decode_round": "256 sequences at 4096+ tokens: pa_bm_append of one token each, "
                             "then pa_bm_block_tables of all 256 rows",
        "host_us_fork_round": round(fork_round_us, 2),
        "fork_round_copies": int(len(copies)),
        "roofline": {"bound": "hbm", "kernel": "copy_blocks_kernel", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": moved,
                     "avg_launch_ms": round(ms, 5)},
        "cpu_baseline": cpu_block,
    }


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}   # MI355X dense fp16/bf16


PREFILL_WORKLOADS = {
    # name: (description, context lengths, chunk lengths)
    "prefill-llama3-8b": ("Llama-3-8B layer shape (32 q / 8 KV heads, d 128, block 16, fp16), "
                          "8 whole prompts of 2048 tokens, 32 layer pools",
                          [2048] * 8, [2048] * 8),
    "chunked-prefill-llama3-8b": ("Llama-3-8B layer shape (32 q / 8 KV heads, d 128, block 16, "
                                  "fp16), 16 sequences each taking a 512-token chunk after 3584 "
                                  "cached positions, 32 layer pools",
                                  [4096] * 16, [512] * 16),
}


def prefill_flops(ctx, tq, hq, d) -> int:
    """Causal attention flops: query at position p scores and mixes p+1 rows,
    2D flops each for q.k and for w.v."""
    total = 0
    for c, t in zip(ctx, tq):
        first = c - t
        total += (t * (first + 1) + t * (t - 1) // 2) * 4 * d * hq
    return total


def prefill_bench(name, dev, steps, warmup, cpu: bool) -> dict:
    import numpy as np

    desc, ctx, tq = PREFILL_WORKLOADS[name]
    hq, hkv, d, bs, layers = 32, 8, 128, 16, 32
    g = torch.Generator(device=dev).manual_seed(0)
    nblk = sum(-(-c // bs) for c in ctx)
    maxb = max(-(-c // bs) for c in ctx)
    perm = torch.randperm(nblk, generator=torch.Generator().manual_seed(1))
    bt = torch.full((len(ctx), maxb), -1, dtype=torch.int32)
    cur = 0
    for s, c in enumerate(ctx):
        k = -(-c // bs)
        bt[s, :k] = perm[cur:cur + k].to(torch.int32)
        cur += k
    bt = bt.to(dev)
    qs = torch.tensor([0] + list(np.cumsum(tq)), dtype=torch.int32, device=dev)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=dev)
    pools = [(torch.randn((nblk, hkv, bs, d), generator=g, device=dev).half(),
              torch.randn((nblk, hkv, bs, d), generator=g, device=dev).half())
             for _ in range(layers)]
    q = torch.randn((sum(tq), hq, d), generator=g, device=dev).half()
    out = torch.empty_like(q)
    scale = d ** -0.5
    maxq = max(tq)

    def step():
        for kc, vc in pools:
            pa.paged_prefill_attention(q, kc, vc, bt, qs, ctx_t, scale, out, maxq)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    step()                              # lead step, untimed (see timed_steps)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = prefill_flops(ctx, tq, hq, d)
    launch_ms = ms / layers
    tflops = flops / (launch_ms / 1e3) / 1e12
    cpu_block = None
    if cpu:
        import oracle

        kh = pools[0][0].cpu().numpy()
        vh = pools[0][1].cpu().numpy()
        qh = q.cpu().numpy()
        rng = np.random.default_rng(3)
        total = sum(tq)
        threads = oracle.max_threads()
        rows, n, t0 = [], 0, time.perf_counter()
        sample_flops = 0
        qs_h, bt_h = qs.cpu().numpy(), bt.cpu().numpy()
        while time.perf_counter() - t0 < 10.0:
            batch = [(int(rng.integers(total)), int(rng.integers(hq))) for _ in range(64)]
            oracle.paged_prefill_attention(qh, kh, vh, bt_h, qs_h, np.array(ctx, np.int32),
                                           scale, rows=batch, num_threads=threads)
            for tok, _ in batch:
                s_ = int(np.searchsorted(qs_h, tok, side="right")) - 1
                pos = ctx[s_] - tq[s_] + tok - int(qs_h[s_])
                sample_flops += (pos + 1) * 4 * d
            n += len(batch)
        dt = time.perf_counter() - t0
        cpu_block = {"value": round(sample_flops / dt / 1e12, 6), "unit": "TFLOP/s",
                     "cores": threads, "kind": "oracle",
                     "sample": f"{n} random (token, head) rows of layer 0, fp64 oracle, "
                               f"{dt:.1f} s on {threads} threads"}
    peak = MFMA_PEAK_TFLOPS["f16"]
    return {
        "metric": "prefill attention TFLOP/s (causal, % of fp16 dense MFMA peak)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic: seeded N(0,1) q/k/v at the layer shape; block tables a seeded "
                "permutation of the pool",
        "config": {"workload": f"{name}: {desc}; step = pa_paged_prefill_attention on each of "
                               f"the 32 layers", "num_seqs": len(ctx), "query_tokens": sum(tq),
                   "context_lens_sum": sum(ctx), "layers": layers},
        "tokens_per_s": round(sum(tq) * 1e3 / ms, 1),
        "roofline": {"bound": "mfma", "kernel": "prefill_mfma_kernel",
                     "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None,
                     "flops_per_launch": flops, "avg_launch_ms": round(launch_ms, 5)},
        "cpu_baseline": cpu_block,
    }


def graph_timed_ms(launches, count):
    """Average duration of the launches one launches() call issues (count of
    them): they run back to back between two events on the stream they use,
    captured once in a HIP graph and replayed, so that neither per-launch
    events nor the binding's host work between launches (which a short kernel
    would wait on) enter the figure; if capture fails, the launches are
    issued directly."""
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            launches()
        graph.replay()                      # first replay: untimed
        torch.cuda.synchronize()
        k0.record()
        graph.replay()
        k1.record()
        how = "hip graph replay of the launches"
    except RuntimeError:
        torch.cuda.synchronize()
        k0.record()
        launches()
        k1.record()
        how = "launches issued back to back"
    torch.cuda.synchronize()
    return k0.elapsed_time(k1) / count, how


def capture_step(b):
    """One whole decode step (every layer's launches, as Bench.step issues
    them) captured in a HIP graph, the way a serving loop replays its decode
    step; None if capture fails.  The step enqueues kernels only (no memset,
    allocation or synchronization), so a replay does exactly the eager
    step's work: the GPU tests replay such captures and compare every replay
    with the eager result bit for bit."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            b.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            b.step()
        torch.cuda.synchronize()
        return graph
    except RuntimeError:
        torch.cuda.synchronize()
        return None


def timed_steps(run, steps):
    """(ms per step over `steps` calls of run() between two events on torch's
    current stream, sorted per-step durations from a second pass).

    One untimed step is queued after the synchronize and before the first
    event (lead_step), so the GPU is busy when that event fires: the host's
    latency to the first launch, about 0.1 ms and so a few percent of a
    one-layer step, stays out of the figure, as it does in a serving loop that
    keeps the queue fed.  An event recorded after every step costs the GPU
    about 6 us per step (seen in kernel traces as a gap before the next
    launch), so the per-step spread comes from a pass of its own."""
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    run()                               # lead step, untimed
    t0.record()
    for _ in range(steps):
        run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    run()
    marks[0].record()
    for i in range(steps):
        run()
        marks[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    return ms, per_step


def eager_timed_ms(launches, count):
    """Average duration of the launches one launches() call issues (count of
    them), issued back to back between two events on the stream they use.
    One untimed pass is queued just before the first event, so the GPU is
    busy while the host issues the timed launches and the first event fires
    behind it: the host's latency to the first launch stays out of the
    figure.  Each is an attention launch of 40 us or more, longer than the
    binding's host work per call, so the queue stays ahead of the GPU and the
    figure is the kernels' own duration plus the gaps between them, as a
    kernel trace sees it (a graph of many chained launches read up to 5 %
    above the trace for some of these kernels)."""
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    launches()
    torch.cuda.synchronize()
    launches()          # the lead pass, untimed
    k0.record()
    launches()
    k1.record()
    torch.cuda.synchronize()
    return k0.elapsed_time(k1) / count, "launches issued back to back"


def attention_launch_ms(b, layers, steps):
    """Average duration of the dominant kernel: the same launches (every
    layer, K times) back to back (eager_timed_ms)."""
    def launches():
        for _ in range(steps):
            for layer in range(layers):
                b.attend(layer)

    return eager_timed_ms(launches, steps * layers)


def append_report(b, layers, steps) -> dict | None:
    """The append on its own (pa_kv_append, or the quantizing append of an
    int8 / fp8 / int4 cache): every layer's new rows at their decode slots,
    K times, timed like the attention launch.  Its bytes: the new K and V rows
    read (fp16 for the quantizing appends) and stored (codes and scales), and
    the slots read."""
    if not b.append:
        return None
    sh = b.shape
    pa.decode_slot_mapping(b.bt, b.ctx, sh.block_size, out=b.slots)

    def launches():
        for _ in range(steps):
            for c in b.cases:
                if b.quant:
                    b.quant_append(c.k_new, c.v_new, b.slots, c.k_cache, c.v_cache, c.k_scale,
                                   c.v_scale)
                else:
                    pa.kv_append(c.k_new, c.v_new, b.slots, c.k_cache, c.v_cache)

    ms, how = graph_timed_ms(launches, steps * layers)
    rows = 2 * sh.num_seqs * sh.num_kv_heads
    d = sh.head_dim
    if b.int4:
        moved = rows * (2 * d + d // 2 + 2 * (d // W.INT4_GROUP))
    elif b.quant:
        moved = rows * (2 * d + d + 2)
    else:
        moved = rows * 2 * d * W.ELEM_BYTES[sh.cache_dtype]
    moved += 8 * sh.num_seqs
    kernel = {"i8": "kv_append_quant_kernel<128, 0>", "fp8": "kv_append_quant_kernel<128, 1>",
              "i4": "kv_append_quant_kernel<128, 2>"}.get(sh.cache_dtype, "kv_append_kernel")
    return {"kernel": kernel, "avg_launch_us": round(ms * 1e3, 2), "bytes_per_launch": moved,
            "GBps": round(moved / (ms / 1e3) / 1e9, 1), "timing": how,
            "note": "timed on its own; the step fuses it into the attention launch"
            if b.fused_append else "timed on its own; the step launches it separately"}


def unique_bytes_report(b, layers, ms_step, kv_step) -> dict:
    """For a pool whose blocks are shared between tables (a common prefix):
    the distinct bytes a step reads, and the rate on those alone."""
    if b.window or int(b.layout.owners.max()) <= 1:
        return {}
    uniq = W.unique_kv_bytes_per_layer_step(b.shape, b.layout) * layers
    return {"unique_kv_bytes_per_step": uniq,
            "unique_GBps": round(uniq / (ms_step / 1e3) / 1e9, 2),
            "unique_fraction_of_logical": round(uniq / kv_step, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 100 warm-up steps (0.5 s of the headline): after 5, some runs still
    # had a slow transient (6246 against 6403-6431 GB/s after 100 or 300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=W.LLAMA2_7B.name,
                    choices=sorted(W.SHAPES) + ["block-pool"] + sorted(PREFILL_WORKLOADS))
    ap.add_argument("--layers", type=int, default=0, help="0: the workload's own layer count")
    ap.add_argument("--partition-tokens", type=int, default=0,
                    help="0: the library's own plan (what pa_paged_decode_attention runs)")
    ap.add_argument("--separate", action="store_true",
                    help="separate launches for slots, append, partitions and merge")
    ap.add_argument("--graph", action="store_true",
                    help="replay a HIP graph of one whole step instead of issuing its launches "
                         "from Python")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-kernel", type=int, default=0,
                    help="only run N copies of a 1 GiB tensor (counter calibration) and exit")
    ap.add_argument("--read-probe", action="store_true",
                    help="only time the HBM read-rate probe over 4 GiB (also random runs of "
                         "2-16 adjacent chunks) and exit")
    ap.add_argument("--no-read-probe", action="store_true")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="only rebuild the headline traffic record from the four rocprofv3 "
                         "--pmc runs under DIR (no GPU) and exit")
    args = ap.parse_args()
    if args.traffic_from:
        print(json.dumps(write_traffic_record(args.traffic_from)))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)

    if args.copy_kernel:
        src = torch.ones(1 << 29, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.copy_kernel):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 2, "copies": args.copy_kernel}))
        return

    if args.read_probe:
        print(json.dumps({"hbm_read_probe": read_probe(dev, groups=(2, 4, 8, 16))}))
        return

    if args.workload == "block-pool":
        print(json.dumps(block_pool_bench(dev, args.steps, args.warmup,
                                          not args.no_cpu_baseline)))
        return

    if args.workload in PREFILL_WORKLOADS:
        print(json.dumps(prefill_bench(args.workload, dev, args.steps, args.warmup,
                                       not args.no_cpu_baseline)))
        return

    shape = W.SHAPES[args.workload]
    layers = args.layers or shape.layers
    b = Bench(shape, layers, dev, args.partition_tokens, args.separate)
    torch.cuda.synchronize()
    b.step()
    torch.cuda.synchronize()
    # The step's launches are issued from Python every step; --graph replays
    # one captured step instead (measured: no faster on the 32-layer steps,
    # and each replay adds ~12 us, which a one-layer step feels).
    graph = capture_step(b) if args.graph else None
    run = graph.replay if graph is not None else b.step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    # Timed region: K whole steps, bracketed by events on torch's current
    # stream, which is the stream the binding hands to every launch (and the
    # one a graph replays on); an event after every step gives the spread of
    # single steps.
    ms_step, per_step = timed_steps(run, args.steps)

    kernel_ms, kernel_timing = attention_launch_ms(b, layers, args.steps)
    append = append_report(b, layers, min(args.steps, 10))

    kv_step = b.kv_bytes_per_layer() * layers
    value = kv_step / (ms_step / 1e3) / 1e9
    io = b.io_bytes_per_layer()
    achieved = io / (kernel_ms / 1e3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": {"median": round(float(np.median(per_step)), 4),
                    "p10": round(float(np.percentile(per_step, 10)), 4),
                    "p90": round(float(np.percentile(per_step, 90)), 4)},
        "step_timing": ("hip graph replay of one whole step (every layer's launches)"
                        if graph is not None else "launches issued from Python every step")
                       + "; one untimed lead step queued before the first event; step_ms "
                         "from a second pass with an event after every step",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.cache_dtype,
        "data": "synthetic: seeded N(0,1) Q/K/V at the layer shape; block tables a seeded "
                "permutation of the pool",
        "config": {
            "workload": f"{shape.name}: {shape.description}; step = per layer "
                        + ("windowed attention launch with the slot and append fused in, "
                           "then merge" if b.window and b.fused_append
                           else "slots, append, then the windowed attention call (partitions, "
                           "merge)" if b.window
                           else "attention launch with the slot and "
                           + ("quantizing " if b.quant else "") + "append fused in, then merge"
                           if b.fused_append
                           else "slots, append, attention partitions, merge launches"
                           if b.append else "attention partitions, merge launches"),
            "num_seqs": shape.num_seqs, "context_lens_sum": int(b.layout.context_lens.sum()),
            "layers": layers, "num_q_heads": shape.num_q_heads,
            "num_kv_heads": shape.num_kv_heads, "head_dim": shape.head_dim,
            "block_size": shape.block_size,
            **({"window": b.window} if b.window else
               {"partition_tokens": b.part, "partitions": b.nparts}),
        },
        "seq_steps_per_s": round(shape.num_seqs * 1e3 / ms_step, 2),
        "steps_per_s": round(1e3 / ms_step, 2),
        **unique_bytes_report(b, layers, ms_step, kv_step),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kv_bytes_per_step": kv_step,
        "roofline": {
            "bound": "hbm",
            "kernel": (("decode_mfma_kernel" if not b.int4 else "decode_mfma_i4h_kernel"
                        if shape.group % 8 == 0 else "decode_mfma_i4_kernel") if b.mfma
                       else "decode_partition_kernel")
                      + (" + lse_merge_kernel (one windowed call)" if b.window else ""),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_block(shape.name, not (args.separate or args.partition_tokens)),
            "bytes_per_launch": io,
            "avg_launch_ms": round(kernel_ms, 5),
            "timing": kernel_timing,
        },
        "cpu_baseline": None,
    }
    if append:
        result["append"] = append
    if not args.no_read_probe:
        probe = read_probe(dev)
        probe["kernel_frac_of_sequential"] = round(achieved / probe["sequential_GB/s"], 4)
        probe["kernel_frac_of_random_chunks"] = round(achieved / probe["random_chunks_GB/s"], 4)
        result["hbm_read_probe"] = probe
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
