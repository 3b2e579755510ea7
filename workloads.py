"""Seeded synthetic inputs for paged KV-cache decode attention.

Shared by the tests, the benchmark and the smoke check, and by nothing on the
product path.  It holds only random draws and the *layout* of the inputs
(shapes, block tables, context lengths, NaN poison); none of the method's
arithmetic (no slot computation, append, un-paging or attention).

The shapes are layer shapes of the models the pages use as examples (the
KV-cache visualization page, "How much memory"): Llama-2-7B (32 KV heads),
Llama-3-8B (8 KV heads), Llama-2-70B (8 KV heads), all with head_dim 128 and
the block size 16 named in "PagedAttention: the cache in blocks".  No trained
weights exist here: every tensor is drawn from N(0, 1).

Seeds: 0 = Q/K/V data, 1 = block-table permutation, 2 = context lengths.
"""
from __future__ import annotations

import dataclasses
import math

import torch

SEED_DATA, SEED_TABLES, SEED_LENGTHS = 0, 1, 2

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "i8": torch.int8, "fp8": torch.float8_e4m3fn,
               "i4": torch.uint8}   # int4: two codes per byte, [NB, Hkv, BS, D/2]
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "fp8": 1}
QUANTIZED = ("i8", "fp8", "i4")   # codes + fp16 scales (i4: one per 32 dims)
INT4_GROUP = 32


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    cache_dtype: str          # "f32" | "f16" | "bf16" | "i8" | "fp8" | "i4"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    layers: int = 1
    description: str = ""
    window: int = 0           # sliding window (0: the whole context)

    @property
    def q_dtype(self) -> str:
        """Queries and outputs: the cache format, or fp16 for a quantized cache."""
        return "f16" if self.cache_dtype in QUANTIZED else self.cache_dtype

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


TINY = Shape("tiny-f32", "f32", 4, 4, 2, 64, 4,
             description="4 seqs, 4 q / 2 KV heads, d 64, block 4, pool 64, ctx {3,7,16,33}")
LLAMA3_8B = Shape("llama3-8b-f16", "f16", 16, 32, 8, 128, 16, layers=32,
                  description="Llama-3-8B layer, fp16, 16 seqs x 4096, block 16")
LLAMA2_7B = Shape("llama2-7b-f16", "f16", 16, 32, 32, 128, 16, layers=32,
                  description="Llama-2-7B MHA layer, fp16, 16 seqs x 4096, 32 layers (32 GiB)")
LLAMA2_70B = Shape("llama2-70b-bf16", "bf16", 64, 64, 8, 128, 16,
                   description="Llama-2-70B GQA layer, bf16, 64 seqs, ctx U[128,32768], "
                               "8 groups of 8 seqs sharing a 1024-token prefix")
LLAMA3_8B_I8 = Shape("llama3-8b-int8kv", "i8", 64, 32, 8, 128, 16,
                     description="Llama-3-8B layer, int8 KV + fp16 scales, 64 seqs x 8192")

LLAMA3_8B_FP8 = Shape("llama3-8b-fp8kv", "fp8", 64, 32, 8, 128, 16,
                      description="Llama-3-8B layer, fp8 (E4M3) KV + fp16 scales, 64 seqs x 8192")

LLAMA3_8B_WINDOW = Shape("llama3-8b-f16-window4k", "f16", 16, 32, 8, 128, 16, layers=32,
                         description="Llama-3-8B layer, fp16, 16 seqs x 16384, sliding window "
                                     "of 4096 positions, 32 layers",
                         window=4096)

LLAMA3_8B_I4 = Shape("llama3-8b-int4kv", "i4", 64, 32, 8, 128, 16,
                     description="Llama-3-8B layer, int4 KV + fp16 scales per 32 dims, "
                                 "64 seqs x 8192")

LLAMA3_70B_I4 = Shape("llama3-70b-int4kv", "i4", 32, 64, 8, 128, 16, layers=4,
                      description="Llama-3-70B layer (64 q / 8 KV heads), int4 KV + fp16 scales "
                                  "per 32 dims, 32 seqs x 8192, 4 layers")

# the headline layer with blocks of 32, in bf16, and with an int8 cache (one
# query head per KV head: the vector-ALU kernel)
LLAMA2_7B_BS32 = Shape("llama2-7b-f16-bs32", "f16", 16, 32, 32, 128, 32, layers=8,
                       description="Llama-2-7B MHA layer, fp16, block 32, 16 seqs x 4096, 8 layers")
LLAMA2_7B_BF16 = Shape("llama2-7b-bf16", "bf16", 16, 32, 32, 128, 16, layers=8,
                       description="Llama-2-7B MHA layer, bf16, 16 seqs x 4096, 8 layers")
LLAMA2_7B_I8 = Shape("llama2-7b-int8kv", "i8", 16, 32, 32, 128, 16, layers=8,
                     description="Llama-2-7B MHA layer, int8 KV + fp16 scales, 16 seqs x 4096, "
                                 "8 layers")

SHAPES = {s.name: s for s in (TINY, LLAMA3_8B, LLAMA2_7B, LLAMA2_70B, LLAMA3_8B_I8,
                              LLAMA3_8B_FP8, LLAMA3_8B_WINDOW, LLAMA3_8B_I4, LLAMA2_7B_BS32,
                              LLAMA2_7B_BF16, LLAMA2_7B_I8, LLAMA3_70B_I4)}

TINY_POOL_BLOCKS = 64
PREFIX_GROUP = 8          # sequences per shared-prefix group (Llama-2-70B workload)
PREFIX_TOKENS = 1024      # tokens of the shared prefix


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def context_lengths(shape: Shape) -> list[int]:
    """Context length of every sequence, counting the token being decoded."""
    if shape.name == TINY.name:
        return [3, 7, 16, 33]
    if shape.name in (LLAMA3_8B.name, LLAMA2_7B.name, LLAMA2_7B_BS32.name, LLAMA2_7B_BF16.name,
                      LLAMA2_7B_I8.name):
        return [4096] * shape.num_seqs
    if shape.name in (LLAMA3_8B_I8.name, LLAMA3_8B_FP8.name, LLAMA3_8B_I4.name,
                      LLAMA3_70B_I4.name):
        return [8192] * shape.num_seqs
    if shape.name == LLAMA3_8B_WINDOW.name:
        return [16384] * shape.num_seqs
    if shape.name == LLAMA2_70B.name:
        lens = torch.randint(128, 32769, (shape.num_seqs,), generator=generator(SEED_LENGTHS))
        return [int(x) for x in lens]
    raise KeyError(shape.name)


@dataclasses.dataclass
class Layout:
    """Block tables of a batch over one shared pool."""
    block_tables: torch.Tensor    # int32 [S, max_blocks]; -1 past a sequence's blocks
    context_lens: torch.Tensor    # int32 [S]
    num_blocks: int
    block_size: int
    owners: torch.Tensor          # int32 [num_blocks]: number of tables naming each block

    @property
    def max_blocks(self) -> int:
        return self.block_tables.shape[1]


def blocks_needed(ctx: int, block_size: int) -> int:
    """Blocks a sequence holds: a new block is taken only when the last is full."""
    return -(-ctx // block_size)


def carve_layout(ctx_lens, block_size, num_blocks=None, max_blocks=None,
                 seed=SEED_TABLES, prefix_group=0, prefix_tokens=0) -> Layout:
    """Hand out blocks of a seeded random permutation of the pool, in order.

    With prefix_group > 0, consecutive groups of that many sequences share the
    blocks of a prefix_tokens-long prefix (the sharing described in
    "PagedAttention: the cache in blocks"); a sequence no longer than the
    prefix uses the first shared blocks only.
    """
    ctx_lens = [int(c) for c in ctx_lens]
    s = len(ctx_lens)
    need = [blocks_needed(c, block_size) for c in ctx_lens]
    if max_blocks is None:
        max_blocks = max(max(need), 1)
    logical = []            # per sequence: list of logical block ids
    next_id = 0
    if prefix_group:
        pb = blocks_needed(prefix_tokens, block_size)
        for g0 in range(0, s, prefix_group):
            shared = list(range(next_id, next_id + pb))
            next_id += pb
            for i in range(g0, min(g0 + prefix_group, s)):
                own = shared[:min(need[i], pb)]
                extra = max(need[i] - pb, 0)
                logical.append(own + list(range(next_id, next_id + extra)))
                next_id += extra
    else:
        for n in need:
            logical.append(list(range(next_id, next_id + n)))
            next_id += n
    total = next_id
    if num_blocks is None:
        num_blocks = total
    assert num_blocks >= total, "pool too small"
    perm = torch.randperm(num_blocks, generator=generator(seed))
    bt = torch.full((s, max_blocks), -1, dtype=torch.int32)
    owners = torch.zeros(num_blocks, dtype=torch.int32)
    for i, ids in enumerate(logical):
        phys = perm[torch.tensor(ids, dtype=torch.long)] if ids else torch.empty(0, dtype=torch.long)
        bt[i, :len(ids)] = phys.to(torch.int32)
        owners.index_add_(0, phys, torch.ones(len(ids), dtype=torch.int32))
    return Layout(bt, torch.tensor(ctx_lens, dtype=torch.int32), num_blocks, block_size, owners)


def layout_for(shape: Shape, ctx_lens=None) -> Layout:
    ctx = context_lengths(shape) if ctx_lens is None else ctx_lens
    if shape.name == TINY.name:
        return carve_layout(ctx, shape.block_size, num_blocks=TINY_POOL_BLOCKS,
                            max_blocks=blocks_needed(max(ctx), shape.block_size))
    if shape.name == LLAMA2_70B.name:
        return carve_layout(ctx, shape.block_size, max_blocks=32768 // shape.block_size,
                            prefix_group=PREFIX_GROUP, prefix_tokens=PREFIX_TOKENS)
    return carve_layout(ctx, shape.block_size)


def randn(shape, dtype: str, seed: int, device="cpu") -> torch.Tensor:
    """N(0, 1) draws in float32, then rounded to the requested format."""
    g = generator(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(TORCH_DTYPE[dtype]) if dtype != "f32" else x


def poison_mask(layout: Layout, device="cpu") -> torch.Tensor:
    """bool [num_blocks, block_size]: slots no sequence's context reaches."""
    nb, bs = layout.num_blocks, layout.block_size
    live = torch.zeros(nb, bs, dtype=torch.bool)
    for s in range(layout.block_tables.shape[0]):
        ctx = int(layout.context_lens[s])
        n = blocks_needed(ctx, bs)
        if n == 0:
            continue
        ids = layout.block_tables[s, :n].long()
        live[ids[:-1]] = True
        last = ctx - (n - 1) * bs
        live[ids[-1], :last] = True
    return (~live).to(device)


@dataclasses.dataclass
class Case:
    """One layer's inputs."""
    shape: Shape
    layout: Layout
    q: torch.Tensor                 # [S, Hq, D] (q_dtype)
    k_cache: torch.Tensor           # [NB, Hkv, BS, D] (cache dtype; fp16 source if quantized)
    v_cache: torch.Tensor
    k_new: torch.Tensor             # [S, Hkv, D]: the decoded token's rows
    v_new: torch.Tensor


def make_case(shape: Shape, layout: Layout | None = None, device="cpu", seed=SEED_DATA,
              poison=True, poison_new_slot=True) -> Case:
    """Seeded Q/K/V for one layer.  For a quantized cache, k_cache/v_cache hold
    the fp16 source rows that the append quantizes.

    poison: NaN in every slot outside all contexts (never to be read).
    poison_new_slot: also NaN at each sequence's last position, which the
    decode step's append must overwrite.
    """
    layout = layout or layout_for(shape)
    src = shape.q_dtype if shape.cache_dtype in QUANTIZED else shape.cache_dtype
    nb, hkv, bs, d = layout.num_blocks, shape.num_kv_heads, shape.block_size, shape.head_dim
    s, hq = shape.num_seqs, shape.num_q_heads
    k = randn((nb, hkv, bs, d), src, seed * 1000 + 1, device)
    v = randn((nb, hkv, bs, d), src, seed * 1000 + 2, device)
    q = randn((s, hq, d), shape.q_dtype, seed * 1000 + 3, device)
    k_new = randn((s, hkv, d), src, seed * 1000 + 4, device)
    v_new = randn((s, hkv, d), src, seed * 1000 + 5, device)
    if poison:
        mask = poison_mask(layout, device)
        if poison_new_slot:
            for i in range(s):
                ctx = int(layout.context_lens[i])
                if ctx > 0:
                    blk = int(layout.block_tables[i, (ctx - 1) // bs])
                    mask[blk, (ctx - 1) % bs] = True
        m = mask[:, None, :, None].expand(nb, hkv, bs, d)
        k = k.masked_fill(m, float("nan"))
        v = v.masked_fill(m, float("nan"))
    return Case(shape, layout, q, k, v, k_new, v_new)


def to_numpy_bits(t: torch.Tensor):
    """Host numpy view of a tensor; bfloat16 travels as uint16 bit patterns and
    fp8 E4M3 as uint8 codes."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def unique_kv_bytes_per_layer_step(shape: Shape, layout: "Layout") -> int:
    """K+V bytes of the distinct pool rows one decode step of one layer reads:
    a block named by several tables counts once, with the most rows any of
    them uses (no window)."""
    rows = {}
    bs = layout.block_size
    for s, c in enumerate(layout.context_lens.tolist()):
        for j in range(blocks_needed(int(c), bs)):
            phys = int(layout.block_tables[s, j])
            rows[phys] = max(rows.get(phys, 0), min(bs, int(c) - j * bs))
    n = sum(rows.values())
    return kv_bytes_per_layer_step(dataclasses.replace(shape, window=0), [n])


def kv_bytes_per_layer_step(shape: Shape, ctx_lens) -> int:
    """Logical K+V bytes one decode step of one layer reads (every sequence reads
    its whole context, shared blocks included, or its last `window` positions),
    plus the scale bytes of a quantized cache."""
    total = sum(min(int(c), shape.window) if shape.window > 0 else int(c) for c in ctx_lens)
    if shape.cache_dtype == "i4":   # half a byte per value, a scale per 32 values
        return total * shape.num_kv_heads * 2 * (shape.head_dim // 2 +
                                                 2 * (shape.head_dim // INT4_GROUP))
    b = total * shape.num_kv_heads * shape.head_dim * 2 * ELEM_BYTES[shape.cache_dtype]
    if shape.cache_dtype in QUANTIZED:
        b += total * shape.num_kv_heads * 2 * 2
    return b
