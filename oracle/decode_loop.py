"""Tiny decode loop with and without a KV cache -- TEST INFRASTRUCTURE ONLY.

Follows the worked example of the KV-cache visualization page, "Without vs
with the cache": a 3-token prompt is prefilled, then 4 tokens are decoded.
Without a cache every step recomputes the K and V rows of the whole prefix;
with a cache a step computes only the newest token's rows and appends them.
The same page says the attention itself is identical in both lanes, so the
outputs must agree exactly, and only the number of K,V rows computed differs.

The "model" is synthetic (no trained weights exist or are needed): token
inputs x_t and projection matrices Wq, Wk, Wv are passed in.  Rows are
projected one at a time with ``oracle_project_row`` in both lanes and stored
in float32, the cache's format in this example.
"""
from __future__ import annotations

import numpy as np

from . import attention_dense, decode_slot_mapping, kv_append, paged_decode_attention, project_row


def run(x, Wq, Wk, Wv, n_prompt, num_q_heads, num_kv_heads, head_dim, block_size,
        block_table, num_blocks, scale, lib=None):
    """Run prefill + decode steps in both lanes.

    x: [n_tokens, d_model] token inputs; the first n_prompt form the prompt.
    block_table: the sequence's block ids in order (enough for n_tokens).
    Returns dict with per-step row counts and outputs of both lanes
    (outputs: [steps][num_q_heads][head_dim] fp64).
    """
    n_tokens = x.shape[0]
    group = num_q_heads // num_kv_heads
    steps = [n_prompt] + list(range(n_prompt + 1, n_tokens + 1))  # prefix length per step

    def project(t):
        q = project_row(x[t], Wq, lib).astype(np.float32).reshape(num_q_heads, head_dim)
        k = project_row(x[t], Wk, lib).astype(np.float32).reshape(num_kv_heads, head_dim)
        v = project_row(x[t], Wv, lib).astype(np.float32).reshape(num_kv_heads, head_dim)
        return q, k, v

    # ---- lane 1: no cache, recompute every row of the prefix each step ----
    rows_no_cache, out_no_cache = [], []
    for n in steps:
        qkv = [project(t) for t in range(n)]
        rows_no_cache.append(n)
        q_last = qkv[-1][0]
        outs = np.empty((num_q_heads, head_dim))
        for h in range(num_q_heads):
            kvh = h // group
            K = np.stack([qkv[t][1][kvh] for t in range(n)]).astype(np.float64)
            V = np.stack([qkv[t][2][kvh] for t in range(n)]).astype(np.float64)
            outs[h], _ = attention_dense(q_last[h].astype(np.float64), K, V, scale, lib)
        out_no_cache.append(outs)

    # ---- lane 2: paged cache, compute only the new rows and append them ----
    max_blocks = len(block_table)
    table = np.asarray(block_table, dtype=np.int32).reshape(1, max_blocks)
    k_cache = np.full((num_blocks, num_kv_heads, block_size, head_dim), np.nan, np.float32)
    v_cache = np.full_like(k_cache, np.nan)
    rows_cache, out_cache = [], []
    done = 0
    for n in steps:
        new = list(range(done, n))
        qkv = [project(t) for t in new]
        rows_cache.append(len(new))
        for t, (_, k, v) in zip(new, qkv):
            slot = decode_slot_mapping(table, np.array([t + 1], np.int32), block_size, lib)
            kv_append(k[None], v[None], slot, k_cache, v_cache, lib=lib)
        done = n
        q_last = qkv[-1][0]
        outs = paged_decode_attention(q_last[None], k_cache, v_cache, table,
                                      np.array([n], np.int32), scale, lib=lib)[0]
        out_cache.append(outs)

    return {
        "prefix_lengths": steps,
        "rows_no_cache": rows_no_cache,
        "rows_cache": rows_cache,
        "out_no_cache": np.stack(out_no_cache),
        "out_cache": np.stack(out_cache),
    }
