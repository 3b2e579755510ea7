// decode_plan.h -- cache-format helpers, argument checks of a cache
// descriptor, and the decode plan: which kernel, how many query heads per
// workgroup, tile and partition lengths, workspace layout (internal; host
// code only).
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "pagedattn.h"
#include "decode_dispatch.h"
#include "status.h"

namespace pa {

inline int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_I8: return 1;
    case PA_FP8: return 1;
    case PA_I4: return 1;  // two codes per byte: see row_bytes
    default: return 0;
  }
}

// int8 or fp8 (E4M3) codes with fp16 per-(token, head) scales, or int4
// codes with a scale per group of 32 dims
inline bool quantized(int32_t dtype) { return dtype == PA_I8 || dtype == PA_FP8 || dtype == PA_I4; }

// Bytes of one cached (token, head) row, and fp16 scales per row.
inline int32_t row_bytes(const pa_cache_desc* c) {
  return c->dtype == PA_I4 ? c->head_dim / 2 : c->head_dim * elem_bytes(c->dtype);
}
inline int32_t scales_per_row(const pa_cache_desc* c) {
  return c->dtype == PA_I4 ? c->head_dim / 32 : quantized(c->dtype) ? 1 : 0;
}

inline bool supported_block(int32_t bs) { return bs == 4 || bs == 8 || bs == 16 || bs == 32; }
inline bool supported_dim(int32_t d) { return d == 64 || d == 128; }

inline pa_status check_cache(const pa_cache_desc* c) {
  if (!c) return fail(PA_ERR_INVALID_ARG, "cache descriptor is NULL");
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->block_size <= 0 || c->head_dim <= 0)
    return fail(PA_ERR_INVALID_ARG, "cache sizes must be positive (blocks %d, kv heads %d, block %d, dim %d)",
                c->num_blocks, c->num_kv_heads, c->block_size, c->head_dim);
  if (!elem_bytes(c->dtype)) return fail(PA_ERR_UNSUPPORTED, "unknown cache dtype %d", c->dtype);
  if (!supported_dim(c->head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", c->head_dim);
  if (!supported_block(c->block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported (4, 8, 16 or 32)", c->block_size);
  if ((int64_t)c->num_blocks * c->block_size > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "pool of %d blocks x %d slots exceeds 2^31 slots",
                c->num_blocks, c->block_size);
  return PA_OK;
}

// ------------------------------------------------------------------ plan

// Partition plan, measured on MI355X (256 CUs):
//  * vector-ALU kernel (64 VGPRs, 8 waves/SIMD): ~2048 workgroups (8 per CU),
//    partitions of at least 256 positions;
//  * matrix-core kernel (3 waves/SIMD, two tiles in flight per wave): as few
//    partitions as keep >= 256 workgroups (one per CU) for 16-bit caches -- its per-workgroup prologue and
//    merge cost more than the imbalance of long partitions (Llama-2-70B's
//    ragged batch runs fastest as one partition per sequence); int8, fp8 and
//    int4 tiles carry half the bytes or less and do best with ~1536
//    workgroups, two full rounds of three per CU (64 sequences x 8192 at the
//    Llama-3-8B shape, same box: 3 partitions against 4, kernel 185-189 us
//    against 191-193 us for fp8, 188-190 against 194 for int8; int4
//    150-154 against 155-156 us, and 83 against 86 us at 64 query heads).
inline constexpr int32_t kTargetWorkgroups = 2048;
// The vector-ALU kernel over int8 caches (93 VGPRs: five waves per SIMD)
// does best with one round of workgroups all resident at once: Llama-2-7B
// MHA int8, 16 sequences x 4096, same box: 1024 workgroups (two partitions)
// 86.7 us per launch, 2048 (four) 89.1-92.7, 1536 (three) 92.9.  The fp16
// and bf16 instances measured best at 2048 (bf16: 163.8 against 164.9 us).
inline constexpr int32_t kTargetWorkgroupsInt8 = 1024;
inline constexpr int32_t kTargetWorkgroupsMfma = 256;
inline constexpr int32_t kTargetWorkgroupsMfmaInt8 = 1536;
// The quantized matrix-core kernels keep three workgroups per CU resident,
// so 768 workgroups are one full round on 256 CUs.  Within the target
// above, a plan takes the fewest partitions that fill whole rounds: a part
// round leaves CUs idle at the end, and every extra round repeats each
// workgroup's prologue and partial store.  Measured on MI355X (Llama-3-70B
// layer, int4, 32 sequences x 8192, 8 KV heads): 768 workgroups (three
// partitions) 72.4-75.2 us per launch, 1536 (six) 77.2-79.2, 1024 (four)
// 84.8-90.9, 512 (two) 83.5.
inline constexpr int32_t kQuantRoundWorkgroups = 768;
inline constexpr int32_t kMinPartitionTokens = 256;
inline constexpr int32_t kMinWindowPartitionTokens = 512;
struct Plan {
  bool mfma = false;      // matrix-core kernel (grouped-query heads)
  int32_t gc = 1;         // query heads per workgroup
  int32_t chunks = 1;     // workgroups per KV head (group / gc)
  int32_t tile = 0;       // positions per tile
  int32_t part_tokens = 0;
  int32_t num_parts = 0;
  bool pair = false;      // matrix-core kernel: two sequences per workgroup
  size_t ml_bytes = 0;    // workspace: partial (max, sum)
  size_t o_offset = 0;    // workspace: offset of the partial outputs
  size_t ws_bytes = 0;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of a multi-partition plan: fp32 (max, sum) [S][Hq][P][2], then
// fp32 unnormalized outputs [S][Hq][P][D].
inline void size_workspace(Plan& p, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim) {
  if (p.num_parts <= 1) {
    p.ml_bytes = p.o_offset = p.ws_bytes = 0;
    return;
  }
  const size_t rows = (size_t)num_seqs * num_q_heads * p.num_parts;
  p.ml_bytes = rows * 2 * sizeof(float);
  p.o_offset = align256(p.ml_bytes);
  p.ws_bytes = p.o_offset + rows * head_dim * sizeof(float);
}

// window > 0: a sliding-window plan, whose partitions are sized from the
// window rather than the table (the partitions before it are no-ops).
inline pa_status make_plan(const pa_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                    int32_t max_blocks, int32_t requested, Plan* out, int32_t window = 0) {
  pa_status st = check_cache(c);
  if (st != PA_OK) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                num_q_heads, c->num_kv_heads);
  if (max_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d <= 0", max_blocks);
  if ((int64_t)max_blocks * c->block_size > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "block table width x block size exceeds 2^31 positions");
  if (requested < 0) return fail(PA_ERR_INVALID_ARG, "partition_tokens %d < 0", requested);
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "window %d < 0", window);
  Plan p;
  const int32_t group = num_q_heads / c->num_kv_heads;
  // Four or more query heads per KV head: the score and value products are
  // dense enough for the matrix cores (fp16 / bf16 / int8 / fp8 caches, and
  // int4 at head_dim 128; blocks of 16 or 32), 4, 8 or 16 heads per
  // workgroup.  Otherwise the vector-ALU kernel, up to 8 heads per workgroup
  // (int4: 2).
  const int32_t gc_mfma = group % 16 == 0 ? 16 : group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : 0;
  if (c->dtype != PA_F32 && (c->dtype != PA_I4 || c->head_dim == 128) &&
      (c->block_size == 16 || c->block_size == 32) && gc_mfma >= 4) {
    p.mfma = true;
    p.gc = gc_mfma;
  } else if (c->dtype == PA_I4) {  // 32 values per lane and head: at most 2 heads
    p.gc = group % 2 == 0 ? 2 : 1;
  } else {
    p.gc = group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
  }
  p.chunks = group / p.gc;
  // positions per tile: a block, or enough rows for one 1 KiB wave-load
  p.tile = std::max<int32_t>(c->block_size, 1024 / row_bytes(c));
  const int64_t max_tok = (int64_t)max_blocks * c->block_size;
  int64_t part;
  if (requested > 0) {
    if (requested % p.tile != 0)
      return fail(PA_ERR_INVALID_ARG,
                  "partition_tokens %d must be a multiple of the tile length %d", requested, p.tile);
    part = requested;
  } else {
    // Enough workgroups to fill the chip, each wave owning whole tiles.
    const int64_t unit = (int64_t)p.tile * pa::kDecodeWaves;
    const int64_t units = (int64_t)(num_seqs > 0 ? num_seqs : 1) * c->num_kv_heads * p.chunks;
    // A window's partitions are counted from its first tile, so a windowed
    // plan splits the window like a plain one splits the table, with the
    // same targets and partitions of at least kMinWindowPartitionTokens
    // (windows are short spans; measured on 16 sequences, 4096-token fp16
    // window, 8 KV heads: 256 workgroups 49.2 us, 512: 50.0, 1024: 52.5,
    // 2048: 55.4; 2048-token windows at 32 and 16 KV heads and a 4096-token
    // int8 window did best at 576-token partitions).
    const int64_t target = !p.mfma ? (c->dtype == PA_I8 ? kTargetWorkgroupsInt8 : kTargetWorkgroups)
                           : quantized(c->dtype) ? kTargetWorkgroupsMfmaInt8
                                                 : kTargetWorkgroupsMfma;
    int64_t want_parts = (target + units - 1) / units;
    if (p.mfma && quantized(c->dtype) && window == 0) {
      for (int64_t q = 1; q < want_parts; ++q) {
        if (units * q >= kQuantRoundWorkgroups && units * q % kQuantRoundWorkgroups == 0) {
          want_parts = q;  // whole rounds, fewer than the target's
          break;
        }
      }
    }
    // a window's partitions start at the tile holding its first position:
    // they cover up to tile - 1 positions before it
    const int64_t span = window > 0 ? std::min<int64_t>(max_tok, (int64_t)window + p.tile - 1)
                                    : max_tok;
    part = (span + want_parts - 1) / want_parts;
    part = std::max<int64_t>(part, window > 0 ? kMinWindowPartitionTokens : kMinPartitionTokens);
    part = (part + unit - 1) / unit * unit;
  }
  if (part >= max_tok) part = (max_tok + p.tile - 1) / p.tile * p.tile;
  p.part_tokens = (int32_t)std::min<int64_t>(part, INT32_MAX / 2);
  p.num_parts = (int32_t)((max_tok + p.part_tokens - 1) / p.part_tokens);
  // Counted from the tile holding its first position, a window spans at
  // most window + tile - 1 positions, ceil((window + tile - 1) / part)
  // partitions: the grid and the workspace hold that many slots.
  if (window > 0 && p.num_parts > 1)
    p.num_parts = (int32_t)std::min<int64_t>(
        p.num_parts, ((int64_t)window + p.tile - 1 + p.part_tokens - 1) / p.part_tokens);
  // Paired plan: one partition per sequence on the matrix cores, with
  // enough (sequence, KV head x chunk) items that half as many workgroups
  // still meet the format's target (16-bit: two items per CU).  A workgroup
  // then takes a long and a short sequence, so that ragged lengths even out
  // per CU (a Llama-2-70B batch with lengths U[128, 32768]: 788 -> 726 us
  // when its sequences were ordered so that each CU drew such a pair).  The
  // quantized kernels need their 2048 workgroups: an int8 batch of 512
  // items run paired in one partition took 275 us against 196 in four.
  const int64_t mfma_target = quantized(c->dtype) ? kTargetWorkgroupsMfmaInt8
                                                  : kTargetWorkgroupsMfma;
  // (The int4 matrix-core kernels take one sequence per workgroup.)
  p.pair = p.mfma && c->dtype != PA_I4 && p.num_parts == 1 && window == 0 && num_seqs >= 2 &&
           num_seqs <= kPairMaxSeqs &&
           (int64_t)num_seqs * c->num_kv_heads * p.chunks >= 2 * mfma_target;
  if (num_seqs > 65535 || (int64_t)c->num_kv_heads * p.chunks > 65535)
    return fail(PA_ERR_UNSUPPORTED, "grid too large (%d sequences, %d KV heads x %d chunks)",
                num_seqs, c->num_kv_heads, p.chunks);
  size_workspace(p, num_seqs, num_q_heads, c->head_dim);
  *out = p;
  return PA_OK;
}

}  // namespace pa
