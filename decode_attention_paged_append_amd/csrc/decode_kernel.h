// decode_kernel.h -- partitioned paged decode attention (phase 1) for gfx950.
//
// Computes, for one sequence s, one KV head and the GC query heads of a
// grouped-query group that read it, the attention of each head's query over
// one partition of the sequence's cached rows:
//   z_i = scale * q . k_i,   p_i = exp(z_i - m),   l = sum p_i,   o = sum p_i v_i
// ("KV cache: the engine behind fast LLM inference", "Concept" and step 3 of
// "What happens at each decoding step").  Rows are reached through the
// sequence's block table ("PagedAttention: the cache in blocks" on the
// KV-cache visualization page).  The softmax runs online, tile by tile, in
// registers: the score row never goes to memory (the guide's "Flash
// attention: don't build the giant matrix").
//
// Work decomposition (wave64, one workgroup = NW waves):
//   grid = (partition, KV head x head chunk, sequence).
//   A tile is TT consecutive positions: one whole block when the block holds
//   at least one wave-load of rows, else several blocks.  Wave w of the
//   workgroup takes tiles w, w+NW, ... of the partition.
//   Each lane loads 16 contiguous bytes per fragment, so one wave-load is
//   1 KiB of consecutive bytes: LR lanes cover one row (head_dim values) and
//   the wave covers RPI = 64/LR rows.  K and V tiles of a block are
//   contiguous (BS x D elements per KV head), so every load is fully
//   coalesced and the whole tile is in flight at once.
//   The K row read by a lane is dotted with all GC queries from registers,
//   so a GQA group reads its KV head once; partial dots are summed across
//   the LR lanes of a row with DPP moves.
//   Every lane keeps its own running (max, sum, output slice) for the rows
//   it sees -- no cross-row traffic inside the loop.  Row groups are merged
//   at the end with shuffles, waves through LDS, and the workgroup writes
//   either the final normalized output (single partition) or its partial
//   (max, sum, unnormalized output) for the log-sum-exp merge.
#pragma once

#include <type_traits>

#include "device.h"
#include "quant.h"

namespace pa {

struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const uint16_t* k_scale;  // quantized caches only: fp16 [NB][Hkv][BS]
  const uint16_t* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;                // final output (single partition)
  float* part_ml;           // [S][Hq][P][2]: running max (log2 units), sum
  float* part_o;            // [S][Hq][P][D]: unnormalized output
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t group;            // Hq / Hkv
  int32_t head_chunks;      // group / GC
  int32_t part_tokens;      // multiple of the tile length
  int32_t num_parts;
  float scale_log2;         // scale * log2(e): scores are kept in log2 units
  // Fused append (optional): the decoded token's K and V rows [S][Hkv][D] in
  // the cache format.  The token sits at position context_len - 1; every
  // workgroup whose partition holds it stores the rows into the pool before
  // it reads the pool (identical bytes when several head chunks do so).
  const void* k_new;
  const void* v_new;
  // Sliding window (0: none): the token attends to the last `window`
  // positions, [ctx - window, ctx).  The grid then covers only the
  // partitions a window can touch: grid slot k of a sequence is the k-th
  // partition counted from the window's first tile (partition_start), and
  // partials are stored by slot (num_parts = slots); slots past the
  // sequence's end are left unwritten.
  int32_t window;
  int32_t tile;             // the plan's tile length (positions)
  // Paired plan (matrix-core kernel, one partition; 0: off): the grid's z
  // dimension holds ceil(num_seqs / 2) workgroups, and workgroup k attends
  // the k-th longest sequence, then the k-th shortest (paired_sequences).
  int32_t pair;
  int32_t num_seqs;
};

// Workgroup coordinates (partition, KV head x chunk, sequence).  Workgroups
// are dealt to the 8 XCDs round-robin by linear id; the linear id is
// renumbered so that each XCD runs one contiguous eighth of the
// (partition-fastest) grid.  Otherwise partition p of every sequence lands
// on XCD p mod 8: a windowed plan, whose active partitions are the last few
// of each sequence, would load two XCDs only, and the multi-partition
// headline plans run ~2-4 % faster this way as well (measured).
struct WgCoord {
  int part, y, s;
};
__device__ __forceinline__ WgCoord wg_coord() {
  const uint32_t nx = gridDim.x, ny = gridDim.y;
  const uint32_t n = nx * ny * gridDim.z;
  const uint32_t lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  constexpr uint32_t kXcds = 8;
  const uint32_t per = n / kXcds;                 // whole eighths; the tail stays put
  const uint32_t logical = lin < per * kXcds ? (lin % kXcds) * per + lin / kXcds : lin;
  return {(int)(logical % nx), (int)(logical / nx % ny), (int)(logical / (nx * ny))};
}

// First position a sequence attends to.
__device__ __forceinline__ int window_start(const DecodeParams& p, int ctx) {
  return p.window > 0 && ctx > p.window ? ctx - p.window : 0;
}

// First position of a grid slot's partition: slot * part_tokens, or for a
// windowed plan the slot-th partition from the tile holding the window's
// first position.  So a window splits into whole partitions from its first
// tile on, whatever its offset, and no partition is cut short at its start
// by an absolute partition boundary.
__device__ __forceinline__ int partition_start(const DecodeParams& p, int slot, int ctx) {
  if (p.window <= 0 || ctx < 0) return slot * p.part_tokens;
  const int start = window_start(p, ctx);
  return start - start % p.tile + slot * p.part_tokens;
}

// Sequences of a paired plan.  Two workgroups share each CU, and with ragged
// lengths the CUs that drew two long sequences finish last; taking a long and
// a short sequence in one workgroup evens out the work per CU.  The context
// lengths are ranked longest first, ties by index: a strict order whatever
// the lengths hold (broken ones included), so the ranks are a permutation and
// every sequence is taken exactly once.  Workgroup k takes ranks k and
// S - 1 - k; *second is -1 when they coincide (the middle of an odd S).
// Every thread of the workgroup must call this.
constexpr int kPairMaxSeqs = 256;
template <int NT>
__device__ __forceinline__ int paired_sequences(const DecodeParams& p, int k, int* second) {
  __shared__ __attribute__((aligned(16))) int s_ctx[kPairMaxSeqs];
  __shared__ int s_pick[2];
  const int S = p.num_seqs;
  const int S4 = (S + 3) / 4;
  // pad to whole int4s with INT_MIN: never longer, and past every index
  for (int i = threadIdx.x; i < 4 * S4; i += NT)
    s_ctx[i] = i < S ? p.context_lens[i] : INT32_MIN;
  __syncthreads();
  for (int i = threadIdx.x; i < S; i += NT) {
    const int ci = s_ctx[i];
    int rank = 0;
    for (int j4 = 0; j4 < S4; ++j4) {
      const int4 c = ((const int4*)s_ctx)[j4];
      const int j = 4 * j4;
      rank += (c.x > ci || (c.x == ci && j < i)) ? 1 : 0;
      rank += (c.y > ci || (c.y == ci && j + 1 < i)) ? 1 : 0;
      rank += (c.z > ci || (c.z == ci && j + 2 < i)) ? 1 : 0;
      rank += (c.w > ci || (c.w == ci && j + 3 < i)) ? 1 : 0;
    }
    if (rank == k) s_pick[0] = i;
    if (rank == S - 1 - k) s_pick[1] = i;
  }
  __syncthreads();
  *second = S - 1 - k != k ? s_pick[1] : -1;
  return s_pick[0];
}

template <Fmt F>
__device__ __forceinline__ void store_out(void* out, size_t idx, float x) {
  if constexpr (F == Fmt::F32) {
    ((float*)out)[idx] = x;
  } else if constexpr (F == Fmt::BF16) {
    ((uint16_t*)out)[idx] = float_to_bf16_rne(x);
  } else {  // fp16 output (also for the quantized caches)
    ((uint16_t*)out)[idx] = float_to_f16_rne(x);
  }
}

// Fused append: store the decoded token's K and V rows (head kvh of sequence
// s) at its slot, table[pos / BS] * BS + pos % BS, if the block id is valid,
// then make them visible to the whole workgroup before it reads the pool.
// Same-CU ordering only: the stores complete (workgroup-scope release) before
// the barrier, and no lane has read those lines yet in this launch.
template <int ROWB, int BS, int NT>
__device__ __forceinline__ void append_new_rows(const DecodeParams& p, const int32_t* table,
                                                int s, int kvh, int pos) {
  const int bid = table[pos / BS];
  if ((unsigned)bid < (unsigned)p.num_blocks) {
    const size_t dst = (((size_t)bid * p.num_kv_heads + kvh) * BS + pos % BS) * ROWB;
    const size_t src = ((size_t)s * p.num_kv_heads + kvh) * ROWB;
    for (int i = threadIdx.x; i < ROWB / 16; i += NT) {
      *(u32x4*)((char*)p.k_cache + dst + 16 * i) = load16((const char*)p.k_new + src + 16 * i);
      *(u32x4*)((char*)p.v_cache + dst + 16 * i) = load16((const char*)p.v_new + src + 16 * i);
    }
  }
  __threadfence_block();
  __syncthreads();
}

// Fused append into a quantized cache (int8, fp8, int4): the new rows come
// as fp16 [S][Hkv][D].  Wave 0 quantizes them, K on lanes [0, D/8) and V on
// lanes [D/8, D/4), 8 dims a lane, with the quantizer of the standalone
// quantizing append, and stores codes and scales at the token's slot; then
// the same workgroup-wide release as above.
template <Fmt F, int D, int BS>
__device__ __forceinline__ void append_new_rows_quant(const DecodeParams& p,
                                                      const int32_t* table, int s, int kvh,
                                                      int pos) {
  constexpr int KIND = quant_kind<F>();
  constexpr int LQ = D / 8;
  constexpr int LG = KIND == kQuantI4 ? kInt4Group / 8 : LQ;
  static_assert(2 * LQ <= kWave, "K and V rows must fit one wave");
  if (threadIdx.x < kWave) {  // wave 0: every lane takes part in the absmax
    const int lane = threadIdx.x;
    const bool is_v = lane >= LQ;
    const int c = lane % LQ;
    const int bid = table[pos / BS];
    const bool store = lane < 2 * LQ && (unsigned)bid < (unsigned)p.num_blocks;
    u32x4 x = {0, 0, 0, 0};
    if (store)
      x = load16((const char*)(is_v ? p.v_new : p.k_new) +
                 (((size_t)s * p.num_kv_heads + kvh) * D + 8 * c) * 2);
    uint32_t packed[2];
    const uint16_t sbits = quantize_piece<KIND, LG>(x, packed);
    if (store) {
      const size_t dst_row = ((size_t)bid * p.num_kv_heads + kvh) * BS + pos % BS;
      store_quant_piece<KIND, D>((uint8_t*)(is_v ? p.v_cache : p.k_cache),
                                 (uint16_t*)(is_v ? p.v_scale : p.k_scale), dst_row, c,
                                 packed, sbits);
    }
  }
  __threadfence_block();
  __syncthreads();
}

// The fused append of the decoded token at position pos, in the cache's
// format.  NT: threads of the workgroup.
template <Fmt F, int D, int BS, int NT>
__device__ __forceinline__ void append_new_token(const DecodeParams& p, const int32_t* table,
                                                 int s, int kvh, int pos) {
  if constexpr (FmtInfo<F>::quantized)
    append_new_rows_quant<F, D, BS>(p, table, s, kvh, pos);
  else
    append_new_rows<D * FmtInfo<F>::bytes, BS, NT>(p, table, s, kvh, pos);
}

// Per-format fragment arithmetic.  A fragment is 16 bytes of cache data.
template <Fmt F> struct Frag;

template <> struct Frag<Fmt::F32> {
  static constexpr int VE = 4;  // elements per fragment
  static constexpr int QW = 4;  // 32-bit words of query per fragment
  __device__ static __forceinline__ float dot(const uint32_t* q, u32x4 k) {
    float s = bits_to_float(q[0]) * bits_to_float(k[0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) s = fmaf(bits_to_float(q[i]), bits_to_float(k[i]), s);
    return s;
  }
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = bits_to_float(v[i]);
  }
};

template <> struct Frag<Fmt::F16> {
  static constexpr int VE = 8;
  static constexpr int QW = 4;
  __device__ static __forceinline__ float dot(const uint32_t* q, u32x4 k) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = __builtin_amdgcn_fdot2(as_h2(q[i]), as_h2(k[i]), s, false);
    return s;
  }
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16_lo(v[i]);
      f[2 * i + 1] = f16_hi(v[i]);
    }
  }
};

template <> struct Frag<Fmt::BF16> {
  static constexpr int VE = 8;
  static constexpr int QW = 4;
  __device__ static __forceinline__ float dot(const uint32_t* q, u32x4 k) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(q[i]), as_bf2(k[i]), s, false);
    return s;
  }
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(v[i]);
      f[2 * i + 1] = bf16_hi(v[i]);
    }
  }
};

// int8 codes: 16 per fragment, dotted with 16 fp16 query values.  Codes are
// turned into binary16 exactly: byte b = code + 128 placed under the exponent
// pattern 0x64 is the half 1024 + b; subtracting 1152 leaves the code.
template <> struct Frag<Fmt::I8> {
  static constexpr int VE = 16;
  static constexpr int QW = 8;
  __device__ static __forceinline__ void codes_to_half2(uint32_t w, h16x2& lo, h16x2& hi) {
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const h16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = as_h2(a) - bias;
    hi = as_h2(b) - bias;
  }
  __device__ static __forceinline__ float dot(const uint32_t* q, u32x4 k) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h16x2 lo, hi;
      codes_to_half2(k[i], lo, hi);
      s = __builtin_amdgcn_fdot2(as_h2(q[2 * i]), lo, s, false);
      s = __builtin_amdgcn_fdot2(as_h2(q[2 * i + 1]), hi, s, false);
    }
    return s;
  }
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * i + b] = (float)(int8_t)(v[i] >> (8 * b));
    }
  }
};

// fp8 E4M3 codes: 16 per fragment, dotted with 16 fp16 query values.  Codes
// are widened to their binary16 values exactly by the hardware conversion
// (e4m3x4_to_f16), two instructions per four codes.
template <> struct Frag<Fmt::FP8> {
  static constexpr int VE = 16;
  static constexpr int QW = 8;
  __device__ static __forceinline__ void codes_to_half2(uint32_t w, h16x2& lo, h16x2& hi) {
    uint32_t a, b;
    e4m3x4_to_f16(w, a, b);
    lo = as_h2(a);
    hi = as_h2(b);
  }
  __device__ static __forceinline__ float dot(const uint32_t* q, u32x4 k) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h16x2 lo, hi;
      codes_to_half2(k[i], lo, hi);
      s = __builtin_amdgcn_fdot2(as_h2(q[2 * i]), lo, s, false);
      s = __builtin_amdgcn_fdot2(as_h2(q[2 * i + 1]), hi, s, false);
    }
    return s;
  }
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h16x2 lo, hi;
      codes_to_half2(v[i], lo, hi);
      f[4 * i] = (float)lo[0];
      f[4 * i + 1] = (float)lo[1];
      f[4 * i + 2] = (float)hi[0];
      f[4 * i + 3] = (float)hi[1];
    }
  }
};

// int4 codes: 32 per fragment (8 per word, dim i of a word in nibble i, as
// code + 8), dotted with 32 fp16 query values; a fragment is one scale group.
// Nibbles k and k+4 of a word come out together: (w >> 4k) & 0x000F000F under
// the exponent pattern 0x6400 is the half pair 1024 + code + 8, minus 1032
// gives the codes exactly.  The query words are regrouped once (prep_q) into
// the same (k, k+4) pairs.
template <> struct Frag<Fmt::I4> {
  static constexpr int VE = 32;
  static constexpr int QW = 16;
  __device__ static __forceinline__ h16x2 pair(uint32_t w, int k) {
    const h16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    return as_h2(((w >> (4 * k)) & 0x000F000Fu) | 0x64006400u) - bias;
  }
  __device__ static __forceinline__ void prep_q(uint32_t* q) {
    uint32_t r[QW];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // halves 8j+k and 8j+k+4 of the lane's 32 query values
        const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
        r[4 * j + k] = __builtin_amdgcn_perm(q[4 * j + 2 + k / 2], q[4 * j + k / 2], sel);
      }
    }
#pragma unroll
    for (int i = 0; i < QW; ++i) q[i] = r[i];
  }
  __device__ static __forceinline__ float dot(const uint32_t* q, u32x4 k) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s = __builtin_amdgcn_fdot2(as_h2(q[4 * j + kk]), pair(k[j], kk), s, false);
    }
    return s;
  }
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h16x2 h = pair(v[j], kk);
        f[8 * j + kk] = (float)h[0];
        f[8 * j + kk + 4] = (float)h[1];
      }
    }
  }
};

// Result of one workgroup for one query head row of one sequence: final when
// the partition is the sequence's only one, else a partial (running max M in
// log2 units, sum L, unnormalized output) for the log-sum-exp merge.
template <Fmt F, int D>
__device__ __forceinline__ void store_result(const DecodeParams& p, bool direct, size_t row,
                                             int part, int d, float M, float L, float o) {
  if (direct) {
    store_out<F>(p.out, row * D + d, o / L);
  } else {
    const size_t slot = row * p.num_parts + part;
    p.part_o[slot * D + d] = o;
    if (d == 0) {
      p.part_ml[2 * slot] = M;
      p.part_ml[2 * slot + 1] = L;
    }
  }
}

// Occupancy hint of the vector-ALU kernel (minimum waves per SIMD): 8, 4
// or 1 for 1, 2 or 8 heads per workgroup; int4 lanes hold 32 values per head
// (the others 16 or fewer), so they get twice the registers.  It is halved
// when one head's rows of a block reach 8 KiB with every format but fp16
// counted as 4 bytes (bf16, int8 and fp8 are widened before use), and
// quartered when they reach 16 KiB with fp32 and int8 counted as 4 bytes and
// the others as 2.  At the full hint those instances spilled 9-414 VGPRs;
// measured on MI355X, the reduced hint ran them 1.2-2.8x faster.
template <Fmt F, int D, int BS, int GC>
constexpr int valu_waves_per_simd() {
  if constexpr (F == Fmt::I4) return GC == 1 ? 4 : 2;
  const int base = GC == 1 ? 8 : GC == 2 ? 4 : 1;
  const int wide = F == Fmt::F16 ? 2 : 4;                         // bytes, for halving
  const int big = F == Fmt::F32 || F == Fmt::I8 ? 4 : 2;          // bytes, for quartering
  const int div = BS * D * big >= 16384 ? 4 : BS * D * wide >= 8192 ? 2 : 1;
  return base / div > 0 ? base / div : 1;
}

template <Fmt F, int D, int BS, int GC, int NW>
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu(valu_waves_per_simd<F, D, BS, GC>(), 8)))
void decode_partition_kernel(const DecodeParams p) {
  using FR = Frag<F>;
  constexpr int QB = FmtInfo<F>::q_bytes;     // bytes per query element
  constexpr int VE = FR::VE;                  // elements per 16-byte fragment
  constexpr int LR = D / VE;                  // lanes per row
  constexpr int RPI = kWave / LR;             // rows per wave-load
  constexpr int TT = BS > RPI ? BS : RPI;     // positions per tile
  constexpr int NJ = TT / RPI;                // fragments per lane per tile (K, and V)
  constexpr int BPT = TT / BS;                // blocks per tile
  constexpr int ROWB = LR * 16;               // bytes per cached row (D * CB, or D / 2)
  constexpr bool kInt4 = F == Fmt::I4;
  constexpr int SPR = kInt4 ? D / kInt4Group : 1;  // scales per cached row
  constexpr bool kQuant = FmtInfo<F>::quantized;
  static_assert(LR >= 1 && LR <= kWave && (kWave % LR) == 0, "row must split over lanes");
  static_assert(TT % RPI == 0 && TT % BS == 0, "tile must be whole loads and blocks");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const WgCoord wc = wg_coord();
  const int slot = wc.part;
  const int kvh = wc.y / p.head_chunks;
  const int chunk = wc.y - kvh * p.head_chunks;
  const int s = wc.s;
  const int h0 = kvh * p.group + chunk * GC;
  const size_t out_row0 = (size_t)s * p.num_q_heads + h0;

  const int ctx = p.context_lens[s];
  const bool single = p.num_parts == 1;
  const int tok0 = partition_start(p, slot, ctx);
  const bool bad_ctx = ctx < 0 || ctx > p.max_blocks * BS;
  if (bad_ctx || tok0 >= ctx) {
    // Nothing to attend in this partition.  The merge skips it; a single
    // pass writes the final rows: NaN for a broken length, zeros for ctx 0.
    if (single) {
      const float fill = bad_ctx ? __builtin_nanf("") : 0.0f;
      for (int i = threadIdx.x; i < GC * D; i += NW * kWave)
        store_out<F>(p.out, out_row0 * D + i, fill);
    }
    return;
  }
  const int tok_end = min(ctx, tok0 + p.part_tokens);
  const int start = window_start(p, ctx);
  if (tok_end <= start) {  // wholly before the window (never the only partition)
    for (int i = threadIdx.x; i < GC * D; i += NW * kWave)
      store_result<F, D>(p, false, out_row0 + i / D, slot, i % D, kMaxInit, 0.0f, 0.0f);
    return;
  }
  const int ntiles = (tok_end - tok0 + TT - 1) / TT;
  const int t_first = (max(tok0, start) - tok0) / TT;   // first tile holding the window
  const bool low_cut = start > tok0 + t_first * TT;      // which then starts mid-tile
  const int32_t* __restrict__ table = p.block_tables + (size_t)s * p.max_blocks;
  // Fused append: the decoded token (position ctx-1) is this partition's last
  // row when tok_end == ctx.
  if (p.k_new != nullptr && tok_end == ctx)
    append_new_token<F, D, BS, NW * kWave>(p, table, s, kvh, ctx - 1);

  const int lrow = lane / LR;  // row of this lane inside a wave-load
  const int lcol = lane % LR;  // 16-byte column of this lane inside a row

  // Query slices this lane multiplies: elements [lcol*VE, lcol*VE+VE).
  uint32_t qf[GC][FR::QW];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const uint32_t* qp = (const uint32_t*)((const char*)p.q +
                                           ((out_row0 + g) * D + (size_t)lcol * VE) * QB);
#pragma unroll
    for (int w = 0; w < FR::QW; ++w) qf[g][w] = qp[w];
    if constexpr (kInt4) FR::prep_q(qf[g]);
  }

  float m[GC], l[GC], acc[GC][VE];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    m[g] = kMaxInit;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[g][e] = 0.0f;
  }
  bool bad_block = false;

  const char* __restrict__ kbase = (const char*)p.k_cache;
  const char* __restrict__ vbase = (const char*)p.v_cache;
  // Block ids of the partition, 64 at a time in one coalesced load: lane i
  // holds the id of block ids_base + i (counted from the partition's first
  // block); a tile then reads its ids with v_readlane, without a memory trip.
  const int blk0 = tok0 / BS;
  const int nblk = (tok_end + BS - 1) / BS - blk0;
  int ids = 0;
  int ids_base = -kWave;
  auto tile = [&](const int t, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    const int ttok = tok0 + t * TT;
    const int nvalid = tok_end - ttok;  // rows of the tile inside the partition
    const int nlow = start - ttok;      // rows below this are before the window
    const int lb = t * BPT;             // first block of the tile
    if (lb >= ids_base + kWave) {       // a wave's tiles come in increasing order
      ids_base = lb & ~(kWave - 1);
      const int bi = ids_base + lane;
      ids = bi < nblk ? table[blk0 + bi] : 0;
    }
    int phys[BPT];
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int id = __builtin_amdgcn_readlane(ids, lb - ids_base + b);
      const bool ok = (unsigned)id < (unsigned)p.num_blocks;
      // a block wholly before the window is never read: its entry may be stale
      const bool needed = !PARTIAL || (b + 1) * BS > nlow;
      bad_block |= !ok && needed;
      phys[b] = ok ? id : 0;
    }
    u32x4 kf[NJ], vf[NJ];
    float ks[NJ], vs[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = j * RPI + lrow;  // row inside the tile
      int pid = phys[0];
#pragma unroll
      for (int b = 1; b < BPT; ++b) pid = (r / BS == b) ? phys[b] : pid;
      const size_t row = ((size_t)pid * p.num_kv_heads + kvh) * BS + (BPT == 1 ? r : r % BS);
      const size_t off = row * ROWB + (size_t)lcol * 16;
      const bool valid = !PARTIAL || (r >= nlow && r < nvalid);
      if (valid) {
        kf[j] = load16_stream(kbase + off);
        vf[j] = load16_stream(vbase + off);
      } else {
        kf[j] = u32x4{0, 0, 0, 0};
        vf[j] = u32x4{0, 0, 0, 0};
      }
      if constexpr (kQuant) {
        // int4: the lane's 32 dims are scale group lcol of the row
        const size_t si = kInt4 ? row * SPR + lcol : row;
        ks[j] = valid ? (float)__builtin_bit_cast(_Float16, p.k_scale[si]) : 0.0f;
        vs[j] = valid ? (float)__builtin_bit_cast(_Float16, p.v_scale[si]) : 0.0f;
      } else {
        ks[j] = 1.0f;
        vs[j] = 1.0f;
      }
    }
    // Keep every K and V load of the tile ahead of the arithmetic, so that
    // the whole tile is in flight at once (one memory round trip per tile).
    __builtin_amdgcn_sched_barrier(0);
    // Scores of every (head, fragment row), summed across the row's lanes.
    float z[GC][NJ];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float z0;
        if constexpr (kInt4) {  // each lane's group has its own scale
          z0 = group_sum<LR>(FR::dot(qf[g], kf[j]) * ks[j]) * p.scale_log2;
        } else {
          const float d = group_sum<LR>(FR::dot(qf[g], kf[j]));
          z0 = kQuant ? d * (ks[j] * p.scale_log2) : d * p.scale_log2;
        }
        z[g][j] = z0;
        if (PARTIAL && (j * RPI + lrow >= nvalid || j * RPI + lrow < nlow))
          z[g][j] = -__builtin_inff();
      }
    }
    float vv[NJ][VE];
#pragma unroll
    for (int j = 0; j < NJ; ++j) FR::unpack(vf[j], vv[j]);
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float mt = z[g][0];
#pragma unroll
      for (int j = 1; j < NJ; ++j) mt = fmaxf(mt, z[g][j]);
      const float mn = fmaxf(m[g], mt);
      const float alpha = fast_exp2(m[g] - mn);
      m[g] = mn;
      float lsum = l[g] * alpha;
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float pj = fast_exp2(z[g][j] - mn);
        lsum += pj;
        const float pv = kQuant ? pj * vs[j] : pj;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(pv, vv[j][e], acc[g][e]);
      }
      l[g] = lsum;
    }
  };

  const int nfull = (tok_end - tok0) / TT;  // tiles with every row valid
  for (int t = t_first + wave; t < ntiles; t += NW) {
    if (t < nfull && !(low_cut && t == t_first)) tile(t, std::false_type{});
    else tile(t, std::true_type{});
  }

  // Merge the row groups of the wave (lanes lcol, lcol+LR, ...).
#pragma unroll
  for (int off = LR; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float a = fast_exp2(m[g] - mn);
      const float b = fast_exp2(mo - mn);
      l[g] = l[g] * a + lo * b;
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float ao = __shfl_xor(acc[g][e], off);
        acc[g][e] = acc[g][e] * a + ao * b;
      }
      m[g] = mn;
    }
  }

  // Merge the waves through LDS and write the result.
  __shared__ float s_ml[NW][GC][2];
  __shared__ float s_acc[NW][GC][D];
  if (lane < LR) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
#pragma unroll
      for (int e = 0; e < VE; ++e) s_acc[wave][g][lcol * VE + e] = acc[g][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      s_ml[wave][g][0] = m[g];
      s_ml[wave][g][1] = l[g];
    }
  }
  const bool bad = __syncthreads_or(bad_block ? 1 : 0) != 0;
  for (int i = threadIdx.x; i < GC * D; i += NW * kWave) {
    const int g = i / D;
    const int d = i - g * D;
    float M = s_ml[0][g][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][g][0]);
    float L = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = fast_exp2(s_ml[w][g][0] - M);
      L = fmaf(a, s_ml[w][g][1], L);
      o = fmaf(a, s_acc[w][g][d], o);
    }
    if (bad) M = L = o = __builtin_nanf("");
    store_result<F, D>(p, single, out_row0 + g, slot, d, M, L, o);
  }
}

// Waves per workgroup of the decode kernel.
constexpr int kDecodeWaves = 4;

// Positions per tile for a format / head_dim / block size (host and device).
__host__ __device__ constexpr int tile_tokens(int elem_bytes, int head_dim, int block_size) {
  // 16-byte fragments: head_dim*elem_bytes/16 lanes per row, 64/that rows per load.
  return block_size > (64 * 16) / (head_dim * elem_bytes) ? block_size
                                                           : (64 * 16) / (head_dim * elem_bytes);
}

}  // namespace pa
