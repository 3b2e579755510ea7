// kv_ops.hip -- slot mapping, append (plain and int8-quantizing) and the
// un-paging gather, for gfx950.
//
// A sequence's positions live in fixed-size blocks of one shared pool, listed
// in order by its block table; the slot of position pos is
// table[pos / BS] * BS + pos % BS ("PagedAttention: the cache in blocks",
// KV-cache visualization page).  A decode step appends the new token's K and
// V rows at its slot ("KV cache: the engine behind fast LLM inference",
// "What happens at each decoding step", step 4).
#include <algorithm>

#include "kv_ops.h"
#include "quant.h"

namespace pa {

// ---------------------------------------------------------------- slots

__global__ void slot_mapping_kernel(const int32_t* __restrict__ tables, int32_t max_blocks,
                                    int32_t num_seqs, const int32_t* __restrict__ token_seq,
                                    const int32_t* __restrict__ token_pos, int64_t num_tokens,
                                    int32_t block_size, int64_t* __restrict__ slots) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  const int32_t s = token_seq[t];
  const int32_t pos = token_pos[t];
  int64_t slot = -1;
  if (s >= 0 && s < num_seqs && pos >= 0 && pos < max_blocks * block_size) {
    const int32_t block = tables[(int64_t)s * max_blocks + pos / block_size];
    slot = (int64_t)block * block_size + pos % block_size;
  }
  slots[t] = slot;
}

__global__ void decode_slot_mapping_kernel(const int32_t* __restrict__ tables,
                                           int32_t max_blocks,
                                           const int32_t* __restrict__ context_lens,
                                           int32_t num_seqs, int32_t block_size,
                                           int64_t* __restrict__ slots) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= num_seqs) return;
  const int32_t ctx = context_lens[s];
  int64_t slot = -1;
  if (ctx > 0 && ctx <= max_blocks * block_size) {
    const int32_t pos = ctx - 1;
    const int32_t block = tables[(int64_t)s * max_blocks + pos / block_size];
    slot = (int64_t)block * block_size + pos % block_size;
  }
  slots[s] = slot;
}

// ---------------------------------------------------------------- slot check

// A slot names one position of one block, so the tokens of one append must
// not share a slot; a slot past the pool names no position at all.  Flags,
// OR-ed into *flags (zeroed by the launcher's first kernel): bit 0 a
// repeated slot (>= 0), bit 1 a slot >= pool_slots.  Negative slots are
// pads and are never compared.  Token i is compared with every j < i, in
// LDS tiles of kSlotTile slots (O(T^2 / 2) compares).
constexpr int kSlotTile = 256;

__global__ void zero_flag_kernel(int32_t* flags) { *flags = 0; }

__global__ __launch_bounds__(kSlotTile) void check_slots_kernel(
    const int64_t* __restrict__ slots, int64_t num_tokens, int64_t pool_slots,
    int32_t* __restrict__ flags) {
  __shared__ int64_t tile[kSlotTile];
  const int64_t i = (int64_t)blockIdx.x * kSlotTile + threadIdx.x;
  const int64_t mine = i < num_tokens ? slots[i] : -1;
  int32_t found = mine >= pool_slots ? 2 : 0;
  for (int64_t base = 0; base <= (int64_t)blockIdx.x * kSlotTile; base += kSlotTile) {
    const int64_t j = base + threadIdx.x;
    tile[threadIdx.x] = j < num_tokens ? slots[j] : -1;
    __syncthreads();
    if (mine >= 0) {
      const int64_t upto = i - base < kSlotTile ? i - base : kSlotTile;   // j < i only
      for (int64_t k = 0; k < upto; ++k) found |= tile[k] == mine ? 1 : 0;
    }
    __syncthreads();
  }
  // one vector atomic per wave that found something
  const uint64_t any = __builtin_amdgcn_ballot_w64(found != 0);
  if (any != 0) {
    int32_t bits = found;
    for (int off = 32; off > 0; off >>= 1) bits |= __shfl_xor(bits, off);
    if ((threadIdx.x & (kWave - 1)) == 0)
      __hip_atomic_fetch_or(flags, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_check_slots(const int64_t* slots, int64_t num_tokens, int64_t pool_slots,
                              int32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(1), 0, stream, flags);
  if (num_tokens > 0)
    hipLaunchKernelGGL(check_slots_kernel, dim3((unsigned)((num_tokens + kSlotTile - 1) / kSlotTile)),
                       dim3(kSlotTile), 0, stream, slots, num_tokens, pool_slots, flags);
  return hipGetLastError();
}

// ---------------------------------------------------------------- append

// One thread per 16-byte piece of a (token, head) row; K and V together.
__global__ void kv_append_kernel(const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
                                 const int64_t* __restrict__ slots, int64_t num_tokens,
                                 u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
                                 int32_t num_kv_heads, int32_t block_size, int32_t pieces,
                                 int64_t pool_slots) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)num_kv_heads * pieces;
  if (i >= num_tokens * per_token) return;
  const int64_t t = i / per_token;
  const int64_t rest = i - t * per_token;  // = h * pieces + c
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= pool_slots) return;
  const int64_t block = slot / block_size;
  const int64_t off = slot - block * block_size;
  const int64_t h = rest / pieces;
  const int64_t c = rest - h * pieces;
  const int64_t dst = ((block * num_kv_heads + h) * block_size + off) * pieces + c;
  k_cache[dst] = k_new[i];
  v_cache[dst] = v_new[i];
}

// Quantizing append.  LQ = D/8 lanes hold one (token, head) row of fp16
// values, 8 each; the quantizer and its reading of the pages are in quant.h
// (KIND 0: int8, 1: fp8 E4M3, both with one fp16 scale per row; KIND 2: int4,
// with one scale per group of kInt4Group dims, the 4 lanes of the group).
template <int D, int KIND>
__global__ __launch_bounds__(256) void kv_append_quant_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
    const int64_t* __restrict__ slots, int64_t num_tokens, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, uint16_t* __restrict__ k_scale, uint16_t* __restrict__ v_scale,
    int32_t num_kv_heads, int32_t block_size, int64_t pool_slots) {
  constexpr int LQ = D / 8;  // lanes per row
  constexpr int LG = KIND == kQuantI4 ? kInt4Group / 8 : LQ;  // lanes sharing a scale
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / LQ;        // (token, head) row
  const int c = (int)(gid % LQ);       // 8-value piece of the row
  const bool live = row < num_tokens * num_kv_heads;
  const int64_t t = live ? row / num_kv_heads : 0;
  const int64_t h = live ? row - t * num_kv_heads : 0;
  const int64_t slot = live ? slots[t] : -1;
  const bool store = live && slot >= 0 && slot < pool_slots;
  // Rows are whole lane groups, so a group shares 'store'; every lane still
  // takes part in the reductions.
  u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
  if (store) {
    kx = k_new[row * LQ + c];
    vx = v_new[row * LQ + c];
  }
  uint32_t kp[2], vp[2];
  const uint16_t ks = quantize_piece<KIND, LG>(kx, kp);
  const uint16_t vs = quantize_piece<KIND, LG>(vx, vp);
  if (store) {
    const int64_t block = slot / block_size;
    const int64_t off = slot - block * block_size;
    const size_t dst_row = (size_t)((block * num_kv_heads + h) * block_size + off);
    store_quant_piece<KIND, D>(k_cache, k_scale, dst_row, c, kp, ks);
    store_quant_piece<KIND, D>(v_cache, v_scale, dst_row, c, vp, vs);
  }
}

// ---------------------------------------------------------------- gather

// Grid-stride over (sequence, position, head, 16-byte piece) of the dense
// output; positions at or past the context length are not written.
__global__ void gather_kv_kernel(const char* __restrict__ k_cache, const char* __restrict__ v_cache,
                                 const uint16_t* __restrict__ k_scale,
                                 const uint16_t* __restrict__ v_scale,
                                 const int32_t* __restrict__ tables, int32_t max_blocks,
                                 const int32_t* __restrict__ context_lens, int32_t num_seqs,
                                 char* __restrict__ k_out, char* __restrict__ v_out,
                                 uint16_t* __restrict__ k_scale_out,
                                 uint16_t* __restrict__ v_scale_out, int32_t num_blocks,
                                 int32_t num_kv_heads, int32_t block_size, int32_t row_bytes,
                                 int32_t scales_per_row) {
  const int32_t pieces = row_bytes / 16;
  const int64_t cap = (int64_t)max_blocks * block_size;
  const int64_t total = (int64_t)num_seqs * cap * num_kv_heads * pieces;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i;
    const int32_t c = (int32_t)(r % pieces); r /= pieces;
    const int32_t h = (int32_t)(r % num_kv_heads); r /= num_kv_heads;
    const int32_t pos = (int32_t)(r % cap);
    const int32_t s = (int32_t)(r / cap);
    const int32_t ctx = context_lens[s];
    if (ctx < 0 || ctx > cap || pos >= ctx) continue;
    const int32_t block = tables[(int64_t)s * max_blocks + pos / block_size];
    if (block < 0 || block >= num_blocks) continue;
    const int64_t src_row = ((int64_t)block * num_kv_heads + h) * block_size + pos % block_size;
    const int64_t dst_row = ((int64_t)s * cap + pos) * num_kv_heads + h;
    *(u32x4*)(k_out + dst_row * row_bytes + c * 16) =
        *(const u32x4*)(k_cache + src_row * row_bytes + c * 16);
    *(u32x4*)(v_out + dst_row * row_bytes + c * 16) =
        *(const u32x4*)(v_cache + src_row * row_bytes + c * 16);
    // scales: one per row, or (int4) one per 16-byte piece = 32 dims
    if (c < scales_per_row && k_scale && k_scale_out)
      k_scale_out[dst_row * scales_per_row + c] = k_scale[src_row * scales_per_row + c];
    if (c < scales_per_row && v_scale && v_scale_out)
      v_scale_out[dst_row * scales_per_row + c] = v_scale[src_row * scales_per_row + c];
  }
}

// ---------------------------------------------------------------- launchers

static inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

hipError_t launch_slot_mapping(const int32_t* tables, int32_t max_blocks, int32_t num_seqs,
                               const int32_t* token_seq, const int32_t* token_pos,
                               int64_t num_tokens, int32_t block_size, int64_t* slots,
                               hipStream_t stream) {
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks_for(num_tokens, 256)), dim3(256), 0, stream,
                     tables, max_blocks, num_seqs, token_seq, token_pos, num_tokens, block_size,
                     slots);
  return hipGetLastError();
}

hipError_t launch_decode_slot_mapping(const int32_t* tables, int32_t max_blocks,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t block_size, int64_t* slots, hipStream_t stream) {
  hipLaunchKernelGGL(decode_slot_mapping_kernel, dim3(blocks_for(num_seqs, 256)), dim3(256), 0,
                     stream, tables, max_blocks, context_lens, num_seqs, block_size, slots);
  return hipGetLastError();
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slots,
                            int64_t num_tokens, void* k_cache, void* v_cache,
                            int32_t num_kv_heads, int32_t block_size, int32_t row_bytes,
                            int64_t pool_slots, hipStream_t stream) {
  const int32_t pieces = row_bytes / 16;
  const int64_t n = num_tokens * num_kv_heads * pieces;
  hipLaunchKernelGGL(kv_append_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, stream,
                     (const u32x4*)k_new, (const u32x4*)v_new, slots, num_tokens,
                     (u32x4*)k_cache, (u32x4*)v_cache, num_kv_heads, block_size, pieces,
                     pool_slots);
  return hipGetLastError();
}

hipError_t launch_kv_append_quant(const void* k_new, const void* v_new, const int64_t* slots,
                                  int64_t num_tokens, void* k_cache, void* v_cache,
                                  void* k_scale, void* v_scale, int32_t num_kv_heads,
                                  int32_t block_size, int32_t head_dim, int64_t pool_slots,
                                  int kind, hipStream_t stream) {
  const int64_t lanes = num_tokens * num_kv_heads * (head_dim / 8);
  const dim3 grid(blocks_for(lanes, 256));
#define PA_APPEND_Q(D, KIND)                                                                   \
  hipLaunchKernelGGL((kv_append_quant_kernel<D, KIND>), grid, dim3(256), 0, stream,             \
                     (const u32x4*)k_new, (const u32x4*)v_new, slots, num_tokens,               \
                     (uint8_t*)k_cache, (uint8_t*)v_cache, (uint16_t*)k_scale,                  \
                     (uint16_t*)v_scale, num_kv_heads, block_size, pool_slots)
  if (kind < 0 || kind > 2) return hipErrorInvalidValue;
  if (head_dim == 64) {
    if (kind == 0) PA_APPEND_Q(64, 0);
    else if (kind == 1) PA_APPEND_Q(64, 1);
    else PA_APPEND_Q(64, 2);
  } else if (head_dim == 128) {
    if (kind == 0) PA_APPEND_Q(128, 0);
    else if (kind == 1) PA_APPEND_Q(128, 1);
    else PA_APPEND_Q(128, 2);
  } else {
    return hipErrorInvalidValue;
  }
#undef PA_APPEND_Q
  return hipGetLastError();
}

hipError_t launch_gather_kv(const void* k_cache, const void* v_cache, const void* k_scale,
                            const void* v_scale, const int32_t* tables, int32_t max_blocks,
                            const int32_t* context_lens, int32_t num_seqs, void* k_out,
                            void* v_out, void* k_scale_out, void* v_scale_out,
                            int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                            int32_t row_bytes, int32_t scales_per_row, hipStream_t stream) {
  const int64_t total = (int64_t)num_seqs * max_blocks * block_size * num_kv_heads * (row_bytes / 16);
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? (want > 0 ? want : 1) : 65536);
  hipLaunchKernelGGL(gather_kv_kernel, dim3(grid), dim3(256), 0, stream, (const char*)k_cache,
                     (const char*)v_cache, (const uint16_t*)k_scale, (const uint16_t*)v_scale,
                     tables, max_blocks, context_lens, num_seqs, (char*)k_out, (char*)v_out,
                     (uint16_t*)k_scale_out, (uint16_t*)v_scale_out, num_blocks, num_kv_heads,
                     block_size, row_bytes, scales_per_row);
  return hipGetLastError();
}

// ---------------------------------------------------------------- block copy

// Copy-on-write of shared blocks: one workgroup moves one 16 KiB chunk of a
// (source, destination) pair's K or V rows (every KV head of a block is one
// contiguous run), plus, in chunk 0, the pair's int8 scales.
constexpr int64_t kCopyChunkPieces = 1024;  // 16-byte pieces per workgroup

__global__ __launch_bounds__(256) void copy_blocks_kernel(
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache, uint16_t* __restrict__ k_scale,
    uint16_t* __restrict__ v_scale, const int32_t* __restrict__ pairs, int32_t num_blocks,
    int64_t block_pieces, int32_t scale_elems, int32_t chunks) {
  const int64_t pair = blockIdx.x;
  const int32_t src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int which = (int)blockIdx.y / chunks;  // 0: K, 1: V
  const int64_t chunk = (int64_t)blockIdx.y - (int64_t)which * chunks;
  u32x4* cache = which ? v_cache : k_cache;
  const u32x4* from = cache + (int64_t)src * block_pieces;
  u32x4* to = cache + (int64_t)dst * block_pieces;
  const int64_t begin = chunk * kCopyChunkPieces;
  const int64_t end = begin + kCopyChunkPieces < block_pieces ? begin + kCopyChunkPieces : block_pieces;
  int64_t i = begin + threadIdx.x;
  for (; i + 3 * 256 < end; i += 4 * 256) {
    const u32x4 a = from[i], b = from[i + 256], c = from[i + 512], d = from[i + 768];
    to[i] = a;
    to[i + 256] = b;
    to[i + 512] = c;
    to[i + 768] = d;
  }
  for (; i < end; i += 256) to[i] = from[i];
  uint16_t* scales = which ? v_scale : k_scale;
  if (chunk == 0 && scales) {
    for (int32_t j = threadIdx.x; j < scale_elems; j += 256)
      scales[(int64_t)dst * scale_elems + j] = scales[(int64_t)src * scale_elems + j];
  }
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                              const int32_t* pairs, int32_t num_pairs, int32_t num_blocks,
                              int32_t num_kv_heads, int32_t block_size, int32_t row_bytes,
                              int32_t scales_per_row, hipStream_t stream) {
  const int64_t block_pieces = (int64_t)num_kv_heads * block_size * (row_bytes / 16);
  const int32_t chunks = (int32_t)((block_pieces + kCopyChunkPieces - 1) / kCopyChunkPieces);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2 * chunks), dim3(256), 0, stream,
                     (u32x4*)k_cache, (u32x4*)v_cache, (uint16_t*)k_scale, (uint16_t*)v_scale,
                     pairs, num_blocks, block_pieces, num_kv_heads * block_size * scales_per_row, chunks);
  return hipGetLastError();
}

// ---- HBM read-rate probe: each wave reads whole 4 KiB chunks (4 loads of
// 16 bytes per lane) in a grid-stride loop over the chunk order; a store that
// depends on the data keeps the loads alive.
constexpr int kProbeThreads = 256;
constexpr int kProbeChunkWords = 4096 / 16;
constexpr uint32_t kProbeNever = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(
    const u32x4* __restrict__ src, const int32_t* __restrict__ order, int64_t chunks,
    uint32_t* sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (kProbeThreads / kWave);
  uint32_t acc = 0;
  for (int64_t c = (int64_t)blockIdx.x * (kProbeThreads / kWave) + threadIdx.x / kWave; c < chunks;
       c += waves) {
    int64_t ch = order ? order[c] : c;
    ch = (uint64_t)ch < (uint64_t)chunks ? ch : 0;
    const u32x4* p = src + ch * kProbeChunkWords + lane;
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + u * kWave);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == kProbeNever) sink[0] = acc;
}

hipError_t launch_hbm_read_probe(const void* src, size_t bytes, const int32_t* chunk_order,
                                 uint32_t* sink, hipStream_t stream) {
  const int64_t chunks = (int64_t)(bytes / 4096);
  // 4 workgroups of 4 waves per CU on 256 CUs (measured best for both
  // orders), or fewer for a small buffer
  const int64_t wgs = std::min<int64_t>(1024, (chunks + 3) / 4);
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3((unsigned)wgs), dim3(kProbeThreads), 0, stream,
                     (const u32x4*)src, chunk_order, chunks, sink);
  return hipGetLastError();
}

}  // namespace pa
