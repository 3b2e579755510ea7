// lse_merge.hip -- log-sum-exp merge of context partitions (phase 2).
//
// Each partition p of a sequence left (m_p, l_p, o_p): its running max (log2
// units), the sum of 2^(z_i - m_p) and the unnormalized sum of those weights
// times the value rows.  Rescaling every partition to the common max
// M = max_p m_p and dividing by the rescaled total gives exactly the softmax
// of the whole context, because splitting the sum in pieces changes nothing
// in exact arithmetic (the guide's "Flash attention: don't build the giant
// matrix": tiling leaves the math as it is).
//
// The launch is tiny (a few hundred KiB of partials) and latency-bound, so
// the kernel is shaped for one memory round trip: a wave takes whole rows
// (64 / (D/4) query-head rows per wave, four output dims per lane), and every
// lane issues the loads of all partitions' (m, l) pairs and its 16-byte
// slice of their outputs at once, together with the sequence's length.
// Slots past the sequence's last partition are loaded too (they lie inside
// the workspace) and masked once the length is known.
#include "kv_ops.h"

namespace pa {

constexpr int kMergeThreads = 64;   // one wave per workgroup
constexpr int kMergeBatch = 8;      // partitions loaded per round trip

template <int OUT_FMT>
__device__ __forceinline__ void store_out4(void* out, size_t idx, const float (&r)[4]) {
  if constexpr (OUT_FMT == (int)Fmt::F32) {
    *(float4*)((float*)out + idx) = make_float4(r[0], r[1], r[2], r[3]);
  } else {
    uint16_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      h[i] = OUT_FMT == (int)Fmt::BF16 ? float_to_bf16_rne(r[i]) : float_to_f16_rne(r[i]);
    const uint32_t lo = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    const uint32_t hi = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    *(uint2*)((uint16_t*)out + idx) = make_uint2(lo, hi);
  }
}

// Merge of one row (sequence s, query head) over its partitions, four dims
// per lane.  The arithmetic order is fixed: the max over the used
// partitions, then the weighted sums in partition order.
template <int OUT_FMT, int D>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_tokens, int32_t part_tokens, int32_t num_parts, int32_t window, int32_t tile,
    void* __restrict__ out) {
  constexpr int LANES = D / 4;                      // lanes per row
  constexpr int ROWS = kMergeThreads / LANES;       // rows per workgroup
  const int lane = threadIdx.x % LANES;
  const size_t row = (size_t)blockIdx.x * ROWS + threadIdx.x / LANES;
  if (row >= (size_t)num_seqs * num_q_heads) return;
  const int s = (int)(row / num_q_heads);
  const float2* ml = (const float2*)(part_ml + row * num_parts * 2);
  const float4* o = (const float4*)(part_o + row * num_parts * D) + lane;

  // Every load of the first batch goes out before the length is used.
  const int ctx = context_lens[s];
  float2 m_l[kMergeBatch];
  float4 o_p[kMergeBatch];
#pragma unroll
  for (int p = 0; p < kMergeBatch; ++p) {
    if (p < num_parts) {
      m_l[p] = ml[p];
      o_p[p] = o[(size_t)p * (D / 4)];
    }
  }

  float r[4];
  if (ctx < 0 || ctx > max_tokens) {
    r[0] = r[1] = r[2] = r[3] = __builtin_nanf("");
  } else if (ctx == 0) {
    r[0] = r[1] = r[2] = r[3] = 0.0f;
  } else {
    // partitions (slots) the sequence used: all up to its end, or for a
    // sliding window those counted from the tile holding the window's first
    // position (the attention kernels' partition_start)
    const int start = window > 0 && ctx > window ? ctx - window : 0;
    const int base = start > 0 ? start - start % tile : 0;     // tile > 0 whenever start > 0
    const int np = (ctx - base + part_tokens - 1) / part_tokens;
    float M = -__builtin_inff();
#pragma unroll
    for (int p = 0; p < kMergeBatch; ++p)
      if (p < np) M = fmaxf(M, m_l[p].x);
    for (int p = kMergeBatch; p < np; ++p) M = fmaxf(M, ml[p].x);
    float L = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < kMergeBatch; ++p) {
      if (p < np) {
        const float w = __builtin_amdgcn_exp2f(m_l[p].x - M);
        L = fmaf(w, m_l[p].y, L);
        acc[0] = fmaf(w, o_p[p].x, acc[0]);
        acc[1] = fmaf(w, o_p[p].y, acc[1]);
        acc[2] = fmaf(w, o_p[p].z, acc[2]);
        acc[3] = fmaf(w, o_p[p].w, acc[3]);
      }
    }
    for (int p = kMergeBatch; p < np; ++p) {      // long contexts: the rest in order
      const float2 mp = ml[p];
      const float4 op = o[(size_t)p * (D / 4)];
      const float w = __builtin_amdgcn_exp2f(mp.x - M);
      L = fmaf(w, mp.y, L);
      acc[0] = fmaf(w, op.x, acc[0]);
      acc[1] = fmaf(w, op.y, acc[1]);
      acc[2] = fmaf(w, op.z, acc[2]);
      acc[3] = fmaf(w, op.w, acc[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = acc[i] / L;
  }
  store_out4<OUT_FMT>(out, row * D + 4 * lane, r);
}

template <int OUT_FMT, int D>
static void launch_merge(const float* part_ml, const float* part_o, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, int32_t max_tokens,
                         int32_t part_tokens, int32_t num_parts, int32_t window, int32_t tile,
                         void* out, hipStream_t stream) {
  constexpr int ROWS = kMergeThreads / (D / 4);
  const size_t rows = (size_t)num_seqs * num_q_heads;
  const dim3 grid((unsigned)((rows + ROWS - 1) / ROWS));
  hipLaunchKernelGGL((lse_merge_kernel<OUT_FMT, D>), grid, dim3(kMergeThreads), 0, stream,
                     part_ml, part_o, context_lens, num_seqs, num_q_heads, max_tokens,
                     part_tokens, num_parts, window, tile, out);
}

template <int OUT_FMT>
static hipError_t launch_merge_fmt(const float* part_ml, const float* part_o,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t head_dim, int32_t max_tokens,
                                   int32_t part_tokens, int32_t num_parts, int32_t window,
                                   int32_t tile, void* out, hipStream_t stream) {
  if (head_dim == 128)
    launch_merge<OUT_FMT, 128>(part_ml, part_o, context_lens, num_seqs, num_q_heads, max_tokens,
                               part_tokens, num_parts, window, tile, out, stream);
  else if (head_dim == 64)
    launch_merge<OUT_FMT, 64>(part_ml, part_o, context_lens, num_seqs, num_q_heads, max_tokens,
                              part_tokens, num_parts, window, tile, out, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* part_ml, const float* part_o,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t head_dim, int32_t max_tokens, int32_t part_tokens,
                            int32_t num_parts, int32_t window, int32_t tile, int32_t out_fmt,
                            void* out, hipStream_t stream) {
  if (num_seqs <= 0 || num_q_heads <= 0) return hipSuccess;
  switch (out_fmt) {
    case (int)Fmt::F32:
      return launch_merge_fmt<(int)Fmt::F32>(part_ml, part_o, context_lens, num_seqs,
                                             num_q_heads, head_dim, max_tokens, part_tokens,
                                             num_parts, window, tile, out, stream);
    case (int)Fmt::F16:
      return launch_merge_fmt<(int)Fmt::F16>(part_ml, part_o, context_lens, num_seqs,
                                             num_q_heads, head_dim, max_tokens, part_tokens,
                                             num_parts, window, tile, out, stream);
    case (int)Fmt::BF16:
      return launch_merge_fmt<(int)Fmt::BF16>(part_ml, part_o, context_lens, num_seqs,
                                              num_q_heads, head_dim, max_tokens, part_tokens,
                                              num_parts, window, tile, out, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pa
