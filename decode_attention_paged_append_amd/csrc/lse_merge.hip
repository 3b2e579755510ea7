// lse_merge.hip -- log-sum-exp merge of context partitions (phase 2).
//
// Each partition p of a sequence left (m_p, l_p, o_p): its running max (log2
// units), the sum of 2^(z_i - m_p) and the unnormalized sum of those weights
// times the value rows.  Rescaling every partition to the common max
// M = max_p m_p and dividing by the rescaled total gives exactly the softmax
// of the whole context, because splitting the sum in pieces changes nothing
// in exact arithmetic (the guide's "Flash attention: don't build the giant
// matrix": tiling leaves the math as it is).
#include "kv_ops.h"

namespace pa {

// One workgroup of head_dim threads per (query head, sequence).
template <int OUT_FMT>
__global__ void lse_merge_kernel(const float* __restrict__ part_ml, const float* __restrict__ part_o,
                                 const int32_t* __restrict__ context_lens, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_tokens, int32_t part_tokens,
                                 int32_t num_parts, int32_t window, int32_t tile,
                                 void* __restrict__ out) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  const int ctx = context_lens[s];
  const size_t row = (size_t)s * num_q_heads + h;
  float result;
  if (ctx < 0 || ctx > max_tokens) {
    result = __builtin_nanf("");
  } else if (ctx == 0) {
    result = 0.0f;
  } else {
    // partitions (slots) the sequence used: all up to its end, or for a
    // sliding window those counted from the tile holding the window's first
    // position (the attention kernels' partition_start)
    const int start = window > 0 && ctx > window ? ctx - window : 0;
    const int base = start - start % tile;
    const int np = (ctx - base + part_tokens - 1) / part_tokens;
    const float* ml = part_ml + row * num_parts * 2;
    const float* o = part_o + row * num_parts * head_dim + d;
    float M = -__builtin_inff();
    for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
    float L = 0.0f, acc = 0.0f;
    for (int p = 0; p < np; ++p) {
      const float w = __builtin_amdgcn_exp2f(ml[2 * p] - M);
      L = fmaf(w, ml[2 * p + 1], L);
      acc = fmaf(w, o[(size_t)p * head_dim], acc);
    }
    result = acc / L;
  }
  const size_t idx = row * head_dim + d;
  if constexpr (OUT_FMT == (int)Fmt::F32) {
    ((float*)out)[idx] = result;
  } else if constexpr (OUT_FMT == (int)Fmt::BF16) {
    ((uint16_t*)out)[idx] = float_to_bf16_rne(result);
  } else {
    ((uint16_t*)out)[idx] = float_to_f16_rne(result);
  }
}

hipError_t launch_lse_merge(const float* part_ml, const float* part_o,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t head_dim, int32_t max_tokens, int32_t part_tokens,
                            int32_t num_parts, int32_t window, int32_t tile, int32_t out_fmt,
                            void* out, hipStream_t stream) {
  const dim3 grid((unsigned)num_q_heads, (unsigned)num_seqs);
  const dim3 block((unsigned)head_dim);
  switch (out_fmt) {
    case (int)Fmt::F32:
      hipLaunchKernelGGL(lse_merge_kernel<(int)Fmt::F32>, grid, block, 0, stream, part_ml, part_o,
                         context_lens, num_q_heads, head_dim, max_tokens, part_tokens, num_parts,
                         window, tile, out);
      break;
    case (int)Fmt::F16:
      hipLaunchKernelGGL(lse_merge_kernel<(int)Fmt::F16>, grid, block, 0, stream, part_ml, part_o,
                         context_lens, num_q_heads, head_dim, max_tokens, part_tokens, num_parts,
                         window, tile, out);
      break;
    case (int)Fmt::BF16:
      hipLaunchKernelGGL(lse_merge_kernel<(int)Fmt::BF16>, grid, block, 0, stream, part_ml,
                         part_o, context_lens, num_q_heads, head_dim, max_tokens, part_tokens,
                         num_parts, window, tile, out);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
