// decode_i4.hip -- decode-kernel instances for the int4 cache format: the
// vector-ALU kernel (any head_dim, up to 2 query heads per workgroup) and the
// matrix-core kernel for grouped-query heads at head_dim 128.
#include "decode_dispatch.h"
#include "decode_mfma_i4.h"

namespace pa {

hipError_t launch_decode_i4(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                            hipStream_t stream) {
  return launch_fmt<Fmt::I4>(p, head_dim, bs, gc, num_seqs, stream);
}

// Four heads per workgroup: (head, group) columns; eight or sixteen: one
// head per column.
template <int BS, int GC>
static hipError_t launch_mfma_i4_one(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_parts, (unsigned)(p.num_kv_heads * p.head_chunks),
                  (unsigned)num_seqs);
  if constexpr (GC == 4)
    hipLaunchKernelGGL((decode_mfma_i4_kernel<BS, GC, kDecodeWaves>), grid,
                       dim3(kDecodeWaves * kWave), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_mfma_i4h_kernel<BS, GC, kDecodeWaves>), grid,
                       dim3(kDecodeWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

template <int BS>
static hipError_t launch_mfma_i4_bs(const DecodeParams& p, int gc, int num_seqs,
                                    hipStream_t stream) {
  switch (gc) {
    case 4: return launch_mfma_i4_one<BS, 4>(p, num_seqs, stream);
    case 8: return launch_mfma_i4_one<BS, 8>(p, num_seqs, stream);
    case 16: return launch_mfma_i4_one<BS, 16>(p, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mfma_i4(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                          hipStream_t stream) {
  if (head_dim != 128) return hipErrorInvalidValue;
  if (bs == 16) return launch_mfma_i4_bs<16>(p, gc, num_seqs, stream);
  if (bs == 32) return launch_mfma_i4_bs<32>(p, gc, num_seqs, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
