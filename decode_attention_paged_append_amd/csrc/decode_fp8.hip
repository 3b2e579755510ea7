// decode_fp8.hip -- decode-kernel instances for the fp8 (E4M3) cache format.
#include "decode_dispatch.h"

namespace pa {

hipError_t launch_decode_fp8(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                             hipStream_t stream) {
  return launch_fmt<Fmt::FP8>(p, head_dim, bs, gc, num_seqs, stream);
}

hipError_t launch_mfma_fp8(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                           hipStream_t stream) {
  return launch_mfma_fmt<Fmt::FP8>(p, head_dim, bs, gc, num_seqs, stream);
}

}  // namespace pa
