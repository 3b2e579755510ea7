// decode_i8.hip -- decode-kernel instances for the i8 cache format.
#include "decode_dispatch.h"

namespace pa {

hipError_t launch_decode_i8(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                            hipStream_t stream) {
  return launch_fmt<Fmt::I8>(p, head_dim, bs, gc, num_seqs, stream);
}

hipError_t launch_mfma_i8(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                           hipStream_t stream) {
  return launch_mfma_fmt<Fmt::I8>(p, head_dim, bs, gc, num_seqs, stream);
}

}  // namespace pa
