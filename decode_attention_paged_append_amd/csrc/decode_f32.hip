// decode_f32.hip -- decode-kernel instances for the f32 cache format.
#include "decode_dispatch.h"

namespace pa {

hipError_t launch_decode_f32(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                            hipStream_t stream) {
  return launch_fmt<Fmt::F32>(p, head_dim, bs, gc, num_seqs, stream);
}

}  // namespace pa
