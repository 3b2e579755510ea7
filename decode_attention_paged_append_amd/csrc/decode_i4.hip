// decode_i4.hip -- decode-kernel instances for the int4 cache format (vector
// ALU kernel only; the plan never routes int4 to the matrix cores).
#include "decode_dispatch.h"

namespace pa {

hipError_t launch_decode_i4(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                            hipStream_t stream) {
  return launch_fmt<Fmt::I4>(p, head_dim, bs, gc, num_seqs, stream);
}

}  // namespace pa
