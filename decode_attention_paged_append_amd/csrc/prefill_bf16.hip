// prefill_bf16.hip -- prefill-kernel instances for the bf16 cache format.
#include "prefill_dispatch.h"

namespace pa {

hipError_t launch_prefill_bf16(const PrefillParams& p, int head_dim, int bs, PrefillShape shape,
                             int row_tiles, int num_seqs, hipStream_t stream) {
  return launch_prefill_fmt<Fmt::BF16>(p, head_dim, bs, shape, row_tiles, num_seqs, stream);
}

}  // namespace pa
