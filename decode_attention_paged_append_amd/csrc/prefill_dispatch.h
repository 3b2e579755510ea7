// prefill_dispatch.h -- runtime (head_dim, block size, rows per wave) ->
// template instance of the prefill kernel (internal).
#pragma once

#include "prefill_mfma.h"

namespace pa {

// Launch shapes.  Long chunks at head_dim 128: 8 waves x 3 row groups (384
// query rows per workgroup; two waves per SIMD fit in the 256 registers), so
// each K/V fragment read from LDS serves three row groups; from 256 to 767
// rows 8 waves x 2 row groups, which leaves less of a last tile idle.  At
// head_dim 64: 4 waves x 4 row groups.  Short chunks: 4 waves x 1 row group.
struct PrefillShape {
  int nr, nw;
  int rows() const { return nr * nw * 16; }
};
inline PrefillShape prefill_shape(int head_dim, int64_t rows) {
  if (rows < 256) return {1, 4};
  if (head_dim != 128) return {4, 4};
  return rows < 768 ? PrefillShape{2, 8} : PrefillShape{3, 8};
}

template <Fmt F, int D, int BS, int NR, int NW>
static hipError_t launch_prefill_one(const PrefillParams& p, int row_tiles, int num_seqs,
                                     hipStream_t stream) {
  hipLaunchKernelGGL((prefill_mfma_kernel<F, D, BS, NR, NW>),
                     dim3(p.num_kv_heads, num_seqs, row_tiles), dim3(NW * kWave), 0, stream, p);
  return hipGetLastError();
}

template <Fmt F, int D, int NR, int NW>
static hipError_t launch_prefill_bs(const PrefillParams& p, int bs, int row_tiles, int num_seqs,
                                    hipStream_t stream) {
  switch (bs) {
    case 4: return launch_prefill_one<F, D, 4, NR, NW>(p, row_tiles, num_seqs, stream);
    case 8: return launch_prefill_one<F, D, 8, NR, NW>(p, row_tiles, num_seqs, stream);
    case 16: return launch_prefill_one<F, D, 16, NR, NW>(p, row_tiles, num_seqs, stream);
    case 32: return launch_prefill_one<F, D, 32, NR, NW>(p, row_tiles, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

template <Fmt F>
static hipError_t launch_prefill_fmt(const PrefillParams& p, int head_dim, int bs,
                                     PrefillShape shape, int row_tiles, int num_seqs,
                                     hipStream_t stream) {
  if (head_dim == 64)
    return shape.nr == 4 ? launch_prefill_bs<F, 64, 4, 4>(p, bs, row_tiles, num_seqs, stream)
                         : launch_prefill_bs<F, 64, 1, 4>(p, bs, row_tiles, num_seqs, stream);
  if (head_dim == 128)
    return shape.nr == 3   ? launch_prefill_bs<F, 128, 3, 8>(p, bs, row_tiles, num_seqs, stream)
           : shape.nr == 2 ? launch_prefill_bs<F, 128, 2, 8>(p, bs, row_tiles, num_seqs, stream)
                           : launch_prefill_bs<F, 128, 1, 4>(p, bs, row_tiles, num_seqs, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_f16(const PrefillParams& p, int head_dim, int bs, PrefillShape shape,
                              int row_tiles, int num_seqs, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillParams& p, int head_dim, int bs, PrefillShape shape,
                               int row_tiles, int num_seqs, hipStream_t stream);

}  // namespace pa
