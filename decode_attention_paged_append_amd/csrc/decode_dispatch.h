// decode_dispatch.h -- runtime (head_dim, block size, head chunk) -> template
// instance of the decode kernel for one cache format (internal header).
#pragma once

#include "decode_mfma.h"

namespace pa {

// LDS reserved (unused) at launch to hold a CU to fewer resident workgroups.
// The plan gives the int8 vector-ALU kernel at one head per workgroup and
// head_dim 128 one round of workgroups, four per CU, but its registers (93
// VGPRs) let five reside, and launches came out either at 87.5 or at 90.5
// us on Llama-2-7B int8 (16 x 4096), as if the dispatcher at times put five
// on some CUs and three on others.  Reserving LDS so that only four fit, the
// launch took 87.4-87.6 us in three alternations on MI355X (uncapped: 87.5
// once, 90.5-90.6 twice).  The 16-bit instances were level under the same
// cap and keep their occupancy.
template <Fmt F, int D, int GC>
constexpr unsigned occupancy_lds() {
  return F == Fmt::I8 && GC == 1 && D == 128 ? 32768u : 0u;
}

template <Fmt F, int D, int BS, int GC>
static hipError_t launch_one(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_parts, (unsigned)(p.num_kv_heads * p.head_chunks),
                  (unsigned)num_seqs);
  constexpr unsigned lds = occupancy_lds<F, D, GC>();
  hipLaunchKernelGGL((decode_partition_kernel<F, D, BS, GC, kDecodeWaves>), grid,
                     dim3(kDecodeWaves * kWave), lds, stream, p);
  return hipGetLastError();
}

// Heads per workgroup of the vector-ALU kernel: up to 8, int4 up to 2 (its
// lanes hold 32 values per head, twice the others).
template <Fmt F>
constexpr int max_heads_per_workgroup() { return F == Fmt::I4 ? 2 : 8; }

template <Fmt F, int D, int BS>
static hipError_t launch_gc(const DecodeParams& p, int gc, int num_seqs, hipStream_t stream) {
  if (gc > max_heads_per_workgroup<F>()) return hipErrorInvalidValue;
  switch (gc) {
    case 1: return launch_one<F, D, BS, 1>(p, num_seqs, stream);
    case 2: return launch_one<F, D, BS, 2>(p, num_seqs, stream);
    case 4:
      if constexpr (max_heads_per_workgroup<F>() >= 4)
        return launch_one<F, D, BS, 4>(p, num_seqs, stream);
      return hipErrorInvalidValue;
    case 8:
      if constexpr (max_heads_per_workgroup<F>() >= 8)
        return launch_one<F, D, BS, 8>(p, num_seqs, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <Fmt F, int D>
static hipError_t launch_bs(const DecodeParams& p, int bs, int gc, int num_seqs,
                            hipStream_t stream) {
  switch (bs) {
    case 4: return launch_gc<F, D, 4>(p, gc, num_seqs, stream);
    case 8: return launch_gc<F, D, 8>(p, gc, num_seqs, stream);
    case 16: return launch_gc<F, D, 16>(p, gc, num_seqs, stream);
    case 32: return launch_gc<F, D, 32>(p, gc, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

template <Fmt F>
static hipError_t launch_fmt(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                             hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_bs<F, 64>(p, bs, gc, num_seqs, stream);
    case 128: return launch_bs<F, 128>(p, bs, gc, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---- matrix-core kernel for grouped-query heads (fp16 / bf16 / int8 / fp8
// caches, int4 at head_dim 128; block size 16 or 32, 4..16 query heads per
// workgroup)
template <Fmt F, int D, int BS, int GC>
static hipError_t launch_mfma_one(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_parts, (unsigned)(p.num_kv_heads * p.head_chunks),
                  (unsigned)(p.pair ? (num_seqs + 1) / 2 : num_seqs));
  hipLaunchKernelGGL((decode_mfma_kernel<F, D, BS, GC, kDecodeWaves>), grid,
                     dim3(kDecodeWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

template <Fmt F, int D, int BS>
static hipError_t launch_mfma_gc(const DecodeParams& p, int gc, int num_seqs, hipStream_t stream) {
  switch (gc) {
    case 4: return launch_mfma_one<F, D, BS, 4>(p, num_seqs, stream);
    case 8: return launch_mfma_one<F, D, BS, 8>(p, num_seqs, stream);
    case 16: return launch_mfma_one<F, D, BS, 16>(p, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

template <Fmt F>
static hipError_t launch_mfma_fmt(const DecodeParams& p, int head_dim, int bs, int gc,
                                  int num_seqs, hipStream_t stream) {
  if (head_dim == 128 && bs == 16) return launch_mfma_gc<F, 128, 16>(p, gc, num_seqs, stream);
  if (head_dim == 128 && bs == 32) return launch_mfma_gc<F, 128, 32>(p, gc, num_seqs, stream);
  if (head_dim == 64 && bs == 16) return launch_mfma_gc<F, 64, 16>(p, gc, num_seqs, stream);
  if (head_dim == 64 && bs == 32) return launch_mfma_gc<F, 64, 32>(p, gc, num_seqs, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_mfma_f16(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                           hipStream_t stream);
hipError_t launch_mfma_bf16(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                            hipStream_t stream);
hipError_t launch_mfma_i8(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                          hipStream_t stream);
hipError_t launch_mfma_fp8(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                           hipStream_t stream);
hipError_t launch_mfma_i4(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                          hipStream_t stream);  // head_dim 128, 4 heads per workgroup

hipError_t launch_decode_f32(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                             hipStream_t stream);
hipError_t launch_decode_f16(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                             hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                              hipStream_t stream);
hipError_t launch_decode_i8(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                            hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                             hipStream_t stream);
hipError_t launch_decode_i4(const DecodeParams& p, int head_dim, int bs, int gc, int num_seqs,
                            hipStream_t stream);

}  // namespace pa
