// device.h -- small device-side helpers shared by the library's kernels
// (internal header, not part of the ABI).  gfx950 / CDNA4, wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
// Running-max start value: finite, so that exp2(m_old - m_new) stays 1 while
// nothing has been seen and becomes 0 at the first real score.
constexpr float kMaxInit = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;

enum class Fmt : int { F32 = 0, F16 = 1, BF16 = 2, I8 = 3, FP8 = 4, I4 = 5 };

// int4 caches: one fp16 scale per group of this many dims of a row.
constexpr int kInt4Group = 32;

// bytes: cache element; q_bytes: query/output element.  Quantized caches
// (int8, fp8 E4M3) hold codes with an fp16 scale per (token, head), int4 one
// per 32 dims, and take fp16 queries; their codes are widened to fp16
// exactly.
template <Fmt F> struct FmtInfo;
template <> struct FmtInfo<Fmt::F32> {
  static constexpr int bytes = 4, q_bytes = 4;
  static constexpr bool quantized = false;
};
template <> struct FmtInfo<Fmt::F16> {
  static constexpr int bytes = 2, q_bytes = 2;
  static constexpr bool quantized = false;
};
template <> struct FmtInfo<Fmt::BF16> {
  static constexpr int bytes = 2, q_bytes = 2;
  static constexpr bool quantized = false;
};
template <> struct FmtInfo<Fmt::I8> {
  static constexpr int bytes = 1, q_bytes = 2;
  static constexpr bool quantized = true;
};
template <> struct FmtInfo<Fmt::FP8> {
  static constexpr int bytes = 1, q_bytes = 2;
  static constexpr bool quantized = true;
};
// int4: two codes per byte (bytes = 0 marks the packed format; rows are D/2
// bytes), a scale per kInt4Group dims.
template <> struct FmtInfo<Fmt::I4> {
  static constexpr int bytes = 0, q_bytes = 2;
  static constexpr bool quantized = true;
};

__device__ __forceinline__ float bits_to_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t float_to_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Reinterpret a 32-bit word as two packed 16-bit floats.  The word is taken
// by value: __builtin_bit_cast applied directly to an ext-vector swizzle such
// as v.y has been seen to read the wrong element, so callers pass v[i].
__device__ __forceinline__ h16x2 as_h2(uint32_t w) { return __builtin_bit_cast(h16x2, w); }
__device__ __forceinline__ bf16x2 as_bf2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// bfloat16 halves of a 32-bit word, as fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return bits_to_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bits_to_float(w & 0xffff0000u); }
// binary16 halves of a 32-bit word, as fp32 (exact).
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)as_h2(w)[0]; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)as_h2(w)[1]; }

// fp32 -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t u = float_to_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t float_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Cross-lane moves inside a row of 16 lanes through DPP (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return bits_to_float((uint32_t)__builtin_amdgcn_update_dpp(
      0, (int)float_to_bits(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

// Sum over aligned groups of N consecutive lanes; every lane of a group ends
// with the same bits (each step adds two equal partial sums in either order).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "");
  if constexpr (N >= 2) x += dpp_mov<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp_mov<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp_mov<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_mov<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_mov<kDppXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_mov<kDppXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_mov<kDppMirror>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Max and sum over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48), with gfx950's row swaps on the vector ALU instead of LDS shuffles.
// v_permlane32_swap of (x, x) leaves lane l holding x[l] and x[l ^ 32] in
// its two results (lanes below 32: own value first; above: the partner's),
// and v_permlane16_swap does the same for l ^ 16 (checked on MI355X for
// every lane), so one swap and one max (or add) combine a pair of halves.
// Every lane ends with the same bits: max is exact, and both lanes of a
// pair add the same two operands in the same order (lower half first).
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(float_to_bits(x), float_to_bits(x), false, false);
  // copied out by value: __builtin_bit_cast of an element of the returned
  // pair read element 0 for both on this compiler
  const uint32_t a0 = a[0], a1 = a[1];
  x = fmaxf(bits_to_float(a0), bits_to_float(a1));
  const auto b = __builtin_amdgcn_permlane16_swap(float_to_bits(x), float_to_bits(x), false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  return fmaxf(bits_to_float(b0), bits_to_float(b1));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(float_to_bits(x), float_to_bits(x), false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  x = bits_to_float(a0) + bits_to_float(a1);
  const auto b = __builtin_amdgcn_permlane16_swap(float_to_bits(x), float_to_bits(x), false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  return bits_to_float(b0) + bits_to_float(b1);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }

// Cache rows are read once per decode step: non-temporal loads stream them
// past the caches instead of evicting lines that are reused (measured: the
// Llama-2-7B attention kernel goes from ~182 us to ~170 us per layer).
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

}  // namespace pa

namespace pa {

// Four OCP E4M3 codes (bytes 0..3 of w) -> binary16 pairs (byte 0, byte 1)
// and (byte 2, byte 3), exactly: every E4M3 value, subnormals included, is a
// binary16 value, and v_cvt_scalef32_pk_f16_fp8 with scale 1 converts each
// code to it (checked on MI355X for all 256 codes in every byte position,
// signed zeros kept).  The NaN code is never stored by the quantizer.
__device__ __forceinline__ void e4m3x4_to_f16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

}  // namespace pa
