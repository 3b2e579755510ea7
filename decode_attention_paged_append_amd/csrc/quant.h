// quant.h -- the quantizer of the int8, fp8 (E4M3) and int4 caches, shared by
// the standalone quantizing append and the append fused into the attention
// launches, so that both store the same codes and scales bit for bit
// (internal header, not part of the ABI).
//
// The pages name 8- and 4-bit cache quantization without fixing a scheme
// (KV-cache visualization page, "What the page leaves out"; KV cache notes,
// "Quantized KV cache").  This library's reading, per (token, head) row
// (int4: per group of kInt4Group dims of the row) of fp16 values x:
//   a = max |x| (exact);  s = fp16(a / R) (IEEE fp32 divide, round to nearest
//   even), R = 127 (int8), 448 (fp8) or 7 (int4);
//   int8: code = clamp(rint(x / s), -127, 127);  fp8: code = E4M3(x / s);
//   int4: code = clamp(rint(x / s), -7, 7), stored as the nibble code + 8
//   (dim 2i low, 2i + 1 high in byte i);
//   codes are 0 when s == 0 (and for a NaN input).
#pragma once

#include "device.h"

namespace pa {

// OCP E4M3 code of r: nearest value, ties to even, magnitudes above 448
// saturate, NaN gives 0.  Exponent e = floor(log2 |r|) from the float's bits;
// from 2^-6 up the code is (e + 7) * 8 + (q - 8) with q = rint(|r| * 2^(3-e))
// in [8, 16] (q = 16 carries into the next exponent); below 2^-6 the step is
// 2^-9 and the code is rint(|r| * 2^9), whose 8 is again the smallest normal.
__device__ __forceinline__ uint32_t e4m3_code(float r) {
  if (r != r) return 0u;
  const float a = fminf(fabsf(r), 448.0f);
  const int e = (int)((float_to_bits(a) >> 23) & 0xffu) - 127;
  uint32_t code;
  if (e < -6) {
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    const float q = rintf(a * bits_to_float((uint32_t)(127 + 3 - e) << 23));
    code = (uint32_t)((e + 7) * 8) + (uint32_t)q - 8u;
  }
  return code | (r < 0.0f && code != 0u ? 0x80u : 0u);
}

// Quantizer kinds, in the order of the cache formats.
enum QuantKind : int { kQuantI8 = 0, kQuantFP8 = 1, kQuantI4 = 2 };

template <Fmt F>
constexpr int quant_kind() {
  static_assert(F == Fmt::I8 || F == Fmt::FP8 || F == Fmt::I4, "not a quantized format");
  return F == Fmt::I8 ? kQuantI8 : F == Fmt::FP8 ? kQuantFP8 : kQuantI4;
}

// Quantize the 8 fp16 values a lane holds (dims 8c..8c+7 of a row).  LG
// aligned consecutive lanes share one scale: the row's D/8 lanes (int8, fp8)
// or a 32-dim group's 4 lanes (int4).  Every lane of the wave must call this
// (the absmax is a DPP reduction over the LG lanes); lanes that store nothing
// pass zeros.  Returns the scale's fp16 bits; the codes go to packed[0..1]
// (int8, fp8: 8 bytes) or packed[0] (int4: 8 nibbles).
template <int KIND, int LG>
__device__ __forceinline__ uint16_t quantize_piece(u32x4 x, uint32_t packed[2]) {
  constexpr float R = KIND == kQuantFP8 ? 448.0f : KIND == kQuantI4 ? 7.0f : 127.0f;
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = f16_lo(x[i]);
    f[2 * i + 1] = f16_hi(x[i]);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
  a = group_max<LG>(a);
  const _Float16 s16 = (_Float16)(a / R);
  const float s = (float)s16;
  packed[0] = 0u;
  packed[1] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t code = 0u;
    if constexpr (KIND == kQuantFP8) {
      if (s != 0.0f) code = e4m3_code(f[i] / s);
      packed[i / 4] |= code << (8 * (i % 4));
    } else {
      const float lim = KIND == kQuantI4 ? 7.0f : 127.0f;
      float r = 0.0f;
      if (s != 0.0f) {
        r = rintf(f[i] / s);
        r = r != r ? 0.0f : fminf(fmaxf(r, -lim), lim);
      }
      if constexpr (KIND == kQuantI4) {
        packed[0] |= ((uint32_t)((int32_t)r + 8) & 0xfu) << (4 * i);
      } else {
        packed[i / 4] |= ((uint32_t)(int32_t)r & 0xffu) << (8 * (i % 4));
      }
    }
  }
  return __builtin_bit_cast(uint16_t, s16);
}

// Store lane piece c of a quantized row (row index dst_row of the pool, as
// [NB][Hkv][BS]): its codes, and the scale from the first lane of each LG.
template <int KIND, int D>
__device__ __forceinline__ void store_quant_piece(uint8_t* cache, uint16_t* scales,
                                                  size_t dst_row, int c,
                                                  const uint32_t packed[2], uint16_t sbits) {
  constexpr int LQ = D / 8;  // lanes per row
  if constexpr (KIND == kQuantI4) {
    constexpr int LG = kInt4Group / 8;
    ((uint32_t*)cache)[dst_row * LQ + c] = packed[0];  // D/2 bytes per row
    if (c % LG == 0) scales[dst_row * (D / kInt4Group) + c / LG] = sbits;
  } else {
    ((u32x2*)cache)[dst_row * LQ + c] = u32x2{packed[0], packed[1]};
    if (c == 0) scales[dst_row] = sbits;
  }
}

}  // namespace pa
