/*
 * oracle.c -- plain, slow, CPU reference for paged KV-cache decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * Sources (the three pages the method is taken from):
 *   [guide]  jovanaeducation.com/guides/l-is-2
 *   [notes]  "KV cache: the engine behind fast LLM inference"
 *            (curiosity-9m6.pages.dev/notes/0043)
 *   [viz]    the KV-cache visualization page
 *            (cuuduongthancong.com/~galles/visualization/KVCache.html)
 *
 * What is computed, and where it is defined:
 *   - attention for one query: softmax(q . K^T * scale) . V over every cached
 *     row of the sequence ([notes] "Concept"; [notes] "What happens at each
 *     decoding step", step 3).  Written out from that definition in fp64.
 *   - un-paging through a block table: a sequence's rows live in fixed-size
 *     blocks of one shared pool, listed in order by a per-sequence block table
 *     ([viz] "PagedAttention: the cache in blocks").
 *   - prefill: every prompt token's query attends causally over the cache
 *     (positions up to its own; [viz] "The idea", "Without vs with the
 *     cache").
 *   - append: the new token's K and V rows are stored into the cache
 *     ([notes] step 4; [guide] "How the cache turns the loop cheap").
 *   - fp8 (E4M3) cache: the same scheme with 8-bit floating-point codes
 *     ([viz] "What the page leaves out" names 8- and 4-bit caches).  PARITY
 *     UNPINNED for the exact codes, as for int8.
 *   - int4 cache: signed 4-bit codes with a scale per group of 32 dims, two
 *     codes per byte (the 4-bit half of [viz]'s "8-bit or 4-bit").  PARITY
 *     UNPINNED for the exact codes.
 *   - int8 cache ([notes] "How serving systems tame the cost", "Quantized KV
 *     cache"): the pages name the format only; the symmetric per-(token, head)
 *     absmax quantizer below is this project's reading.  PARITY UNPINNED by
 *     the pages for the quantizer's exact codes: it is pinned only by its own
 *     error bound and by special cases (all-zero row, exact dequantization).
 *
 * Cache layout (part of the library's ABI, so the oracle reads the same one):
 *   k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim]
 *   int8 scales      : [num_blocks][num_kv_heads][block_size]   (fp16 bits)
 *   block_tables     : int32 [num_seqs][max_blocks]
 *   context_lens     : int32 [num_seqs], counting the token just appended
 *   q                : [num_seqs][num_q_heads][head_dim]
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Every function returns 0 on success and a negative code on bad input.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_I8 = 3, OR_FP8 = 4, OR_I4 = 5 };

/* int4 caches: one fp16 scale per group of this many dims of a row. */
enum { OR_I4_GROUP = 32 };

enum {
  OR_OK = 0,
  OR_BAD_ARG = -1,
  OR_BAD_SLOT = -2,
  OR_DUP_SLOT = -3,
  OR_BAD_CTX = -4,
  OR_BAD_BLOCK = -5,
  OR_NO_MEM = -6
};

/* ------------------------------------------------------------------------ */
/* Number formats, decoded from their bit patterns (IEEE binary16, bfloat16). */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (expo == 0)
    v = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
  else if (expo == 31)
    v = frac ? NAN : INFINITY;
  else
    v = ldexp((double)(frac | 0x400), expo - 25); /* 1.frac * 2^(expo-15) */
  return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits
 * (bias 7), 3 fraction bits.  Exponent field 0 holds the subnormals
 * frac/8 * 2^-6; S.1111.111 is NaN; there are no infinities, so the largest
 * finite magnitude is 1.75 * 2^8 = 448. */
double oracle_fp8_e4m3_to_double(uint8_t b) {
  int sign = b >> 7, expo = (b >> 3) & 15, frac = b & 7;
  if (expo == 15 && frac == 7) return NAN;
  double v = expo == 0 ? ldexp((double)frac, -9) : ldexp(8.0 + frac, expo - 10);
  return sign ? -v : v;
}

/* The E4M3 code nearest to x, found by trying every finite code; a tie goes
 * to the code with an even last bit.  Magnitudes above 448 give +-448
 * (saturation); NaN gives 0. */
uint8_t oracle_double_to_fp8_e4m3(double x) {
  if (x != x) return 0;
  double a = fabs(x);
  int best = 0;
  double best_err = a;  /* code 0 is the value 0 */
  for (int c = 1; c < 127; ++c) {
    double err = fabs(oracle_fp8_e4m3_to_double((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(best | (x < 0 && best != 0 ? 0x80 : 0));
}

/* Round a finite non-negative value to the nearest binary16 value, ties to
 * even, and return its bit pattern.  Values at or above 65520 become +inf. */
uint16_t oracle_double_to_f16_bits(double a) {
  if (a != a) return 0x7e00;
  int neg = a < 0;
  if (neg) a = -a;
  uint16_t out;
  if (a == 0) {
    out = 0;
  } else if (a >= 65520.0) {
    out = 0x7c00;
  } else {
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): leading bit has weight 2^(e-1) */
    int lead = e - 1;
    if (lead < -14) lead = -14;           /* subnormal range shares 2^-14's quantum */
    double quantum = ldexp(1.0, lead - 10); /* 10 fraction bits */
    double n = nearbyint(a / quantum);      /* exact quotient, rounded half-even */
    double r = n * quantum;
    if (r >= 65520.0) {
      out = 0x7c00;
    } else if (r < ldexp(1.0, -14)) {
      out = (uint16_t)(r / ldexp(1.0, -24)); /* subnormal fraction */
    } else {
      int e2;
      double f2 = frexp(r, &e2);            /* r = f2 * 2^e2 */
      int expo = e2 - 1 + 15;
      int frac = (int)(ldexp(f2, 11) - 1024.0);
      out = (uint16_t)((expo << 10) | frac);
    }
  }
  return (uint16_t)(out | (neg ? 0x8000 : 0));
}

static size_t elem_bytes(int dtype) {
  switch (dtype) {
    case OR_F32: return 4;
    case OR_F16: return 2;
    case OR_BF16: return 2;
    case OR_I8: return 1;
    case OR_FP8: return 1;
    case OR_I4: return 1; /* two codes per byte: rows are head_dim / 2 bytes */
    default: return 0;
  }
}

/* Value of element idx of an array of the given format (int8: the raw code). */
static double load_elem(const void* base, int dtype, size_t idx) {
  switch (dtype) {
    case OR_F32: {
      float f;
      memcpy(&f, (const char*)base + 4 * idx, 4);
      return (double)f;
    }
    case OR_F16: {
      uint16_t h;
      memcpy(&h, (const char*)base + 2 * idx, 2);
      return oracle_f16_to_double(h);
    }
    case OR_BF16: {
      uint16_t h;
      memcpy(&h, (const char*)base + 2 * idx, 2);
      return oracle_bf16_to_double(h);
    }
    case OR_I8:
      return (double)((const int8_t*)base)[idx];
    case OR_FP8:
      return oracle_fp8_e4m3_to_double(((const uint8_t*)base)[idx]);
    case OR_I4: {
      /* element 2i in the low nibble of byte i, 2i+1 in the high nibble,
       * stored as code + 8 */
      uint8_t byte = ((const uint8_t*)base)[idx / 2];
      int nib = idx % 2 ? byte >> 4 : byte & 15;
      return (double)(nib - 8);
    }
    default:
      return NAN;
  }
}

/* ------------------------------------------------------------------------ */
/* Slot of a token position: the block table lists the sequence's blocks in
 * order, each holding block_size consecutive positions ([viz] "PagedAttention:
 * the cache in blocks").  slot = block * block_size + offset.                */
int oracle_slot_mapping(const int32_t* block_tables, int32_t max_blocks,
                        const int32_t* token_seq, const int32_t* token_pos,
                        int64_t num_tokens, int32_t block_size,
                        int64_t* slots) {
  if (num_tokens < 0 || block_size <= 0 || max_blocks <= 0) return OR_BAD_ARG;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int32_t pos = token_pos[t];
    if (pos < 0 || pos >= max_blocks * block_size) return OR_BAD_CTX;
    int32_t block = block_tables[(int64_t)token_seq[t] * max_blocks + pos / block_size];
    slots[t] = (int64_t)block * block_size + pos % block_size;
  }
  return OR_OK;
}

/* Decode step: the appended token sits at position context_len - 1 (the
 * length already counts it).  A sequence with length 0 gets slot -1. */
int oracle_decode_slot_mapping(const int32_t* block_tables, int32_t max_blocks,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t block_size, int64_t* slots) {
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t ctx = context_lens[s];
    if (ctx < 0 || ctx > max_blocks * block_size) return OR_BAD_CTX;
    if (ctx == 0) {
      slots[s] = -1;
      continue;
    }
    int32_t pos = ctx - 1;
    int32_t block = block_tables[(int64_t)s * max_blocks + pos / block_size];
    slots[s] = (int64_t)block * block_size + pos % block_size;
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Append: store token t's row for every KV head at its slot.  The copy is of
 * the element bytes, so it is exact.  Negative slots are padding and are
 * skipped; a slot outside the pool, or used twice, is an error (checked
 * before anything is written).                                               */
int oracle_kv_append(const void* k_new, const void* v_new, const int64_t* slots,
                     int64_t num_tokens, void* k_cache, void* v_cache,
                     int32_t num_blocks, int32_t num_kv_heads,
                     int32_t block_size, int32_t head_dim, int32_t dtype) {
  size_t eb = elem_bytes(dtype);
  if (!eb || num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 ||
      block_size <= 0 || head_dim <= 0)
    return OR_BAD_ARG;
  int64_t pool_slots = (int64_t)num_blocks * block_size;
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] >= pool_slots) return OR_BAD_SLOT;
    if (slots[t] < 0) continue;
    for (int64_t u = 0; u < t; ++u)
      if (slots[u] == slots[t]) return OR_DUP_SLOT;
  }
  size_t row = (size_t)head_dim * eb;
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] < 0) continue;
    int64_t block = slots[t] / block_size, off = slots[t] % block_size;
    for (int32_t h = 0; h < num_kv_heads; ++h) {
      size_t src = ((size_t)t * num_kv_heads + h) * row;
      size_t dst = (((size_t)block * num_kv_heads + h) * block_size + off) * row;
      memcpy((char*)k_cache + dst, (const char*)k_new + src, row);
      memcpy((char*)v_cache + dst, (const char*)v_new + src, row);
    }
  }
  return OR_OK;
}

/* int8 quantizer for one row of fp16 values (this project's reading of the
 * "Quantized KV cache" paragraph of [notes]; see the file header):
 *   a = max |x|                         (exact)
 *   s = binary16 nearest to fp32(a / 127)   (fp32 IEEE division, then RNE)
 *   q = clamp(round_half_even(fp32(x / s)), -127, 127), q = 0 when s == 0
 *   (and for a NaN input),
 * so that q * s reproduces x to within half a step.  All divisions are IEEE
 * binary32, which the GPU reproduces exactly.                               */
void oracle_quantize_row_int8(const uint16_t* x_f16, int32_t n, int8_t* q,
                              uint16_t* scale_f16) {
  float a = 0.0f;
  for (int32_t d = 0; d < n; ++d) {
    float x = (float)oracle_f16_to_double(x_f16[d]);
    float ax = fabsf(x);
    if (ax > a) a = ax;
  }
  volatile float ratio = a / 127.0f; /* binary32 quotient */
  uint16_t sbits = oracle_double_to_f16_bits((double)ratio);
  float s = (float)oracle_f16_to_double(sbits);
  *scale_f16 = sbits;
  for (int32_t d = 0; d < n; ++d) {
    if (s == 0.0f) {
      q[d] = 0;
      continue;
    }
    float x = (float)oracle_f16_to_double(x_f16[d]);
    volatile float r = x / s; /* binary32 quotient */
    float c = rintf(r);       /* default rounding mode: half to even */
    if (c != c) c = 0.0f;     /* a NaN input encodes as 0 */
    if (c > 127.0f) c = 127.0f;
    if (c < -127.0f) c = -127.0f;
    q[d] = (int8_t)c;
  }
}

/* Append into an int8 cache: quantize each (token, head) row, then store the
 * codes and the scale at the token's slot. */
int oracle_kv_append_int8(const uint16_t* k_new, const uint16_t* v_new,
                          const int64_t* slots, int64_t num_tokens,
                          int8_t* k_cache, int8_t* v_cache, uint16_t* k_scale,
                          uint16_t* v_scale, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t block_size,
                          int32_t head_dim) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 ||
      block_size <= 0 || head_dim <= 0)
    return OR_BAD_ARG;
  int64_t pool_slots = (int64_t)num_blocks * block_size;
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] >= pool_slots) return OR_BAD_SLOT;
    if (slots[t] < 0) continue;
    for (int64_t u = 0; u < t; ++u)
      if (slots[u] == slots[t]) return OR_DUP_SLOT;
  }
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] < 0) continue;
    int64_t block = slots[t] / block_size, off = slots[t] % block_size;
    for (int32_t h = 0; h < num_kv_heads; ++h) {
      size_t src = ((size_t)t * num_kv_heads + h) * head_dim;
      size_t srow = ((size_t)block * num_kv_heads + h) * block_size + off;
      oracle_quantize_row_int8(k_new + src, head_dim, k_cache + srow * head_dim,
                               &k_scale[srow]);
      oracle_quantize_row_int8(v_new + src, head_dim, v_cache + srow * head_dim,
                               &v_scale[srow]);
    }
  }
  return OR_OK;
}

/* fp8 quantizer for one row of fp16 values: the int8 scheme above with E4M3
 * codes ("8-bit or 4-bit" cache quantization: [viz] "What the page leaves
 * out"; the format and the per-(token, head) scale are this project's
 * reading, PARITY UNPINNED like the int8 codes):
 *   a = max |x|                            (exact)
 *   s = binary16 nearest to fp32(a / 448)  (fp32 IEEE division, then RNE)
 *   code = E4M3 nearest to fp32(x / s), ties to even, saturating at +-448;
 *   code = 0 when s == 0 (and for a NaN input).                              */
void oracle_quantize_row_fp8(const uint16_t* x_f16, int32_t n, uint8_t* q,
                             uint16_t* scale_f16) {
  float a = 0.0f;
  for (int32_t d = 0; d < n; ++d) {
    float ax = fabsf((float)oracle_f16_to_double(x_f16[d]));
    if (ax > a) a = ax;
  }
  volatile float ratio = a / 448.0f; /* binary32 quotient */
  uint16_t sbits = oracle_double_to_f16_bits((double)ratio);
  float s = (float)oracle_f16_to_double(sbits);
  *scale_f16 = sbits;
  for (int32_t d = 0; d < n; ++d) {
    if (s == 0.0f) {
      q[d] = 0;
      continue;
    }
    volatile float r = (float)oracle_f16_to_double(x_f16[d]) / s; /* binary32 */
    q[d] = oracle_double_to_fp8_e4m3((double)r);
  }
}

/* Append into an fp8 cache: quantize each (token, head) row, then store the
 * codes and the scale at the token's slot. */
int oracle_kv_append_fp8(const uint16_t* k_new, const uint16_t* v_new,
                         const int64_t* slots, int64_t num_tokens,
                         uint8_t* k_cache, uint8_t* v_cache, uint16_t* k_scale,
                         uint16_t* v_scale, int32_t num_blocks,
                         int32_t num_kv_heads, int32_t block_size,
                         int32_t head_dim) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 ||
      block_size <= 0 || head_dim <= 0)
    return OR_BAD_ARG;
  int64_t pool_slots = (int64_t)num_blocks * block_size;
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] >= pool_slots) return OR_BAD_SLOT;
    if (slots[t] < 0) continue;
    for (int64_t u = 0; u < t; ++u)
      if (slots[u] == slots[t]) return OR_DUP_SLOT;
  }
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] < 0) continue;
    int64_t block = slots[t] / block_size, off = slots[t] % block_size;
    for (int32_t h = 0; h < num_kv_heads; ++h) {
      size_t src = ((size_t)t * num_kv_heads + h) * head_dim;
      size_t srow = ((size_t)block * num_kv_heads + h) * block_size + off;
      oracle_quantize_row_fp8(k_new + src, head_dim, k_cache + srow * head_dim,
                              &k_scale[srow]);
      oracle_quantize_row_fp8(v_new + src, head_dim, v_cache + srow * head_dim,
                              &v_scale[srow]);
    }
  }
  return OR_OK;
}

/* int4 quantizer for one row of fp16 values ("8-bit or 4-bit" cache
 * quantization: [viz] "What the page leaves out"; groups and scales are this
 * project's reading, PARITY UNPINNED like the int8 codes).  For each group of
 * OR_I4_GROUP consecutive dims:
 *   a = max |x| over the group         (exact)
 *   s = binary16 nearest to fp32(a / 7)  (fp32 IEEE division, then RNE)
 *   q = clamp(round_half_even(fp32(x / s)), -7, 7), 0 when s == 0 or x is NaN,
 * stored as the nibble q + 8: dim 2i in the low half of byte i, dim 2i + 1
 * in the high half.  scales receives n / OR_I4_GROUP binary16 values.      */
void oracle_quantize_row_int4(const uint16_t* x_f16, int32_t n, uint8_t* packed,
                              uint16_t* scales_f16) {
  for (int32_t i = 0; i < n / 2; ++i) packed[i] = 0;
  for (int32_t g = 0; g < n / OR_I4_GROUP; ++g) {
    const uint16_t* x = x_f16 + g * OR_I4_GROUP;
    float a = 0.0f;
    for (int32_t d = 0; d < OR_I4_GROUP; ++d) {
      float ax = fabsf((float)oracle_f16_to_double(x[d]));
      if (ax > a) a = ax;
    }
    volatile float ratio = a / 7.0f; /* binary32 quotient */
    uint16_t sbits = oracle_double_to_f16_bits((double)ratio);
    float s = (float)oracle_f16_to_double(sbits);
    scales_f16[g] = sbits;
    for (int32_t d = 0; d < OR_I4_GROUP; ++d) {
      float c = 0.0f;
      if (s != 0.0f) {
        volatile float r = (float)oracle_f16_to_double(x[d]) / s; /* binary32 */
        c = rintf(r);
        if (c != c) c = 0.0f;
        if (c > 7.0f) c = 7.0f;
        if (c < -7.0f) c = -7.0f;
      }
      int32_t e = g * OR_I4_GROUP + d;
      uint8_t nib = (uint8_t)((int)c + 8);
      packed[e / 2] |= (uint8_t)(e % 2 ? nib << 4 : nib);
    }
  }
}

/* Append into an int4 cache: quantize each (token, head) row, then store the
 * packed codes and its group scales at the token's slot. */
int oracle_kv_append_int4(const uint16_t* k_new, const uint16_t* v_new,
                          const int64_t* slots, int64_t num_tokens,
                          uint8_t* k_cache, uint8_t* v_cache, uint16_t* k_scale,
                          uint16_t* v_scale, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t block_size,
                          int32_t head_dim) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 ||
      block_size <= 0 || head_dim <= 0 || head_dim % OR_I4_GROUP)
    return OR_BAD_ARG;
  int64_t pool_slots = (int64_t)num_blocks * block_size;
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] >= pool_slots) return OR_BAD_SLOT;
    if (slots[t] < 0) continue;
    for (int64_t u = 0; u < t; ++u)
      if (slots[u] == slots[t]) return OR_DUP_SLOT;
  }
  int32_t groups = head_dim / OR_I4_GROUP;
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] < 0) continue;
    int64_t block = slots[t] / block_size, off = slots[t] % block_size;
    for (int32_t h = 0; h < num_kv_heads; ++h) {
      size_t src = ((size_t)t * num_kv_heads + h) * head_dim;
      size_t srow = ((size_t)block * num_kv_heads + h) * block_size + off;
      oracle_quantize_row_int4(k_new + src, head_dim, k_cache + srow * (head_dim / 2),
                               &k_scale[srow * groups]);
      oracle_quantize_row_int4(v_new + src, head_dim, v_cache + srow * (head_dim / 2),
                               &v_scale[srow * groups]);
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention of one query over n cached rows, straight from the definition
 * softmax(q . K^T * scale) . V ([notes] "Concept"), in fp64:
 *   z_i = scale * sum_d q_d K_id
 *   w_i = exp(z_i - max z) / sum_j exp(z_j - max z)
 *   out_d = sum_i w_i V_id
 * Subtracting max z leaves every w_i unchanged; it only keeps exp finite.
 * n == 0 gives a zero output.  weights (optional) receives w.              */
int oracle_attention_dense(const double* q, const double* K, const double* V,
                           int64_t n, int32_t head_dim, double scale,
                           double* out, double* weights) {
  for (int32_t d = 0; d < head_dim; ++d) out[d] = 0.0;
  if (n <= 0) return OR_OK;
  double* z = (double*)malloc(sizeof(double) * (size_t)n);
  if (!z) return OR_NO_MEM;
  for (int64_t i = 0; i < n; ++i) {
    double dot = 0.0;
    for (int32_t d = 0; d < head_dim; ++d) dot += q[d] * K[i * head_dim + d];
    z[i] = scale * dot;
  }
  double m = z[0];
  for (int64_t i = 1; i < n; ++i)
    if (z[i] > m) m = z[i];
  double total = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    z[i] = exp(z[i] - m);
    total += z[i];
  }
  for (int64_t i = 0; i < n; ++i) {
    double w = z[i] / total;
    if (weights) weights[i] = w;
    for (int32_t d = 0; d < head_dim; ++d) out[d] += w * V[i * head_dim + d];
  }
  free(z);
  return OR_OK;
}

/* Un-page one sequence's rows for one KV head into dense [ctx][head_dim]
 * fp64 arrays: position i lives in block block_table[i / block_size] at
 * offset i % block_size ([viz] "PagedAttention: the cache in blocks").
 * int8 rows are dequantized as code * scale (exact in fp64).              */
static int unpage(const void* k_cache, const void* v_cache,
                  const uint16_t* k_scale, const uint16_t* v_scale, int dtype,
                  const int32_t* table, int32_t ctx, int32_t kvh,
                  int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                  int32_t head_dim, double* K, double* V) {
  for (int32_t i = 0; i < ctx; ++i) {
    int32_t block = table[i / block_size];
    if (block < 0 || block >= num_blocks) return OR_BAD_BLOCK;
    size_t row = ((size_t)block * num_kv_heads + kvh) * block_size + i % block_size;
    double sk = 1.0, sv = 1.0;
    if (dtype == OR_I8 || dtype == OR_FP8) {
      sk = oracle_f16_to_double(k_scale[row]);
      sv = oracle_f16_to_double(v_scale[row]);
    }
    for (int32_t d = 0; d < head_dim; ++d) {
      if (dtype == OR_I4) { /* a scale per group of OR_I4_GROUP dims */
        size_t g = row * (head_dim / OR_I4_GROUP) + d / OR_I4_GROUP;
        sk = oracle_f16_to_double(k_scale[g]);
        sv = oracle_f16_to_double(v_scale[g]);
      }
      K[(size_t)i * head_dim + d] = load_elem(k_cache, dtype, row * head_dim + d) * sk;
      V[(size_t)i * head_dim + d] = load_elem(v_cache, dtype, row * head_dim + d) * sv;
    }
  }
  return OR_OK;
}

/* Paged decode attention: for every requested (sequence, query head) pair,
 * un-page the sequence's K and V rows of the head's KV head and apply the
 * dense definition above.  q has dtype q_dtype (the int8 cache takes fp16
 * queries).  pairs: optional list of n_pairs (seq, head) pairs; when NULL
 * every pair is computed in order s-major.  out: fp64 [n_pairs][head_dim].
 * Work is split over threads by pair only; each pair's arithmetic is the
 * same sequential loop whatever the thread count.                         */
int oracle_paged_decode_attention(
    const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
    const uint16_t* k_scale, const uint16_t* v_scale, int32_t cache_dtype,
    const int32_t* block_tables, int32_t max_blocks,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t num_blocks, int32_t block_size,
    int32_t head_dim, double scale, const int32_t* pairs, int64_t n_pairs,
    double* out, int32_t num_threads) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || block_size <= 0 || head_dim <= 0 ||
      max_blocks <= 0 || !elem_bytes(cache_dtype) || !elem_bytes(q_dtype))
    return OR_BAD_ARG;
  if ((cache_dtype == OR_I8 || cache_dtype == OR_FP8 || cache_dtype == OR_I4) &&
      (!k_scale || !v_scale))
    return OR_BAD_ARG;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (context_lens[s] < 0 || context_lens[s] > max_blocks * block_size)
      return OR_BAD_CTX;
  if (!pairs) n_pairs = (int64_t)num_seqs * num_q_heads;
  for (int64_t p = 0; pairs && p < n_pairs; ++p)
    if (pairs[2 * p] < 0 || pairs[2 * p] >= num_seqs || pairs[2 * p + 1] < 0 ||
        pairs[2 * p + 1] >= num_q_heads)
      return OR_BAD_ARG;
  int32_t group = num_q_heads / num_kv_heads;
  int status = OR_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t p = 0; p < n_pairs; ++p) {
    int32_t s = pairs ? pairs[2 * p] : (int32_t)(p / num_q_heads);
    int32_t h = pairs ? pairs[2 * p + 1] : (int32_t)(p % num_q_heads);
    int32_t ctx = context_lens[s];
    int32_t kvh = h / group;
    size_t n = (size_t)(ctx > 0 ? ctx : 1) * head_dim;
    double* K = (double*)malloc(sizeof(double) * n);
    double* V = (double*)malloc(sizeof(double) * n);
    double* qv = (double*)malloc(sizeof(double) * head_dim);
    int st = (K && V && qv) ? OR_OK : OR_NO_MEM;
    if (st == OR_OK)
      st = unpage(k_cache, v_cache, k_scale, v_scale, cache_dtype,
                  block_tables + (size_t)s * max_blocks, ctx, kvh, num_blocks,
                  num_kv_heads, block_size, head_dim, K, V);
    if (st == OR_OK) {
      for (int32_t d = 0; d < head_dim; ++d)
        qv[d] = load_elem(q, q_dtype, ((size_t)s * num_q_heads + h) * head_dim + d);
      st = oracle_attention_dense(qv, K, V, ctx, head_dim, scale,
                                  out + (size_t)p * head_dim, NULL);
    }
    if (st != OR_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
      status = st;
    }
    free(K);
    free(V);
    free(qv);
  }
  return status;
}

/* Sliding-window decode attention ([viz] "What the page leaves out" names
 * sliding-window attention): the new token attends only to the last `window`
 * positions of its sequence, [max(0, ctx - window), ctx); window <= 0 means
 * the whole context.  The rows of that range are un-paged and the dense
 * definition above applied, exactly as for the whole context.  Blocks wholly
 * before the window are never read, so their table entries may be anything. */
int oracle_paged_decode_attention_window(
    const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
    const uint16_t* k_scale, const uint16_t* v_scale, int32_t cache_dtype,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t num_blocks,
    int32_t block_size, int32_t head_dim, double scale, int32_t window,
    const int32_t* pairs, int64_t n_pairs, double* out, int32_t num_threads) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || block_size <= 0 || head_dim <= 0 ||
      max_blocks <= 0 || !elem_bytes(cache_dtype) || !elem_bytes(q_dtype))
    return OR_BAD_ARG;
  if ((cache_dtype == OR_I8 || cache_dtype == OR_FP8 || cache_dtype == OR_I4) &&
      (!k_scale || !v_scale))
    return OR_BAD_ARG;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (context_lens[s] < 0 || context_lens[s] > max_blocks * block_size)
      return OR_BAD_CTX;
  if (!pairs) n_pairs = (int64_t)num_seqs * num_q_heads;
  for (int64_t p = 0; pairs && p < n_pairs; ++p)
    if (pairs[2 * p] < 0 || pairs[2 * p] >= num_seqs || pairs[2 * p + 1] < 0 ||
        pairs[2 * p + 1] >= num_q_heads)
      return OR_BAD_ARG;
  int32_t group = num_q_heads / num_kv_heads;
  int status = OR_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t p = 0; p < n_pairs; ++p) {
    int32_t s = pairs ? pairs[2 * p] : (int32_t)(p / num_q_heads);
    int32_t h = pairs ? pairs[2 * p + 1] : (int32_t)(p % num_q_heads);
    int32_t ctx = context_lens[s];
    int32_t first = window > 0 && ctx > window ? ctx - window : 0;
    int32_t n = ctx - first;
    int32_t kvh = h / group;
    size_t rows = (size_t)(ctx > 0 ? ctx : 1) * head_dim;
    double* K = (double*)malloc(sizeof(double) * rows);
    double* V = (double*)malloc(sizeof(double) * rows);
    double* qv = (double*)malloc(sizeof(double) * head_dim);
    int st = (K && V && qv) ? OR_OK : OR_NO_MEM;
    /* un-page positions first..ctx-1 only: un-page the whole context through
     * a table shifted to start at the window's first block, then drop the
     * leading rows of that block */
    int32_t b0 = first / block_size;
    if (st == OR_OK)
      st = unpage(k_cache, v_cache, k_scale, v_scale, cache_dtype,
                  block_tables + (size_t)s * max_blocks + b0, ctx - b0 * block_size, kvh,
                  num_blocks, num_kv_heads, block_size, head_dim, K, V);
    if (st == OR_OK) {
      size_t skip = (size_t)(first - b0 * block_size) * head_dim;
      for (int32_t d = 0; d < head_dim; ++d)
        qv[d] = load_elem(q, q_dtype, ((size_t)s * num_q_heads + h) * head_dim + d);
      st = oracle_attention_dense(qv, K + skip, V + skip, n, head_dim, scale,
                                  out + (size_t)p * head_dim, NULL);
    }
    if (st != OR_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
      status = st;
    }
    free(K);
    free(V);
    free(qv);
  }
  return status;
}

/* Prefill (and chunked prefill) attention: several query tokens of one
 * sequence at once ([viz] "Without vs with the cache": the prefill pass takes
 * all prompt tokens in one go; [viz] "Prefill and decode feel different").
 * Sequence s brings T_s = query_start[s+1] - query_start[s] query tokens whose
 * K and V rows are already in the cache as its last T_s positions, so query
 * token i of s sits at position p = context_lens[s] - T_s + i.  Under the
 * causal mask a token never looks ahead ([viz] "The idea"): it attends to
 * positions 0..p, with the dense definition above.
 * q: [total][num_q_heads][head_dim] with total = query_start[num_seqs].
 * rows: optional list of n_rows (token, head) pairs; NULL = every pair,
 * token-major.  out: fp64 [n_rows][head_dim].                              */
int oracle_paged_prefill_attention(
    const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
    const uint16_t* k_scale, const uint16_t* v_scale, int32_t cache_dtype,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* query_start,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t num_blocks, int32_t block_size,
    int32_t head_dim, double scale, const int32_t* rows, int64_t n_rows,
    double* out, int32_t num_threads) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || block_size <= 0 || head_dim <= 0 ||
      max_blocks <= 0 || !elem_bytes(cache_dtype) || !elem_bytes(q_dtype) ||
      !query_start || query_start[0] != 0)
    return OR_BAD_ARG;
  if ((cache_dtype == OR_I8 || cache_dtype == OR_FP8 || cache_dtype == OR_I4) &&
      (!k_scale || !v_scale))
    return OR_BAD_ARG;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t t = query_start[s + 1] - query_start[s];
    if (t < 0) return OR_BAD_ARG;
    if (context_lens[s] < t || context_lens[s] > max_blocks * block_size) return OR_BAD_CTX;
  }
  const int64_t total = query_start[num_seqs];
  if (!rows) n_rows = total * num_q_heads;
  for (int64_t r = 0; rows && r < n_rows; ++r)
    if (rows[2 * r] < 0 || rows[2 * r] >= total || rows[2 * r + 1] < 0 ||
        rows[2 * r + 1] >= num_q_heads)
      return OR_BAD_ARG;
  int32_t group = num_q_heads / num_kv_heads;
  int status = OR_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t tok = rows ? rows[2 * r] : r / num_q_heads;
    int32_t h = rows ? rows[2 * r + 1] : (int32_t)(r % num_q_heads);
    int32_t s = 0;
    while (query_start[s + 1] <= tok) ++s;  /* the sequence holding token tok */
    int32_t t_s = query_start[s + 1] - query_start[s];
    int32_t pos = context_lens[s] - t_s + (int32_t)(tok - query_start[s]);
    int32_t n = pos + 1;                    /* positions 0..pos */
    int32_t kvh = h / group;
    double* K = (double*)malloc(sizeof(double) * (size_t)n * head_dim);
    double* V = (double*)malloc(sizeof(double) * (size_t)n * head_dim);
    double* qv = (double*)malloc(sizeof(double) * head_dim);
    int st = (K && V && qv) ? OR_OK : OR_NO_MEM;
    if (st == OR_OK)
      st = unpage(k_cache, v_cache, k_scale, v_scale, cache_dtype,
                  block_tables + (size_t)s * max_blocks, n, kvh, num_blocks,
                  num_kv_heads, block_size, head_dim, K, V);
    if (st == OR_OK) {
      for (int32_t d = 0; d < head_dim; ++d)
        qv[d] = load_elem(q, q_dtype, ((size_t)tok * num_q_heads + h) * head_dim + d);
      st = oracle_attention_dense(qv, K, V, n, head_dim, scale,
                                  out + (size_t)r * head_dim, NULL);
    }
    if (st != OR_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
      status = st;
    }
    free(K);
    free(V);
    free(qv);
  }
  return status;
}

/* Un-page every sequence to dense [num_seqs][max_blocks*block_size][kv_heads]
 * [head_dim] arrays by copying element bytes (exact).  Rows at or past a
 * sequence's context length are left untouched.  int8 scales are gathered
 * the same way into [num_seqs][max_blocks*block_size][kv_heads] when given. */
int oracle_gather_kv(const void* k_cache, const void* v_cache,
                     const uint16_t* k_scale, const uint16_t* v_scale,
                     const int32_t* block_tables, int32_t max_blocks,
                     const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_blocks, int32_t num_kv_heads,
                     int32_t block_size, int32_t head_dim, int32_t dtype,
                     void* k_out, void* v_out, uint16_t* k_scale_out,
                     uint16_t* v_scale_out) {
  size_t eb = elem_bytes(dtype);
  if (!eb || num_seqs < 0 || max_blocks <= 0) return OR_BAD_ARG;
  size_t row = dtype == OR_I4 ? (size_t)head_dim / 2 : (size_t)head_dim * eb;
  size_t spr = dtype == OR_I4 ? (size_t)head_dim / OR_I4_GROUP : 1; /* scales per row */
  int64_t cap = (int64_t)max_blocks * block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t ctx = context_lens[s];
    if (ctx < 0 || ctx > cap) return OR_BAD_CTX;
    for (int32_t i = 0; i < ctx; ++i) {
      int32_t block = block_tables[(size_t)s * max_blocks + i / block_size];
      if (block < 0 || block >= num_blocks) return OR_BAD_BLOCK;
      for (int32_t h = 0; h < num_kv_heads; ++h) {
        size_t src_row = ((size_t)block * num_kv_heads + h) * block_size + i % block_size;
        size_t dst_row = ((size_t)s * cap + i) * num_kv_heads + h;
        memcpy((char*)k_out + dst_row * row, (const char*)k_cache + src_row * row, row);
        memcpy((char*)v_out + dst_row * row, (const char*)v_cache + src_row * row, row);
        for (size_t g = 0; g < spr; ++g) {
          if (k_scale && k_scale_out) k_scale_out[dst_row * spr + g] = k_scale[src_row * spr + g];
          if (v_scale && v_scale_out) v_scale_out[dst_row * spr + g] = v_scale[src_row * spr + g];
        }
      }
    }
  }
  return OR_OK;
}

/* Per-row projection x . W (x: [d_in], W: [d_in][d_out] row-major) summed in
 * index order.  Used by the tiny decode loop that checks cached decode
 * against full recomputation; both of its lanes project rows with this one
 * routine so that equal inputs give equal bits. */
void oracle_project_row(const double* x, const double* W, int32_t d_in,
                        int32_t d_out, double* y) {
  for (int32_t j = 0; j < d_out; ++j) {
    double acc = 0.0;
    for (int32_t i = 0; i < d_in; ++i) acc += x[i] * W[(size_t)i * d_out + j];
    y[j] = acc;
  }
}

/* Bytes of cache per token ([viz] "How much memory"): a K row and a V row of
 * head_dim numbers for every KV head of every layer. */
int64_t oracle_kv_bytes_per_token(int64_t n_layers, int64_t n_kv_heads,
                                  int64_t head_dim, int64_t bytes_per_number) {
  return 2 * n_layers * n_kv_heads * head_dim * bytes_per_number;
}

int32_t oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
