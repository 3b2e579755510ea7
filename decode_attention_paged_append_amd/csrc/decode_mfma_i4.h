// decode_mfma_i4.h -- grouped-query paged decode attention over an int4 cache
// on the matrix cores (head_dim 128).
//
// Same computation and partials as the other decode kernels (phase 1 of the
// decode: "KV cache: the engine behind fast LLM inference", "Concept" and
// step 3; online softmax per "Flash attention: don't build the giant
// matrix"), over a cache of 4-bit codes with an fp16 scale per 32 dims (the
// 4-bit half of "What the page leaves out" on the KV-cache visualization
// page).  A cached value is (nibble - 8) * scale of its group.
//
// An int4 tile carries a quarter of the bytes of an fp16 one, so the work of
// widening codes decides the speed.  Both products take the codes exactly,
// as fp16 subnormals: the byte 0x0n under a zero high byte is n * 2^-24.
// One AND / shift splits a word into even and odd nibbles, one v_perm then
// builds a pair of subnormals; the +8 of the stored nibbles is taken out
// once per product, never per element.
//
//  * Scores.  One 16x16x32 MFMA contracts exactly one scale group (32 dims),
//    so each group's product has its own accumulator, started at
//    -8 * 2^-24 * sum(q over the group) to remove the bias, and the key
//    scale multiplies it in fp32 (v_fma_mix on the fp16 scale).
//  * Values.  O^T[dim][col] += V^T[dim][tok] . B[tok][col] with the sixteen
//    columns taken as (head, scale group) pairs: column n is head n % 4 of
//    the column set and group n / 4, and B = p * (value scale of that group),
//    rounded to fp16 like the weights of the 16-bit caches.  The rows of
//    value MFMA e are dims 16e .. 16e+15 (group e / 2), read from a raw-code
//    LDS tile by 4-bit transposing reads (i4_value_read), so each lane keeps
//    MFMAs 2(n / 4) and 2(n / 4) + 1, those of its column's group: 2^24 *
//    O^T - 8 * (column sum of B), the column sums kept beside the running
//    sums.  Odd MFMAs take 16 * code (the high nibble masked in place), and
//    their rows drop the 16 with the 2^24.
//  * Four heads per column set; the score MFMA repeats each head's query in
//    all four groups of columns, so every lane already holds the weights of
//    its column's head (its softmax runs four times over, in lanes that would
//    otherwise be padding).  Eight heads per workgroup would be two sets; at
//    two waves per SIMD that instance spilled 28 VGPRs and ran 1.7x slower
//    than two four-head workgroups per KV head, so only GC = 4 is launched.
//    Groups of eight or more heads take decode_mfma_i4h_kernel below, which
//    widens a tile once for sixteen heads.
//  * The rescale of the accumulators by alpha is a real branch: it runs only
//    on tiles that raise some running max.
//
// Tiling and the cross-wave merge follow the decode_mfma_kernel
// (decode_mfma.h); the K tile reaches the score MFMAs through two rounds of
// cross-row lane swaps (i4_key_transpose), not through LDS.
#pragma once

#include "decode_mfma.h"

namespace pa {

// v_perm selectors: bytes k of the two sources become the low bytes of the
// two halves of the result (high bytes zero): {lo.byte k, 0, hi.byte k, 0}.
__device__ __forceinline__ constexpr uint32_t i4_sel(int k) {
  return 0x0C000C00u | ((uint32_t)(4 + k) << 16) | (uint32_t)k;
}
constexpr uint32_t kNibbles = 0x0F0F0F0Fu;
typedef int i32x2 __attribute__((ext_vector_type(2)));
constexpr float kTwo24 = 16777216.0f;    // 2^24
constexpr float kTwoM24 = 1.0f / kTwo24;

// One K tile (16 rows of 64 bytes) is loaded with lane (q, r) = (lane / 16,
// lane % 16) holding row r, dims 32q + 8w .. +8 in word w.  Exchanging lane
// bit 5 with bit 1 of the word index, then lane bit 4 with bit 0 (the
// cross-row swaps of gfx950) leaves lane (g, n) = (lane / 16, lane % 16)
// holding row n, dims 32c + 8g .. +8 in word c: the A operand of score MFMA
// c, one scale group, with no trip through LDS.
__device__ __forceinline__ void i4_key_transpose(uint32_t (&x)[4]) {
  const auto a02 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
  const auto a13 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
  const auto b01 = __builtin_amdgcn_permlane16_swap(a02[0], a13[0], false, false);
  const auto b23 = __builtin_amdgcn_permlane16_swap(a02[1], a13[1], false, false);
  x[0] = b01[0];
  x[1] = b01[1];
  x[2] = b23[0];
  x[3] = b23[1];
}

// Eight codes (one word) as eight fp16 subnormals in dim order.
__device__ __forceinline__ u32x4 i4_widen(uint32_t x) {
  const uint32_t lo = x & kNibbles, hi = (x >> 4) & kNibbles;
  return u32x4{__builtin_amdgcn_perm(hi, lo, i4_sel(0)), __builtin_amdgcn_perm(hi, lo, i4_sel(1)),
               __builtin_amdgcn_perm(hi, lo, i4_sel(2)), __builtin_amdgcn_perm(hi, lo, i4_sel(3))};
}

// ---- V tile of raw codes in LDS (16 rows of 64 bytes, 1 KiB a wave).
// The 32-byte halves of row r trade places when bits 1 and 2 of r differ:
// the rows one transposing read touches (4g + k / 4 over the lanes of a
// pass) then fall on distinct banks.
__device__ __forceinline__ int i4_vhalf(int r) { return ((r >> 1) ^ (r >> 2)) & 1; }

// Lane l's 16-byte load: row l / 4, chunk l % 4.
__device__ __forceinline__ void i4_value_store(u32x4* vtile, int lane, u32x4 v) {
  const int r = lane >> 2;
  vtile[4 * r + ((lane & 3) ^ (2 * i4_vhalf(r)))] = v;
}

// Two 4-bit transposing reads (ds_read_b64_tr_b4: within each 16-lane group
// lane b receives, as its nibble k, nibble b of the 8 bytes that lane k
// points at).  In read h lane (g, k) points at token row 4g + k / 4, dims
// 64h + 16(k % 4) .. +16, so nibble k of lane (g, n)'s result is dim
// 64h + 16(k % 4) + n of token 4g + k / 4: byte b of word w holds token
// 4g + 2w + b / 2, its low nibble for value MFMA 4h + 2(b % 2), its high
// one for the next.
__device__ __forceinline__ void i4_value_read(const u32x4* vtile, int g, int n, u32x2 (&vw)[2]) {
  const int vrow = 4 * g + (n >> 2);
  const char* vt = (const char*)vtile + vrow * 64 + 8 * (n & 3);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    vw[h] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                (__attribute__((address_space(3))) i32x2*)(vt + 32 * (h ^ i4_vhalf(vrow)))));
}

// A operands of value MFMAs 2c (dims 32c + n, low nibbles) and 2c + 1
// (dims 32c + 16 + n, high nibbles masked in place: 16 x code), tokens
// 4g .. 4g+3: bytes c % 2 and c % 2 + 2 of each word, tokens (4g, 4g+1)
// from word 0 and (4g+2, 4g+3) from word 1, each under a zero high byte.
__device__ __forceinline__ void i4_value_operands(const u32x2 (&vw)[2], int c, u32x2& a0, u32x2& a1) {
  const uint32_t x0 = vw[c >> 1][0], x1 = vw[c >> 1][1];
  const uint32_t sel = 0x0C000C00u | ((uint32_t)((c & 1) + 2) << 16) | (uint32_t)(c & 1);
  a0 = u32x2{__builtin_amdgcn_perm(0u, x0 & kNibbles, sel), __builtin_amdgcn_perm(0u, x1 & kNibbles, sel)};
  a1 = u32x2{__builtin_amdgcn_perm(0u, x0 & ~kNibbles, sel), __builtin_amdgcn_perm(0u, x1 & ~kNibbles, sel)};
}

template <int BS, int GC, int NW>
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu(GC == 4 ? 3 : 2, 8)))
void decode_mfma_i4_kernel(const DecodeParams p) {
  constexpr int D = 128;
  constexpr int TT = 16;                  // positions per tile
  constexpr int ROWB = D / 2;             // cache bytes per row
  constexpr int KG = D / kInt4Group;      // scale groups per row = score MFMAs
  constexpr int VE = D / 16;              // value MFMAs per column set
  constexpr int CS = GC / 4;              // column sets
  constexpr int TPI = GC == 4 ? 2 : 1;    // tiles fetched per loop iteration
  static_assert(GC == 4 || GC == 8, "four or eight heads per workgroup");
  static_assert(BS % TT == 0, "a tile lies inside one block");
  static_assert(TT * ROWB == kWave * 16, "one K tile = one 16-byte load per lane");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int n = lane & 15;
  const WgCoord wc = wg_coord();
  const int slot = wc.part;
  const int kvh = wc.y / p.head_chunks;
  const int chunk = wc.y - kvh * p.head_chunks;
  const int s = wc.s;
  const int h0 = kvh * p.group + chunk * GC;
  const size_t out_row0 = (size_t)s * p.num_q_heads + h0;

  const int ctx = p.context_lens[s];
  const bool single = p.num_parts == 1;
  const int tok0 = partition_start(p, slot, ctx);
  const bool bad_ctx = ctx < 0 || ctx > p.max_blocks * BS;
  if (bad_ctx || tok0 >= ctx) {
    if (single) {
      const float fill = bad_ctx ? __builtin_nanf("") : 0.0f;
      for (int i = threadIdx.x; i < GC * D; i += NW * kWave)
        store_out<Fmt::I4>(p.out, out_row0 * D + i, fill);
    }
    return;
  }
  const int tok_end = min(ctx, tok0 + p.part_tokens);
  const int start = window_start(p, ctx);
  if (tok_end <= start) {  // wholly before the window (never the only partition)
    for (int i = threadIdx.x; i < GC * D; i += NW * kWave)
      store_result<Fmt::I4, D>(p, false, out_row0 + i / D, slot, i % D, kMaxInit, 0.0f, 0.0f);
    return;
  }
  const int ntiles = (tok_end - tok0 + TT - 1) / TT;
  const int t_first = (max(tok0, start) - tok0) / TT;
  const bool low_cut = start > tok0 + t_first * TT;
  const int32_t* __restrict__ table = p.block_tables + (size_t)s * p.max_blocks;
  // Fused append: the decoded token (position ctx-1) is this partition's last
  // row when tok_end == ctx.
  if (p.k_new != nullptr && tok_end == ctx)
    append_new_token<Fmt::I4, D, BS, NW * kWave>(p, table, s, kvh, ctx - 1);

  // Query of column n's head (4 sigma + n % 4), dims 32c + 8g .. +8: the B
  // operand of score MFMA c; the accumulator start removes the code bias.
  u32x4 qb[CS][KG];
  float qbias[CS][KG];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
#pragma unroll
    for (int c = 0; c < KG; ++c) {
      qb[cs][c] = *(const u32x4*)((const char*)p.q +
                                  ((out_row0 + 4 * cs + (n & 3)) * D + 32 * c + 8 * g) * 2);
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) t += f16_lo(qb[cs][c][w]) + f16_hi(qb[cs][c][w]);
      t = rows_sum(t);
      qbias[cs][c] = -8.0f * kTwoM24 * t;
    }
  }

  float m[CS], lsum[CS], corr[CS];  // per column: running max, sum, sum of B
  f32x4 o[CS][VE];                  // O^T * 2^-24 (biased codes): rows 8(4g+i)+e
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    m[cs] = kMaxInit;
    lsum[cs] = corr[cs] = 0.0f;
#pragma unroll
    for (int e = 0; e < VE; ++e) o[cs][e] = f32x4{0, 0, 0, 0};
  }
  bool bad_block = false;

  constexpr int REGION = GC * D * 4;  // one wave's accumulators for the merge
  constexpr int SC_WORDS = TT * KG / 2;  // words of one tile's key (or value) scales
  static_assert(2 * SC_WORDS == kWave, "one scale word per lane");
  __shared__ __attribute__((aligned(16))) char s_mem[NW * REGION];
  __shared__ float s_ml[NW][GC][2];
  __shared__ __attribute__((aligned(16))) uint32_t s_sc[NW][2 * SC_WORDS];  // a tile's scales
  __shared__ u32x4 s_v[NW][TT * ROWB / 16];  // a tile's raw value codes

  const char* __restrict__ kbase = (const char*)p.k_cache;
  const char* __restrict__ vbase = (const char*)p.v_cache;
  // lanes 0..31 fetch the tile's key scale words, 32..63 its value scale
  // words, each [row][group pair] in order
  const int sw = lane & (SC_WORDS - 1);
  const int sr = sw / (KG / 2);  // row of this lane's scale word
  const uint32_t* const ssrc = (const uint32_t*)(lane < SC_WORDS ? p.k_scale : p.v_scale) + sw;
  const uint32_t koff = n * ROWB + g * 16;  // lane (g, n): key row n, chunk g
  const uint32_t voff = lane * 16;          // value row lane / 4, chunk lane % 4
  const int blk0 = tok0 / BS;
  const int nblk = (tok_end + BS - 1) / BS - blk0;
  int ids = 0;
  int ids_base = -kWave;

  struct Raw {
    u32x4 k;           // 32 codes: row n, dims 32 g ..
    u32x4 v;           // 32 codes: row lane / 4, dims 32 (lane % 4) ..
    uint32_t sc;       // scale word lane % 32 of the tile (zero on masked rows)
    int nvalid;        // rows of the tile inside the partition
    int nlow;          // rows below this one are before the window
  };

  // The cache block of tile t (wave-uniform), from the 64 ids held one per
  // lane; reading an id waits for every load before it, so a loop step reads
  // all its tiles' ids before loading any of their rows.
  auto block_of = [&](const int t) {
    const int rel = (tok0 + t * TT) / BS - blk0;
    if (rel >= ids_base + kWave) {
      ids_base = rel & ~(kWave - 1);
      const int bi = ids_base + lane;
      ids = bi < nblk ? table[blk0 + bi] : 0;
    }
    const int phys = __builtin_amdgcn_readlane(ids, rel - ids_base);
    const bool ok = (unsigned)phys < (unsigned)p.num_blocks;
    bad_block |= !ok;
    return ok ? phys : 0;
  };

  auto fetch = [&](const int t, const int phys, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    Raw raw;
    const int ttok = tok0 + t * TT;
    const int nvalid = tok_end - ttok;
    const int nlow = start - ttok;
    raw.nvalid = nvalid;
    raw.nlow = nlow;
    const size_t row0 = ((size_t)phys * p.num_kv_heads + kvh) * BS + ttok % BS;
    const char* const kt = kbase + row0 * ROWB;  // the tile's rows (wave-uniform)
    const char* const vt = vbase + row0 * ROWB;

    const int r = lane >> 2;
    raw.k = u32x4{0, 0, 0, 0};
    raw.v = u32x4{0, 0, 0, 0};
    if (!PARTIAL || (n >= nlow && n < nvalid)) raw.k = load16_stream(kt + koff);
    if (!PARTIAL || (r >= nlow && r < nvalid)) raw.v = load16_stream(vt + voff);
    // rows outside [nlow, nvalid) get zero scales: their B is 0
    raw.sc = (!PARTIAL || (sr >= nlow && sr < nvalid)) ? ssrc[row0 * (KG / 2)] : 0u;
    return raw;
  };

  auto consume = [&](const Raw& raw, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    const int nvalid = raw.nvalid;
    const int nlow = raw.nlow;

    // ---- scales through LDS: key scales of tokens 4g .. 4g+3 x KG groups
    // (one address per 16 lanes), value scales of the same tokens in group
    // n / 4 as fp16 pairs
    uint32_t* const st = s_sc[wave];
    st[lane] = raw.sc;
    i4_value_store(s_v[wave], lane, raw.v);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t ks[8], vs[2];
    {
      const u32x4* s4 = (const u32x4*)st;
      const u32x4 k0 = s4[2 * g], k1 = s4[2 * g + 1];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        ks[w] = k0[w];
        ks[4 + w] = k1[w];
      }
      // token 4g+j's words sit at 2(4g+j) + (group / 2); the group's half of
      // two tokens' words makes one pair
      const uint32_t* vsw = st + SC_WORDS + 8 * g + (n >> 3);
      const uint32_t sel = ((n >> 2) & 1) ? 0x07060302u : 0x05040100u;
      vs[0] = __builtin_amdgcn_perm(vsw[2], vsw[0], sel);
      vs[1] = __builtin_amdgcn_perm(vsw[6], vsw[4], sel);
    }

    // ---- value A operands: dims 16e + n of tokens 4g..4g+3 (shared by the sets)
    u32x2 va[VE];
    {
      u32x2 vw[2];
      i4_value_read(s_v[wave], g, n, vw);
#pragma unroll
      for (int c = 0; c < KG; ++c) i4_value_operands(vw, c, va[2 * c], va[2 * c + 1]);
    }

    // ---- K: the score MFMAs' A operands straight from registers
    u32x4 ka[KG];
    {
      uint32_t x[4] = {raw.k[0], raw.k[1], raw.k[2], raw.k[3]};
      i4_key_transpose(x);
#pragma unroll
      for (int c = 0; c < KG; ++c) ka[c] = i4_widen(x[c]);
    }

#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      // ---- scores: one accumulator per scale group, scaled in fp32
      float sacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < KG; ++c) {
        const float b0 = qbias[cs][c];
        const f32x4 sc = Mfma<Fmt::F16>::qk(ka[c], qb[cs][c], f32x4{b0, b0, b0, b0});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = ks[(i * KG + c) >> 1];
          sacc[i] = fmaf(sc[i], (c & 1) ? f16_hi(w) : f16_lo(w), sacc[i]);
        }
      }
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = sacc[i] * (p.scale_log2 * kTwo24);
        if (PARTIAL && (4 * g + i >= nvalid || 4 * g + i < nlow)) z[i] = -__builtin_inff();
      }
      float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      mt = rows_max(mt);
      const float mn = fmaxf(m[cs], mt);
      const bool moved = mn > m[cs];
      const float alpha = fast_exp2(m[cs] - mn);
      m[cs] = mn;
      float pw[4];
      float ps = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[i] = fast_exp2(z[i] - mn);
        ps += pw[i];
      }
      lsum[cs] = fmaf(lsum[cs], alpha, ps);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(moved) != 0, 0)) {
#pragma unroll
        for (int e = 0; e < VE; ++e) o[cs][e] *= alpha;
        corr[cs] *= alpha;
      }
      // ---- values: B = p * value scale of column n's group, fp16
      // p * scale as one mixed-precision FMA each (fp16 scale, fp32 product)
      const u32x2 pb = {Mfma<Fmt::F16>::pack(fmaf(pw[0], f16_lo(vs[0]), 0.0f),
                                             fmaf(pw[1], f16_hi(vs[0]), 0.0f)),
                        Mfma<Fmt::F16>::pack(fmaf(pw[2], f16_lo(vs[1]), 0.0f),
                                             fmaf(pw[3], f16_hi(vs[1]), 0.0f))};
      corr[cs] = Mfma<Fmt::F16>::sum2(pb[1], Mfma<Fmt::F16>::sum2(pb[0], corr[cs]));
#pragma unroll
      for (int e = 0; e < VE; ++e) o[cs][e] = Mfma<Fmt::F16>::pv(va[e], pb, o[cs][e]);
    }
  };

  const int nfull = (tok_end - tok0) / TT;
  int t = t_first + wave;
  if (low_cut && wave == 0) {
    const Raw a = fetch(t, block_of(t), std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    consume(a, std::true_type{});
    t += NW;
  }
  if constexpr (TPI == 2) {
    for (; t + NW < nfull; t += 2 * NW) {
      const int ba = block_of(t);
      const int bb = block_of(t + NW);
      const Raw a = fetch(t, ba, std::false_type{});
      const Raw b = fetch(t + NW, bb, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      consume(a, std::false_type{});
      consume(b, std::false_type{});
    }
  }
  for (; t < ntiles; t += NW) {
    if (t < nfull) {
      const Raw a = fetch(t, block_of(t), std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      consume(a, std::false_type{});
    } else {
      const Raw a = fetch(t, block_of(t), std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      consume(a, std::true_type{});
    }
  }

  // ---- merge: the lanes' shares of l and of the column sums, then the
  // waves through LDS
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    lsum[cs] = rows_sum(lsum[cs]);
    corr[cs] = rows_sum(corr[cs]);
  }
  float* const s_acc = (float*)(s_mem + wave * REGION);  // [GC][D]
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    const int hh = 4 * cs + (n & 3);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      if (e / 2 != (n >> 2)) continue;  // MFMA e holds column group n / 4's dims
      const float f = (e & 1) ? kTwo24 / 16.0f : kTwo24;  // odd e: 16 x code
      const float b = -8.0f * corr[cs];
      *(f32x4*)(s_acc + hh * D + 16 * e + 4 * g) =
          f32x4{fmaf(o[cs][e][0], f, b), fmaf(o[cs][e][1], f, b), fmaf(o[cs][e][2], f, b),
                fmaf(o[cs][e][3], f, b)};
    }
  }
  if (g == 0 && n < 4) {
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      s_ml[wave][4 * cs + n][0] = m[cs];
      s_ml[wave][4 * cs + n][1] = lsum[cs];
    }
  }
  const bool bad = __syncthreads_or(bad_block ? 1 : 0) != 0;
  for (int i = threadIdx.x; i < GC * D; i += NW * kWave) {
    const int h = i / D;
    const int d = i - h * D;
    float M = s_ml[0][h][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = fast_exp2(s_ml[w][h][0] - M);
      L = fmaf(a, s_ml[w][h][1], L);
      acc = fmaf(a, ((const float*)(s_mem + w * REGION))[h * D + d], acc);
    }
    if (bad) M = L = acc = __builtin_nanf("");
    store_result<Fmt::I4, D>(p, single, out_row0 + h, slot, d, M, L, acc);
  }
}

// Eight or sixteen query heads per workgroup, one head per column: the
// matrix-core path for int4 caches with GQA groups of 8 or more.  With
// (head, group) columns a workgroup holds 4 heads and every further four
// fetch and widen the same tile again; here a tile is fetched and widened
// once for all GC heads.
//
//  * Scores as in decode_mfma_i4_kernel (one MFMA and accumulator per scale
//    group), with column n standing for head n % GC: at GC = 8 the second
//    eight columns repeat the first and are not stored.
//  * Values per scale group c: O^T[dim][head] += V^T[dim][tok] . B_c[tok][head]
//    over the 32 dims of group c (two MFMAs of 16 rows), B_c = p * (value
//    scale of group c at tok), rounded to fp16.  Every row of an MFMA lies
//    in one group, so its B operand carries that group's scale.  The rows of
//    value MFMA e are dims 16e .. 16e+15, which no lane's 16-byte load holds
//    for four tokens at once: the raw codes go through a per-wave LDS tile
//    (1 KiB), and two 4-bit transposing reads (ds_read_b64_tr_b4) give lane
//    (g, n) dim 16e + n of tokens 4g .. 4g+3 for all eight MFMAs, widened
//    to subnormals after the read.  The codes of odd MFMAs enter as
//    16 * code (the high nibble masked in place); their output rows drop
//    the 16 with the 2^24.
//  * S^T comes out with lane (g, n) holding tokens 4g .. 4g+3 of head n,
//    which is the B operand layout: the weights never move, and the running
//    max, sum and column sums of B are per lane.  Lane (g, n) ends with dims
//    16e + 4g + i of head n; the result is 2^24 * O^T - 8 * (column sum of
//    B_c) per group.
template <int BS, int GC, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(3, 8)))
void decode_mfma_i4h_kernel(const DecodeParams p) {
  constexpr int D = 128;
  constexpr int TT = 16;                  // positions per tile
  constexpr int ROWB = D / 2;             // cache bytes per row
  constexpr int KG = D / kInt4Group;      // scale groups per row = score MFMAs
  constexpr int VE = D / 16;              // value MFMAs (two per group)
  constexpr int K_LPR = ROWB / 16;        // lanes per row in a V load
  constexpr int ACC_STRIDE = D + 4;       // floats per head row of the merge buffer
  constexpr int TPI = 2;                  // tiles fetched per loop iteration
  constexpr int SC_WORDS = TT * KG / 2;   // words of one tile's key (or value) scales
  static_assert(GC == 8 || GC == 16, "eight or sixteen heads per workgroup");
  static_assert(BS % TT == 0, "a tile lies inside one block");
  static_assert(TT * ROWB == kWave * 16, "one K or V tile = one 16-byte load per lane");
  static_assert(VE == 2 * KG, "two value MFMAs per scale group");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int head = n % GC;  // this lane's column
  const WgCoord wc = wg_coord();
  const int slot = wc.part;
  const int kvh = wc.y / p.head_chunks;
  const int chunk = wc.y - kvh * p.head_chunks;
  const int s = wc.s;
  const int h0 = kvh * p.group + chunk * GC;
  const size_t out_row0 = (size_t)s * p.num_q_heads + h0;

  const int ctx = p.context_lens[s];
  const bool single = p.num_parts == 1;
  const int tok0 = partition_start(p, slot, ctx);
  const bool bad_ctx = ctx < 0 || ctx > p.max_blocks * BS;
  if (bad_ctx || tok0 >= ctx) {
    if (single) {
      const float fill = bad_ctx ? __builtin_nanf("") : 0.0f;
      for (int i = threadIdx.x; i < GC * D; i += NW * kWave)
        store_out<Fmt::I4>(p.out, out_row0 * D + i, fill);
    }
    return;
  }
  const int tok_end = min(ctx, tok0 + p.part_tokens);
  const int start = window_start(p, ctx);
  if (tok_end <= start) {  // wholly before the window (never the only partition)
    for (int i = threadIdx.x; i < GC * D; i += NW * kWave)
      store_result<Fmt::I4, D>(p, false, out_row0 + i / D, slot, i % D, kMaxInit, 0.0f, 0.0f);
    return;
  }
  const int ntiles = (tok_end - tok0 + TT - 1) / TT;
  const int t_first = (max(tok0, start) - tok0) / TT;
  const bool low_cut = start > tok0 + t_first * TT;
  const int32_t* __restrict__ table = p.block_tables + (size_t)s * p.max_blocks;
  // Fused append: the decoded token (position ctx-1) is this partition's last
  // row when tok_end == ctx.
  if (p.k_new != nullptr && tok_end == ctx)
    append_new_token<Fmt::I4, D, BS, NW * kWave>(p, table, s, kvh, ctx - 1);

  // Query of column n's head, dims 32c + 8g .. +8: the B operand of score
  // MFMA c; the accumulator start removes the code bias.
  u32x4 qb[KG];
  float qbias[KG];
#pragma unroll
  for (int c = 0; c < KG; ++c) {
    qb[c] = *(const u32x4*)((const char*)p.q + ((out_row0 + head) * D + 32 * c + 8 * g) * 2);
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) t += f16_lo(qb[c][w]) + f16_hi(qb[c][w]);
    t = rows_sum(t);
    qbias[c] = -8.0f * kTwoM24 * t;
  }

  float m = kMaxInit, lsum = 0.0f;
  float corr[KG];  // column sums of B_c (this lane's tokens)
  f32x4 o[VE];     // O^T * 2^-24 (biased codes): dims 16e + 4g + i, head n
#pragma unroll
  for (int c = 0; c < KG; ++c) corr[c] = 0.0f;
#pragma unroll
  for (int e = 0; e < VE; ++e) o[e] = f32x4{0, 0, 0, 0};
  bool bad_block = false;

  constexpr int TILE_BYTES = TT * ROWB;            // one V tile of raw codes
  constexpr int TILES_BYTES = TILE_BYTES + 2 * SC_WORDS * 4;  // V, then the scales
  constexpr int ACC_BYTES = GC * ACC_STRIDE * 4;
  constexpr int REGION = TILES_BYTES > ACC_BYTES ? TILES_BYTES : ACC_BYTES;
  static_assert(2 * SC_WORDS == kWave, "one scale word per lane");
  __shared__ __attribute__((aligned(16))) char s_mem[NW * REGION];
  __shared__ float s_ml[NW][GC][2];
  u32x4* const vtile = (u32x4*)(s_mem + wave * REGION);
  uint32_t* const stile = (uint32_t*)(vtile + TT * K_LPR);  // key, then value scales

  const char* __restrict__ kbase = (const char*)p.k_cache;
  const char* __restrict__ vbase = (const char*)p.v_cache;
  const uint32_t koff = n * ROWB + g * 16;  // lane (g, n): key row n, chunk g
  const uint32_t voff = lane * 16;          // value row lane / 4, chunk lane % 4
  const int blk0 = tok0 / BS;
  const int nblk = (tok_end + BS - 1) / BS - blk0;
  int ids = 0;
  int ids_base = -kWave;

  // The tile's scales arrive as one word per lane (lanes 0..31 the key
  // scales, 32..63 the value scales, each [row][group] in order) and are
  // spread through LDS: fetched whole by every lane, they took two thirds
  // of the registers of a tile in flight.  Key words land as they arrive;
  // value halves are re-laid [row / 4][group][row % 4], so one lane's two
  // 16-byte reads give each group's scales of its four tokens as fp16 pairs.
  const int sw = lane & (SC_WORDS - 1);  // this lane's scale word
  const int sr = sw / (KG / 2);          // and its row
  const uint32_t* const ssrc = (const uint32_t*)(lane < SC_WORDS ? p.k_scale : p.v_scale) + sw;
  const int sh0 = lane < SC_WORDS ? 2 * lane
                                  : 2 * SC_WORDS + (sr >> 2) * 16 + 2 * (sw & 1) * 4 + (sr & 3);
  const int sh1 = lane < SC_WORDS ? 2 * lane + 1 : sh0 + 4;  // the word's second group
  struct Raw {
    u32x4 k;           // 32 codes: row n, dims 32 g ..
    u32x4 v;           // 32 codes: row lane / 4, dims 32 (lane % 4) ..
    uint32_t sc;       // scale word lane % 32 of the tile (zero on masked rows)
    int nvalid;        // rows of the tile inside the partition
    int nlow;          // rows below this one are before the window
  };

  // The cache block of tile t (wave-uniform), from the 64 ids held one per
  // lane; reading an id waits for every load before it, so a loop step reads
  // all its tiles' ids before loading any of their rows.
  auto block_of = [&](const int t) {
    const int rel = (tok0 + t * TT) / BS - blk0;
    if (rel >= ids_base + kWave) {
      ids_base = rel & ~(kWave - 1);
      const int bi = ids_base + lane;
      ids = bi < nblk ? table[blk0 + bi] : 0;
    }
    const int phys = __builtin_amdgcn_readlane(ids, rel - ids_base);
    const bool ok = (unsigned)phys < (unsigned)p.num_blocks;
    bad_block |= !ok;
    return ok ? phys : 0;
  };

  auto fetch = [&](const int t, const int phys, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    Raw raw;
    const int ttok = tok0 + t * TT;
    const int nvalid = tok_end - ttok;
    const int nlow = start - ttok;
    raw.nvalid = nvalid;
    raw.nlow = nlow;
    const size_t row0 = ((size_t)phys * p.num_kv_heads + kvh) * BS + ttok % BS;
    const char* const kt = kbase + row0 * ROWB;  // the tile's rows (wave-uniform)
    const char* const vt = vbase + row0 * ROWB;

    const int r = lane / K_LPR;
    raw.k = u32x4{0, 0, 0, 0};
    raw.v = u32x4{0, 0, 0, 0};
    if (!PARTIAL || (n >= nlow && n < nvalid)) raw.k = load16_stream(kt + koff);
    if (!PARTIAL || (r >= nlow && r < nvalid)) raw.v = load16_stream(vt + voff);
    // rows outside [nlow, nvalid) get zero scales: their B is 0
    raw.sc = (!PARTIAL || (sr >= nlow && sr < nvalid)) ? ssrc[row0 * (KG / 2)] : 0u;
    return raw;
  };

  auto consume = [&](const Raw& raw, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    const int nvalid = raw.nvalid;
    const int nlow = raw.nlow;

    // ---- K: the score MFMAs' A operands straight from registers
    u32x4 ka[KG];
    {
      uint32_t x[4] = {raw.k[0], raw.k[1], raw.k[2], raw.k[3]};
      i4_key_transpose(x);
#pragma unroll
      for (int c = 0; c < KG; ++c) ka[c] = i4_widen(x[c]);
    }
    // ---- V tile -> LDS as raw codes; the scales beside it
    i4_value_store(vtile, lane, raw.v);
    ((uint16_t*)stile)[sh0] = (uint16_t)raw.sc;
    ((uint16_t*)stile)[sh1] = (uint16_t)(raw.sc >> 16);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // scales of tokens 4g .. 4g+3 x KG groups (one address per 16 lanes):
    // key words [token][group pair], value pairs vs[2c + j] = group c of
    // tokens 4g + 2j, 4g + 2j + 1
    uint32_t ks[8], vs[8];
    {
      const u32x4* s4 = (const u32x4*)stile;
      const u32x4 k0 = s4[2 * g], k1 = s4[2 * g + 1];
      const u32x4 v0 = s4[8 + 2 * g], v1 = s4[8 + 2 * g + 1];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        ks[w] = k0[w];
        ks[4 + w] = k1[w];
        vs[w] = v0[w];
        vs[4 + w] = v1[w];
      }
    }

    // ---- scores: one accumulator per scale group, scaled in fp32
    float sacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < KG; ++c) {
      const float b0 = qbias[c];
      const f32x4 sc = Mfma<Fmt::F16>::qk(ka[c], qb[c], f32x4{b0, b0, b0, b0});
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = ks[(i * KG + c) >> 1];
        sacc[i] = fmaf(sc[i], (c & 1) ? f16_hi(w) : f16_lo(w), sacc[i]);
      }
    }
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = sacc[i] * (p.scale_log2 * kTwo24);
      if (PARTIAL && (4 * g + i >= nvalid || 4 * g + i < nlow)) z[i] = -__builtin_inff();
    }
    float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mt = rows_max(mt);
    const float mn = fmaxf(m, mt);
    const bool moved = mn > m;
    const float alpha = fast_exp2(m - mn);
    m = mn;
    float pw[4];
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = fast_exp2(z[i] - mn);
      ps += pw[i];
    }
    lsum = fmaf(lsum, alpha, ps);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(moved) != 0, 0)) {
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] *= alpha;
#pragma unroll
      for (int c = 0; c < KG; ++c) corr[c] *= alpha;
    }

    // ---- values: B_c = p * value scale of group c, fp16; A = V^T from the
    // transposing reads
    u32x2 vw[2];
    i4_value_read(vtile, g, n, vw);
    // the weights rounded to fp16 once, times each group's scale pairs
    // (v_pk_mul_f16): B_c carries two roundings
    const uint32_t pp0 = Mfma<Fmt::F16>::pack(pw[0], pw[1]), pp1 = Mfma<Fmt::F16>::pack(pw[2], pw[3]);
#pragma unroll
    for (int c = 0; c < KG; ++c) {
      const u32x2 pb = {__builtin_bit_cast(uint32_t, as_h2(pp0) * as_h2(vs[2 * c])),
                        __builtin_bit_cast(uint32_t, as_h2(pp1) * as_h2(vs[2 * c + 1]))};
      corr[c] = Mfma<Fmt::F16>::sum2(pb[1], Mfma<Fmt::F16>::sum2(pb[0], corr[c]));
      u32x2 a0, a1;
      i4_value_operands(vw, c, a0, a1);
      o[2 * c] = Mfma<Fmt::F16>::pv(a0, pb, o[2 * c]);
      o[2 * c + 1] = Mfma<Fmt::F16>::pv(a1, pb, o[2 * c + 1]);
    }
  };

  const int nfull = (tok_end - tok0) / TT;
  int t = t_first + wave;
  if (low_cut && wave == 0) {
    const Raw a = fetch(t, block_of(t), std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    consume(a, std::true_type{});
    t += NW;
  }
  for (; t + (TPI - 1) * NW < nfull; t += TPI * NW) {
    int bl[TPI];
#pragma unroll
    for (int i = 0; i < TPI; ++i) bl[i] = block_of(t + i * NW);
    Raw r[TPI];
#pragma unroll
    for (int i = 0; i < TPI; ++i) r[i] = fetch(t + i * NW, bl[i], std::false_type{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TPI; ++i) consume(r[i], std::false_type{});
  }
  for (; t < ntiles; t += NW) {
    if (t < nfull) {
      const Raw a = fetch(t, block_of(t), std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      consume(a, std::false_type{});
    } else {
      const Raw a = fetch(t, block_of(t), std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      consume(a, std::true_type{});
    }
  }

  // ---- merge: the lanes' shares of l and of the column sums, then the
  // waves through LDS (head rows padded by 4 floats: conflict-free stores)
  lsum = rows_sum(lsum);
#pragma unroll
  for (int c = 0; c < KG; ++c) {
    corr[c] = rows_sum(corr[c]);
  }
  __syncthreads();  // every wave is done with its tile region
  float* const s_acc = (float*)(s_mem + wave * REGION);  // [GC][ACC_STRIDE]
  if (n < GC) {
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const float b = -8.0f * corr[e / 2];
      const float f = (e & 1) ? kTwo24 / 16.0f : kTwo24;  // odd e: 16 x code
      *(f32x4*)(s_acc + n * ACC_STRIDE + 16 * e + 4 * g) =
          f32x4{fmaf(o[e][0], f, b), fmaf(o[e][1], f, b), fmaf(o[e][2], f, b), fmaf(o[e][3], f, b)};
    }
    if (g == 0) {
      s_ml[wave][n][0] = m;
      s_ml[wave][n][1] = lsum;
    }
  }
  const bool bad = __syncthreads_or(bad_block ? 1 : 0) != 0;
  for (int i = threadIdx.x; i < GC * D; i += NW * kWave) {
    const int h = i / D;
    const int d = i - h * D;
    float M = s_ml[0][h][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = fast_exp2(s_ml[w][h][0] - M);
      L = fmaf(a, s_ml[w][h][1], L);
      acc = fmaf(a, ((const float*)(s_mem + w * REGION))[h * ACC_STRIDE + d], acc);
    }
    if (bad) M = L = acc = __builtin_nanf("");
    store_result<Fmt::I4, D>(p, single, out_row0 + h, slot, d, M, L, acc);
  }
}

}  // namespace pa
