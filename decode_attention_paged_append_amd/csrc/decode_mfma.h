// decode_mfma.h -- grouped-query paged decode attention on the matrix cores.
//
// Same computation and same partials as decode_partition_kernel (phase 1 of
// the decode: "KV cache: the engine behind fast LLM inference", "Concept" and
// step 3; online softmax per the guide's "Flash attention: don't build the
// giant matrix"), for GQA groups of 4..16 query heads per KV head ("How much
// memory" on the KV-cache visualization page).  With several query heads per
// key row the vector-ALU path spends ~4G VALU instructions per cached element,
// more than the HBM time; here both products are dense contractions and run
// as MFMA:
//
//   S^T[tok][head] = K[tok][:] . Q[head][:]      v_mfma_f32_16x16x32_{f16,bf16}
//   O^T[dim][head] += V^T[dim][tok] . P^T[tok][head]  v_mfma_f32_16x16x16_{f16,bf16}
//
// A tile is 16 consecutive positions of one block; each wave of the
// workgroup takes every NW-th tile of the partition.  Lane l = 16g + n.
//
//  * K reaches the MFMA A layout (lane l: row n) with no trip through LDS.
//    Each 16-byte wave-load covers whole 128-byte lines: 16 rows of 64 bytes,
//    or 8 rows of a 128-byte span, lane l taking row l % 8 of its load and
//    chunk l / 8.  In the second case two loads cover rows 0..7 and 8..15,
//    and one DPP exchange (row_ror:8 under bank masks) trades lane bit 3 with
//    the load index, leaving lane l all chunks of row n it needs: those at
//    bytes kbyte(g, c) below, whose dims the query operand follows.
//  * S^T comes out with lane l holding tokens 4g..4g+3 of head n: exactly the
//    B operand P^T of the value product, so the softmax weights never move.
//  * V needs no LDS: lane l loads tokens 4g..4g+3 of its own dims n*D/16..;
//    packing one dim of those 4 tokens gives the A operand of MFMA e directly
//    when MFMA e's row r stands for dim r*D/16 + e.  Every load is still one
//    whole row per 16 lanes (coalesced).
//  * The online max is per head = per lane column, so the output rescale is
//    a per-lane multiply; it is skipped when no running max moved.
//  * P is rounded to the operand format (fp16 / bf16) for the value product;
//    the running sum uses the fp32 weights.
//  * int8 caches: a code c enters both products as the fp16 subnormal
//    (c + 128) * 2^-24, exactly (its byte with the sign bit flipped, under a
//    zero high byte: one XOR and a v_perm per two codes).  The +128 comes out
//    once per product: the score MFMAs start from -128 * 2^-24 * sum(q), and
//    the value result drops 128 * (column sum of the weights), kept beside
//    the running sums.  The key scale multiplies the score, the value scale
//    the weight of its token.
//  * fp8 caches: codes become fp16 exactly (v_cvt_scalef32_pk_f16_fp8).
#pragma once

#include "decode_kernel.h"

namespace pa {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Matrix-core operations in the operand format of a cache format.
template <Fmt F> struct Mfma;
template <> struct Mfma<Fmt::F16> {
  __device__ static __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8, a),
                                                   __builtin_bit_cast(h16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h16x4, a),
                                                  __builtin_bit_cast(h16x4, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
    const f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, h16x2));
  }
  // acc + both halves of a packed pair (v_dot2 with ones)
  __device__ static __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(as_h2(w), h16x2{1, 1}, acc, false);
  }
};
template <> struct Mfma<Fmt::BF16> {
  __device__ static __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                      __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
    const f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  }
  __device__ static __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w), bf16x2{1, 1}, acc, false);
  }
};

// Four 8-bit codes -> four exact fp16 values (two words, element order kept);
// int8 codes as the biased subnormals (c + 128) * 2^-24.
template <Fmt F>
__device__ __forceinline__ u32x2 codes4_to_f16(uint32_t w) {
  if constexpr (F == Fmt::I8) {
    const uint32_t u = w ^ 0x80808080u;
    return u32x2{__builtin_amdgcn_perm(0u, u, 0x0C010C00u), __builtin_amdgcn_perm(0u, u, 0x0C030C02u)};
  } else {
    h16x2 lo, hi;
    Frag<F>::codes_to_half2(w, lo, hi);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  }
}
constexpr float kSub = 16777216.0f;  // 2^24: scale of the int8 subnormal codes

// Heads per workgroup (GC, padded to 16 in the MFMA) x NW waves.
template <Fmt F, int D, int BS, int GC, int NW>
__device__ __forceinline__ void decode_mfma_item(const DecodeParams& p, const WgCoord wc) {
  constexpr bool kQuant = FmtInfo<F>::quantized;
  constexpr bool kBias = F == Fmt::I8;          // codes biased by +128 (subnormals)
  constexpr Fmt OF = kQuant ? Fmt::F16 : F;     // MFMA operand format
  using MM = Mfma<OF>;
  constexpr int EB = FmtInfo<F>::bytes;         // cache element bytes
  constexpr int TT = 16;                        // positions per tile
  constexpr int ROWB = D * EB;                  // cache bytes per row
  constexpr int K_LOADS = TT * ROWB / 1024;     // 1 KiB wave-loads per K tile
  // byte of row n where lane (g, n)'s 8 dims of score MFMA c start, after
  // the loads and the exchange
  auto kbyte = [](int g, int c) {
    if constexpr (ROWB == 64) return 16 * g + 8 * c;                      // 8-bit, D 64
    else if constexpr (EB == 1) return 32 * g + 8 * c;                    // 8-bit, D 128
    else if constexpr (ROWB == 128) return 32 * g + 16 * c;               // 16-bit, D 64
    else return 128 * (c >> 1) + 32 * g + 16 * (c & 1);                   // 16-bit, D 128
  };
  constexpr int VW = ROWB / 16;                 // V bytes per lane per row (16, 8 or 4)
  constexpr int VE = D / 16;                    // dims per lane = value MFMAs per tile
  constexpr int QKS = D / 32;                   // 16x16x32 MFMAs per score tile
  constexpr int TPI = 2;                        // tiles fetched per loop iteration
  static_assert(BS % TT == 0, "a tile lies inside one block");
  static_assert(GC >= 1 && GC <= 16, "at most 16 heads per workgroup");
  static_assert(ROWB == 64 || ROWB == 128 || ROWB == 256, "K rows of 64, 128 or 256 bytes");
  static_assert(K_LOADS * (EB == 1 ? 2 : 1) == QKS, "one or two score MFMAs per K load");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int n = lane & 15;
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
        store_out<F>(p.out, out_row0 * D + i, fill);
    }
    return;
  }
  const int tok_end = min(ctx, tok0 + p.part_tokens);
  const int start = window_start(p, ctx);
  if (tok_end <= start) {  // wholly before the window (never the only partition)
    for (int i = threadIdx.x; i < GC * D; i += NW * kWave)
      store_result<F, D>(p, false, out_row0 + i / D, slot, i % D, kMaxInit, 0.0f, 0.0f);
    return;
  }
  const int ntiles = (tok_end - tok0 + TT - 1) / TT;
  const int t_first = (max(tok0, start) - tok0) / TT;   // first tile holding the window
  const bool low_cut = start > tok0 + t_first * TT;      // which then starts mid-tile
  const int32_t* __restrict__ table = p.block_tables + (size_t)s * p.max_blocks;
  // Fused append: the decoded token (position ctx-1) is this partition's last
  // row when tok_end == ctx.
  if (p.k_new != nullptr && tok_end == ctx)
    append_new_token<F, D, BS, NW * kWave>(p, table, s, kvh, ctx - 1);

  // B operand of the score product: Q^T, lane (g, n) holds head n's dims
  // kbyte(g, c) / EB .. +8 (zero for padding heads).
  u32x4 qb[QKS];
#pragma unroll
  for (int c = 0; c < QKS; ++c) {
    qb[c] = u32x4{0, 0, 0, 0};
    if (n < GC)
      qb[c] = *(const u32x4*)((const char*)p.q + ((out_row0 + n) * D + kbyte(g, c) / EB) * 2);
  }
  // int8: start of the score accumulation, -128 * 2^-24 * sum of head n's q
  float qbias = 0.0f;
  if constexpr (kBias) {
#pragma unroll
    for (int c = 0; c < QKS; ++c) {
#pragma unroll
      for (int w = 0; w < 4; ++w) qbias += f16_lo(qb[c][w]) + f16_hi(qb[c][w]);
    }
    qbias = rows_sum(qbias) * (-128.0f / kSub);
  }

  float m = kMaxInit;  // running max of head n (log2 units), same in all g
  float lsum = 0.0f;   // this lane's share of head n's running sum
  float corr = 0.0f;   // int8: this lane's share of head n's sum of fp16 weights
  f32x4 o[VE];         // O^T: rows dim (D/16)*(4g+i) + e, column head n
#pragma unroll
  for (int e = 0; e < VE; ++e) o[e] = f32x4{0, 0, 0, 0};
  bool bad_block = false;

  // LDS: the wave partials of the merge.
  constexpr int REGION = GC * D * 4;
  __shared__ __attribute__((aligned(16))) char s_mem[NW * REGION];
  __shared__ float s_ml[NW][GC][2];

  const char* __restrict__ kbase = (const char*)p.k_cache;
  const char* __restrict__ vbase = (const char*)p.v_cache;
  const int blk0 = tok0 / BS;
  const int nblk = (tok_end + BS - 1) / BS - blk0;
  int ids = 0;
  int ids_base = -kWave;

  // Raw data of one tile, as loaded.
  struct Raw {
    u32x4 k[K_LOADS];
    uint32_t v[4][VW / 4];
    uint32_t ks[2], vs[2];  // fp16 scales of tokens 4g..4g+3 (quantized caches)
    int nvalid;  // rows of the tile inside the partition
    int nlow;    // rows below this one are before the window
  };

  auto fetch = [&](const int t, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    Raw raw;
    const int ttok = tok0 + t * TT;
    const int nvalid = tok_end - ttok;
    const int nlow = start - ttok;
    raw.nvalid = nvalid;
    raw.nlow = nlow;
    const int rel = ttok / BS - blk0;  // block of the tile, from the partition's first
    if (rel >= ids_base + kWave) {
      ids_base = rel & ~(kWave - 1);
      const int bi = ids_base + lane;
      ids = bi < nblk ? table[blk0 + bi] : 0;
    }
    int phys = __builtin_amdgcn_readlane(ids, rel - ids_base);
    const bool ok = (unsigned)phys < (unsigned)p.num_blocks;
    bad_block |= !ok;
    phys = ok ? phys : 0;
    const size_t row0 = ((size_t)phys * p.num_kv_heads + kvh) * BS + ttok % BS;
    const char* kt = kbase + row0 * ROWB;
    const char* vt = vbase + row0 * ROWB;

    // ---- loads: K (whole lines), V (token 4g+j, dims of lane n), int8 scales
    u32x4* const kraw = raw.k;
#pragma unroll
    for (int j = 0; j < K_LOADS; ++j) {
      // 64-byte rows: row n, chunk g; else row 8 (j % 2) + lane % 8, chunk
      // 8 (j / 2) + lane / 8
      const int r = ROWB == 64 ? n : 8 * (j & 1) + (lane & 7);
      const int off = ROWB == 64 ? n * ROWB + 16 * g
                                 : r * ROWB + 128 * (j >> 1) + 16 * (lane >> 3);
      kraw[j] = u32x4{0, 0, 0, 0};
      if (!PARTIAL || (r >= nlow && r < nvalid)) kraw[j] = load16_stream(kt + off);
    }
    uint32_t (*const vraw)[VW / 4] = raw.v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * g + j;
      const char* src = vt + (size_t)r * ROWB + n * VW;
      const bool valid = !PARTIAL || (r >= nlow && r < nvalid);
      if constexpr (VW == 16) {
        u32x4 v = valid ? load16_stream(src) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < 4; ++w) vraw[j][w] = v[w];
      } else if constexpr (VW == 8) {
        u32x2 v = valid ? __builtin_nontemporal_load((const u32x2*)src) : u32x2{0, 0};
        vraw[j][0] = v[0];
        vraw[j][1] = v[1];
      } else {
        vraw[j][0] = valid ? __builtin_nontemporal_load((const uint32_t*)src) : 0u;
      }
    }
    if constexpr (kQuant) {
      // scales of tokens 4g..4g+3: 8 contiguous bytes, kept as fp16 pairs
      const size_t srow = row0 + 4 * g;
      const bool any = !PARTIAL || (4 * g < nvalid && 4 * g + 3 >= nlow);
      const u32x2 kw = any ? *(const u32x2*)(p.k_scale + srow) : u32x2{0, 0};
      const u32x2 vw = any ? *(const u32x2*)(p.v_scale + srow) : u32x2{0, 0};
      raw.ks[0] = kw[0]; raw.ks[1] = kw[1];
      raw.vs[0] = vw[0]; raw.vs[1] = vw[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // rows outside [nlow, nvalid) never contribute (their weight is 0)
        if (PARTIAL && (4 * g + i >= nvalid || 4 * g + i < nlow)) {
          const uint32_t keep = (i & 1) ? 0x0000FFFFu : 0xFFFF0000u;
          raw.ks[i >> 1] &= keep;
          raw.vs[i >> 1] &= keep;
        }
      }
    }
    return raw;
  };

  auto consume = [&](const Raw& raw, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    const int nvalid = raw.nvalid;
    const int nlow = raw.nlow;
    const u32x4* const kraw = raw.k;
    const uint32_t (*const vraw)[VW / 4] = raw.v;
    // scale of token 4g+i as the f16 operand of a v_fma_mix
    auto scale_of = [](const uint32_t* w, int i) { return (i & 1) ? f16_hi(w[i >> 1]) : f16_lo(w[i >> 1]); };

    // ---- K: lanes with bit 3 set swap their load 2i with the other lanes'
    // load 2i + 1 (row_ror:8 reaches lane ^ 8): lane (g, n) then holds row n
    u32x4 kx[K_LOADS];
#pragma unroll
    for (int j = 0; j < K_LOADS; ++j) kx[j] = kraw[j];
    if constexpr (ROWB != 64) {
#pragma unroll
      for (int j = 0; j < K_LOADS; j += 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x0 = kraw[j][w], x1 = kraw[j + 1][w];
          kx[j][w] = __builtin_amdgcn_update_dpp(x0, x1, 0x128, 0xF, 0xC, false);
          kx[j + 1][w] = __builtin_amdgcn_update_dpp(x1, x0, 0x128, 0xF, 0x3, false);
        }
      }
    }

    // ---- scores: S^T = K . Q^T, lane (g, n): tokens 4g+i of head n
    f32x4 sacc = {qbias, qbias, qbias, qbias};
#pragma unroll
    for (int c = 0; c < QKS; ++c) {
      u32x4 a;
      if constexpr (EB == 1) {
        // codes 8(c % 2) .. +8 of register c / 2, widened in order
        const u32x2 lo = codes4_to_f16<F>(kx[c >> 1][2 * (c & 1)]);
        const u32x2 hi = codes4_to_f16<F>(kx[c >> 1][2 * (c & 1) + 1]);
        a = u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        a = kx[c];
      }
      sacc = MM::qk(a, qb[c], sacc);
    }
    constexpr float zs = kBias ? kSub : 1.0f;
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = kQuant ? fmaf(sacc[i], scale_of(raw.ks, i), 0.0f) * (p.scale_log2 * zs)
                    : sacc[i] * p.scale_log2;
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
    // a real branch (the hint keeps the compiler from if-converting it): the
    // rescale runs only on tiles that raise some running max
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(moved) != 0, 0)) {
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] *= alpha;
      corr *= alpha;
    }
    if constexpr (kQuant) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = fmaf(pw[i], scale_of(raw.vs, i), 0.0f);
    }
    const u32x2 pb = {MM::pack(pw[0], pw[1]), MM::pack(pw[2], pw[3])};
    if constexpr (kBias) corr = MM::sum2(pb[1], MM::sum2(pb[0], corr));

    // ---- values: O^T += V^T . P^T, MFMA e uses dim (D/16)*row + e
    if constexpr (F == Fmt::I8) {
      // bias every code once (c ^ 0x80 = c + 128 mod 256: the low byte of its
      // fp16 subnormal); the v_perm then takes byte e of two tokens' words,
      // each under a zero high byte: dim e of tokens 4g..4g+3, widened
      uint32_t vb[4][VW / 4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int w = 0; w < VW / 4; ++w) vb[j][w] = vraw[j][w] ^ 0x80808080u;
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const int w = e >> 2;
        const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + (e & 3)) << 16) | (uint32_t)(e & 3);
        const u32x2 a = {__builtin_amdgcn_perm(vb[1][w], vb[0][w], sel),
                         __builtin_amdgcn_perm(vb[3][w], vb[2][w], sel)};
        o[e] = MM::pv(a, pb, o[e]);
      }
      return;
    }
    uint32_t vh[4][VE / 2];  // fp16/bf16 words of tokens 4g+j, dims of lane n
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (kQuant) {
#pragma unroll
        for (int w = 0; w < VW / 4; ++w) {
          const u32x2 h = codes4_to_f16<F>(vraw[j][w]);
          vh[j][2 * w] = h[0];
          vh[j][2 * w + 1] = h[1];
        }
      } else {
#pragma unroll
        for (int w = 0; w < VE / 2; ++w) vh[j][w] = vraw[j][w];
      }
    }
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const int w = e >> 1;
      const u32x2 a = {__builtin_amdgcn_perm(vh[1][w], vh[0][w], sel),
                       __builtin_amdgcn_perm(vh[3][w], vh[2][w], sel)};
      o[e] = MM::pv(a, pb, o[e]);
    }
  };

  // TPI tiles a loop step.  The second tile's block id is read (v_readlane of
  // the ids) after the first tile's loads are issued, and the read waits for
  // them: the first tile lands before the second's loads go out, which then
  // overlap the first tile's math.  Reading both ids first, so that both
  // tiles' loads are in flight together, measured 0.6-1.8 % slower on the
  // 16-bit, int8 and fp8 workloads (the int4 kernels do read them first).
  const int nfull = (tok_end - tok0) / TT;  // tiles with every row valid
  int t = t_first + wave;
  if (low_cut && wave == 0) {  // the window starts inside this wave's first tile
    const Raw a = fetch(t, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    consume(a, std::true_type{});
    t += NW;
  }
  if constexpr (TPI == 2) {
    for (; t + NW < nfull; t += 2 * NW) {
      const Raw a = fetch(t, std::false_type{});
      const Raw b = fetch(t + NW, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      consume(a, std::false_type{});
      consume(b, std::false_type{});
    }
  }
  for (; t < ntiles; t += NW) {
    if (t < nfull) {
      const Raw a = fetch(t, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      consume(a, std::false_type{});
    } else {
      const Raw a = fetch(t, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      consume(a, std::true_type{});
    }
  }

  // ---- merge: sum the lanes' shares of l, then the waves through LDS
  lsum = rows_sum(lsum);
  if constexpr (kBias) corr = rows_sum(corr);
  float* const s_acc = (float*)(s_mem + wave * REGION);  // [GC][D]
  if (n < GC) {
#pragma unroll
    for (int e = 0; e < VE; ++e) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_acc[n * D + (D / 16) * (4 * g + i) + e] =
            kBias ? fmaf(o[e][i], kSub, -128.0f * corr) : o[e][i];
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
      acc = fmaf(a, ((const float*)(s_mem + w * REGION))[h * D + d], acc);
    }
    if (bad) M = L = acc = __builtin_nanf("");
    store_result<F, D>(p, single, out_row0 + h, slot, d, M, L, acc);
  }
}

// One (partition, KV head x chunk, sequence) item per workgroup, or for a
// paired plan two sequences one after the other (paired_sequences).
template <Fmt F, int D, int BS, int GC, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(3, 8)))
void decode_mfma_kernel(const DecodeParams p) {
  WgCoord wc = wg_coord();
  if (!p.pair) {
    decode_mfma_item<F, D, BS, GC, NW>(p, wc);
    return;
  }
  int second;
  wc.s = paired_sequences<NW * kWave>(p, wc.s, &second);
  decode_mfma_item<F, D, BS, GC, NW>(p, wc);
  if (second >= 0) {
    __syncthreads();  // the first sequence's merge is done with LDS
    wc.s = second;
    decode_mfma_item<F, D, BS, GC, NW>(p, wc);
  }
}

}  // namespace pa
