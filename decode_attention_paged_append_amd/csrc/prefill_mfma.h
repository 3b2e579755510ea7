// prefill_mfma.h -- causal attention of query chunks over the paged cache
// (prefill and chunked prefill) on the matrix cores.
//
// The prefill pass takes all prompt tokens at once and is bound by arithmetic,
// not memory ("Without vs with the cache" and "Prefill and decode feel
// different" on the KV-cache visualization page).  Sequence s brings T_s query
// tokens whose K/V rows already sit in the cache as its last T_s positions;
// the query at position p attends to positions 0..p (a token never looks
// ahead: "The idea" on the same page).  Tiles stream through on-chip memory
// with an online softmax and the score matrix is never stored (the
// jovanaeducation guide, "Flash attention: don't build the giant matrix").
//
// Work split: a workgroup owns RWG = NW waves x 16*NR query rows of one
// (sequence, KV head); rows are (token, head of the group) pairs, token-major,
// so all query heads of a KV head share every K/V tile.  The workgroup walks
// the KV positions 0..(its last row's position) in tiles of 32, staged in LDS
// (double-buffered, one barrier per tile) and read by all its waves:
//
//   S^T[tok][row] = K[tok][:] . Q[row][:]       v_mfma_f32_16x16x32_{f16,bf16}
//   O^T[dim][row] += V^T[dim][tok] . P^T[tok][row]   v_mfma_f32_16x16x32_{f16,bf16}
//
// Lane l = 16g + n.  The two 16-token halves of a score tile leave lane (g, n)
// holding tokens {4g..4g+3, 16+4g..16+4g+3} of row n, which is the B operand
// P^T of the value product when its 32 k-slots are mapped to those tokens;
// the A operand V^T comes straight from LDS through transposing reads
// (ds_read_b64_tr_b16): dim 16e + n of those 8 tokens for value MFMA e.
#pragma once

#include "decode_mfma.h"

namespace pa {

struct VtOperand {  // the two transposed reads of a value MFMA's A operand
  i16x4 lo, hi;
};

struct PrefillParams {
  const void* q;            // [total][Hq][D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* query_start;  // [S+1]
  const int32_t* context_lens; // [S]
  void* out;                // [total][Hq][D]
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t group;
  float scale_log2;         // scale * log2(e)
};

constexpr float kLazyRescale = 8.0f;  // log2 units
constexpr int kPrefillTile = 32;  // KV positions per tile

template <Fmt F, int D, int BS, int NR, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(NW / 4, 2)))
void prefill_mfma_kernel(const PrefillParams p) {
  using MM = Mfma<F>;
  constexpr int TT = kPrefillTile;
  constexpr int RW = 16 * NR;                  // query rows per wave
  constexpr int RWG = NW * RW;                 // query rows per workgroup
  constexpr int CH = D / 8;                    // 16-byte chunks per row
  constexpr int QKS = D / 32;                  // score MFMAs per 16 tokens and 16 rows
  constexpr int VE = D / 16;                   // dims per lane = value MFMAs per 16 rows
  constexpr int TILE_CHUNKS = TT * CH;         // 16-byte chunks per K (or V) tile
  constexpr int PER_THREAD = (TILE_CHUNKS + NW * kWave - 1) / (NW * kWave);
  constexpr bool EVEN = PER_THREAD * NW * kWave == TILE_CHUNKS;  // else the last pass is partial
  // V chunk c of row r sits at c ^ vswz(r).  A transposing read of value
  // MFMA e touches chunks 2e, 2e+1 of rows 4g .. 4g+3 (and 16 + those): at 16
  // chunks a row, XOR-ing 2(r & 7) gives each of 8 rows its own 32-byte pair
  // of banks (chunk ^ (r & 7) left two rows on each pair: 2-way conflicts,
  // 1.2 conflict cycles per LDS instruction); at 8 chunks, r & 7.
  auto vswz = [](int r) { return CH == 16 ? 2 * (r & 7) : (r & 7); };

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int n = lane & 15;
  // grid (KV head, sequence, row tile): the KV head runs fastest, so every
  // row tile of a (sequence, KV head) lands on the same XCD (the one whose L2
  // holds its K/V), and the row tile slowest, so all the longest tiles of the
  // launch are dispatched first
  const int kvh = blockIdx.x;
  const int s = blockIdx.y;
  const int G = p.group;
  const int q0 = p.query_start[s];
  const int T = p.query_start[s + 1] - q0;
  const int ctx = p.context_lens[s];
  const int R0 = ((int)gridDim.z - 1 - (int)blockIdx.z) * RWG;  // late rows (most work) first
  if (R0 >= T * G) return;
  const int Hq = p.num_q_heads;

  const bool bad_ctx = T < 0 || ctx < T || ctx > p.max_blocks * BS;
  const int base = ctx - T;  // position of the chunk's first query token
  if (bad_ctx) {
    const int rows = min(RWG, T * G - R0);
    for (int i = threadIdx.x; i < rows * D; i += NW * kWave) {
      const int rr = R0 + i / D;
      const size_t orow = (size_t)(q0 + rr / G) * Hq + kvh * G + rr % G;
      store_out<F>(p.out, orow * D + i % D, __builtin_nanf(""));
    }
    return;
  }

  // ---- this lane's query rows: group r, column n
  const int Rw = R0 + wave * RW;
  int qpos[NR];
  u32x4 qb[NR][QKS];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rr = Rw + 16 * r + n;
    const int tok = rr / G;
    qpos[r] = base + tok;  // rows past the chunk compute garbage that is never stored
#pragma unroll
    for (int c = 0; c < QKS; ++c) {
      qb[r][c] = u32x4{0, 0, 0, 0};
      if (tok < T) {
        const size_t qrow = (size_t)(q0 + tok) * Hq + kvh * G + rr % G;
        qb[r][c] = load16((const char*)p.q + (qrow * D + 32 * c + 8 * g) * 2);
      }
    }
  }
  const int last_tok_wg = min(T - 1, (R0 + RWG - 1) / G);
  const int ntiles = (base + last_tok_wg) / TT + 1;
  const int wave_first_tok = Rw / G;
  const int wave_last_tok = min(T - 1, (Rw + RW - 1) / G);
  const bool wave_live = wave_first_tok < T;
  const int wave_qmin = base + wave_first_tok;
  const int wave_qmax = base + wave_last_tok;

  float m[NR], lsum[NR], thr[NR];  // thr: the lazy-rescale threshold on raw scores
  f32x4 o[NR][VE];
  const float inv_scale_log2 = 1.0f / p.scale_log2;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    m[r] = kMaxInit;
    thr[r] = (kMaxInit + kLazyRescale) * inv_scale_log2;
    lsum[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < VE; ++e) o[r][e] = f32x4{0, 0, 0, 0};
  }

  __shared__ __attribute__((aligned(16))) u32x4 s_k[2][TILE_CHUNKS];
  __shared__ __attribute__((aligned(16))) u32x4 s_v[2][TILE_CHUNKS];

  const int32_t* __restrict__ table = p.block_tables + (size_t)s * p.max_blocks;
  const char* __restrict__ kbase = (const char*)p.k_cache;
  const char* __restrict__ vbase = (const char*)p.v_cache;
  bool bad_block = false;

  // Cooperative tile loads: chunk idx = row * CH + c of a tile.  Stage s of
  // the pipeline is {K of tile s, V of tile s-1}: the value product of a tile
  // runs one step after its scores.  Stages are fetched two steps ahead of
  // their use (two register stages), a tile's block ids one step ahead of its
  // rows, so neither the table nor the cache rows are waited for while there
  // is math to do.
  struct Stage {
    u32x4 k[PER_THREAD], v[PER_THREAD];
  };
  auto load_ids = [&](const int t, int (&ids)[PER_THREAD]) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int idx = j * NW * kWave + threadIdx.x;
      const int row = idx / CH;
      const int pos = t * TT + row;
      ids[j] = (EVEN || idx < TILE_CHUNKS) && t < ntiles && pos < ctx ? table[pos / BS] : 0;
    }
  };
  auto load_rows = [&](const char* base_ptr, const int t, const int (&ids)[PER_THREAD],
                       u32x4 (&dst)[PER_THREAD]) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int idx = j * NW * kWave + threadIdx.x;
      const int row = idx / CH;
      const int c = idx - row * CH;
      const int pos = t * TT + row;
      dst[j] = u32x4{0, 0, 0, 0};
      if ((EVEN || idx < TILE_CHUNKS) && t >= 0 && t < ntiles && pos < ctx) {
        int blk = ids[j];
        const bool ok = (unsigned)blk < (unsigned)p.num_blocks;
        bad_block |= !ok;
        blk = ok ? blk : 0;
        const size_t off = ((((size_t)blk * p.num_kv_heads + kvh) * BS + pos % BS) * CH + c) * 16;
        dst[j] = load16(base_ptr + off);
      }
    }
  };
  auto store_stage = [&](const int s, const Stage& st) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int idx = j * NW * kWave + threadIdx.x;
      const int row = idx / CH;
      const int c = idx - row * CH;
      if (!EVEN && idx >= TILE_CHUNKS) continue;
      if (s < ntiles) s_k[s & 1][row * CH + (c ^ (row % CH))] = st.k[j];
      if (s >= 1) s_v[(s - 1) & 1][row * CH + (c ^ vswz(row))] = st.v[j];
    }
  };

  // ---- the three pieces of a tile's math
  auto tile_live = [&](const int t) { return wave_live && t >= 0 && t < ntiles && t * TT <= wave_qmax; };

  // S^T = K . Q^T for the wave's row groups, two 16-token halves
  auto scores = [&](const int t, f32x4 (&sacc)[2][NR]) {
    const int buf = t & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int krow = 16 * h + n;
      u32x4 a[QKS];
#pragma unroll
      for (int c = 0; c < QKS; ++c) a[c] = s_k[buf][krow * CH + ((4 * c + g) ^ (krow % CH))];
      // chunk outer, row group inner: NR independent accumulation chains
#pragma unroll
      for (int r = 0; r < NR; ++r) sacc[h][r] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < QKS; ++c) {
#pragma unroll
        for (int r = 0; r < NR; ++r) sacc[h][r] = MM::qk(a[c], qb[r][c], sacc[h][r]);
      }
    }
  };

  // Online softmax of a score tile into the fp16/bf16 weights pb.  Scores
  // stay raw (the scale is positive, so maxima commute with it); a weight is
  // exp2(s * scale_log2 - m) in one FMA and one v_exp.  The accumulators hold
  // the tiles before this one when it rescales them.
  auto softmax = [&](const int t, const f32x4 (&sacc)[2][NR], u32x4 (&pb)[NR]) {
    const int t0 = t * TT;
    auto body = [&](auto diag_tag) {
      constexpr bool DIAG = decltype(diag_tag)::value;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float sv[2][4];
        bool need = false;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[h][i] = sacc[h][r][i];
            if (DIAG && t0 + 16 * h + 4 * g + i > qpos[r]) sv[h][i] = -__builtin_inff();
            need |= sv[h][i] > thr[r];
          }
        }
        // The reference max m of a row moves only when one of its scores
        // exceeds it by more than kLazyRescale.  The result is the same for
        // any reference (it cancels in the normalisation); weights stay
        // <= 2^kLazyRescale, far inside the operand formats' range; and on
        // almost every tile neither the row-wide max (two cross-lane steps)
        // nor the accumulator rescale is needed.  The test compares the raw
        // scores with thr = (m + kLazyRescale) / scale_log2 (scale_log2 > 0:
        // the library rejects other scales): compares, unlike a max, take the
        // matrix cores' results as they are.
        float mn = m[r];
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
          float mt = -__builtin_inff();
#pragma unroll
          for (int h = 0; h < 2; ++h)
            mt = fmaxf(mt, fmaxf(fmaxf(sv[h][0], sv[h][1]), fmaxf(sv[h][2], sv[h][3])));
          mt = rows_max(mt) * p.scale_log2;
          if (mt > m[r] + kLazyRescale) mn = mt;  // same decision on the row's 4 lanes
          const float alpha = fast_exp2(m[r] - mn);
#pragma unroll
          for (int e = 0; e < VE; ++e) o[r][e] *= alpha;
          lsum[r] *= alpha;
          m[r] = mn;
          thr[r] = (mn + kLazyRescale) * inv_scale_log2;
        }
        float pw[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int i = 0; i < 4; ++i) pw[h][i] = fast_exp2(fmaf(sv[h][i], p.scale_log2, -mn));
        }
        pb[r] = u32x4{MM::pack(pw[0][0], pw[0][1]), MM::pack(pw[0][2], pw[0][3]),
                      MM::pack(pw[1][0], pw[1][1]), MM::pack(pw[1][2], pw[1][3])};
        // the row sum of the rounded weights, the ones the value product uses
        float ps = lsum[r];
#pragma unroll
        for (int w = 0; w < 4; ++w) ps = MM::sum2(pb[r][w], ps);
        lsum[r] = ps;
      }
    };
    if (t0 + TT - 1 > wave_qmin)  // some (row, token) pair is masked
      body(std::true_type{});
    else
      body(std::false_type{});
  };

  // O^T += V^T . P^T
  auto values = [&](const int t, const u32x4 (&pb)[NR]) {
    const int buf = t & 1;
    const _Float16* vt = (const _Float16*)&s_v[buf][0];
    // Transposing LDS reads (ds_read_b64_tr_b16): within each 16-lane group,
    // lane 4q + j receives half j of the 8 bytes that lanes 4k + q (k = 0..3)
    // point at.  Lane (g, 4k + q) points at token row 4g + k, dims 16e + 4q
    // .. +3, so lane (g, n) receives dim 16e + n of tokens 4g .. 4g+3: the A
    // operand V^T of value MFMA e (row n = dim 16e + n), with a second read
    // for tokens 16 + 4g .. (the k-slots 4..7 of the lane's weights).  V's
    // 16-byte chunks sit XOR-swizzled by vswz(row); reading row-major rows
    // whole and regrouping them with v_perm was 4-6 % slower.
    const int k = n >> 2, q = n & 3;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const int chunk = 2 * e + (q >> 1);
      auto read = [&](const int row) {
        const int off = row * D + (chunk ^ vswz(row)) * 8 + (q & 1) * 4;
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vt + off));
      };
      const u32x4 va = __builtin_bit_cast(u32x4, VtOperand{read(4 * g + k), read(16 + 4 * g + k)});
#pragma unroll
      for (int r = 0; r < NR; ++r) o[r][e] = MM::qk(va, pb[r], o[r][e]);
    }
  };

  // ---- pipeline.  Step t holds K of tile t and V of tile t-1 in LDS: a wave
  // runs the value product of t-1 and the scores of t back to back on the
  // matrix cores (32 MFMAs at NR = 2), then the softmax of t on the vector ALU.
  // Measured on MI355X this beats scores, softmax and values of one tile in a
  // row (+7 % whole prompts, +12 % chunks), and beats splitting the waves of
  // each SIMD into two groups in opposite phases (a second barrier per tile).
  f32x4 sacc[2][NR];
  u32x4 pb[NR];
  Stage st;
  int ids_next[PER_THREAD], ids_last[PER_THREAD];
  {
    load_ids(0, ids_last);
    load_rows(kbase, 0, ids_last, st.k);        // stage 0: K(0)
    load_ids(1, ids_next);
  }
  store_stage(0, st);
  __syncthreads();

  auto step = [&](const int t) {
    if (t + 1 <= ntiles) {  // stage t+1: K(t+1) (ids one step ahead), V(t)
      int idk[PER_THREAD];
#pragma unroll
      for (int j = 0; j < PER_THREAD; ++j) idk[j] = ids_next[j];
      load_rows(kbase, t + 1, idk, st.k);
      load_rows(vbase, t, ids_last, st.v);
#pragma unroll
      for (int j = 0; j < PER_THREAD; ++j) ids_last[j] = idk[j];
      load_ids(t + 2, ids_next);
    }
    if (tile_live(t - 1)) values(t - 1, pb);
    if (tile_live(t)) {
      scores(t, sacc);
      softmax(t, sacc, pb);
    }
    if (t + 1 <= ntiles) store_stage(t + 1, st);
    __syncthreads();
  };
  for (int t = 0; t <= ntiles; ++t) step(t);

  // ---- normalise and store: lane (g, n) holds dims 16e + 4g + i of row n
  const bool bad = __syncthreads_or(bad_block ? 1 : 0) != 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float l = lsum[r];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = bad ? __builtin_nanf("") : 1.0f / l;
    const int rr = Rw + 16 * r + n;
    const int tok = rr / G;
    if (tok >= T) continue;
    const size_t orow = (size_t)(q0 + tok) * Hq + kvh * G + rr % G;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const size_t off = orow * D + 16 * e + 4 * g;
      const u32x2 w = {MM::pack(o[r][e][0] * inv, o[r][e][1] * inv),
                       MM::pack(o[r][e][2] * inv, o[r][e][3] * inv)};
      *(u32x2*)((char*)p.out + off * 2) = w;
    }
  }
}

}  // namespace pa
