/*
 * pagedattn.h -- C ABI of libpagedattn.so: single-token decode attention over
 * a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * The operations come from three pages on the KV cache:
 *   [guide] jovanaeducation.com/guides/l-is-2
 *   [notes] "KV cache: the engine behind fast LLM inference"
 *           (curiosity-9m6.pages.dev/notes/0043)
 *   [viz]   the KV-cache visualization page
 *           (cuuduongthancong.com/~galles/visualization/KVCache.html)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers named as device pointers must point to GPU memory on the current
 * HIP device; "host" pointers point to CPU memory.  Every device buffer is
 * owned by the caller: the library never allocates or frees memory, never
 * synchronizes, and keeps no state between calls except a thread-local error
 * message.  All GPU work is enqueued on `stream` (a hipStream_t; NULL is the
 * default stream) and calls return before it completes.
 *
 * Layouts (row-major, C order):
 *   k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim]
 *                      one contiguous block_size x head_dim tile per
 *                      (block, KV head)
 *   k_scale, v_scale : [num_blocks][num_kv_heads][block_size] fp16, quantized
 *                      (int8, fp8) caches only; int4: [...][block_size][head_dim/32]
 *   int4 k/v_cache   : [num_blocks][num_kv_heads][block_size][head_dim/2] bytes,
 *                      dim 2i in the low nibble of byte i, 2i+1 in the high
 *                      nibble, each stored as code + 8 (code in [-7, 7])
 *   block_tables     : int32 [num_seqs][max_blocks_per_seq]; entry j of row s
 *                      is the pool block holding positions [j*BS, (j+1)*BS)
 *                      of sequence s.  Entries past ceil(ctx/BS) are never read.
 *   context_lens     : int32 [num_seqs]; the number of cached positions of
 *                      each sequence, counting the token appended this step
 *   q, out           : [num_seqs][num_q_heads][head_dim]
 *   k_new, v_new     : [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping     : int64 [num_tokens]; slot = block * block_size + offset
 * Query head h reads KV head h / (num_q_heads / num_kv_heads) (grouped-query
 * attention: consecutive query heads share a KV head, [viz] "How much
 * memory").
 *
 * Supported: head_dim in {64, 128}; block_size in {4, 8, 16, 32}; element
 * formats fp32, fp16, bf16 (q, caches and out share one format), int8 or fp8
 * (E4M3) caches with fp16 q/out and per-(token, head) fp16 scales, and int4
 * caches with fp16 q/out and fp16 scales per (token, head, 32 dims).
 *
 * Errors: arguments are checked on the host before anything is enqueued.
 * A non-PA_OK status means nothing was enqueued (except PA_ERR_HIP, which
 * reports a launch failure); pa_last_error() then describes the problem.
 * Device data that breaks the contract cannot be checked on the host without
 * a synchronization; the kernels never read or write outside the buffers the
 * descriptor describes, and mark the affected output instead:
 *   - a context length < 0 or > max_blocks_per_seq * block_size, or a block
 *     id outside [0, num_blocks) among a sequence's first ceil(ctx/BS)
 *     entries, makes that sequence's output rows NaN;
 *   - a slot outside [0, num_blocks * block_size) is skipped by the appends
 *     (negative slots are padding by contract);
 *   - two tokens with the same slot in one append race: which row lands
 *     there is unspecified.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 4

typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_I8 = 3,
  PA_FP8 = 4, /* OCP fp8 E4M3 codes (1 sign, 4 exponent bits of bias 7, 3 fraction bits) */
  PA_I4 = 5   /* int4 codes, two per byte, a scale per 32 dims (layout below) */
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, negative size, Hq % Hkv != 0 ... */
  PA_ERR_UNSUPPORTED = 2, /* head_dim, block_size or dtype outside the list */
  PA_ERR_WORKSPACE = 3,   /* workspace smaller than pa_decode_workspace_bytes */
  PA_ERR_HIP = 4,         /* a HIP launch reported an error */
  PA_ERR_OUT_OF_BLOCKS = 5 /* the block pool cannot hold the request */
} pa_status;

/* Shape and element format of one layer's block pool (K and V alike). */
typedef struct {
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  int32_t dtype; /* pa_dtype of the cache elements */
} pa_cache_desc;

typedef void* pa_stream_t; /* a hipStream_t */

/* ---------------------------------------------------------------- slots */

/* Slot of each appended token: slot = block_tables[seq][pos / BS] * BS +
 * pos % BS, i.e. the position's block from the sequence's ordered block
 * table and the offset inside it ([viz] "PagedAttention: the cache in
 * blocks").  token_seq, token_pos: device int32 [num_tokens]; slot_mapping:
 * device int64 [num_tokens] (written).  A token whose seq or position falls
 * outside the table gets slot -1. */
pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t num_seqs, const int32_t* token_seq,
                          const int32_t* token_pos, int64_t num_tokens,
                          int32_t block_size, int64_t* slot_mapping,
                          pa_stream_t stream);

/* Decode-step slots: each sequence appends one token at position
 * context_lens[s] - 1 (the length already counts it; [notes] "What happens at
 * each decoding step", steps 2 and 4).  slot_mapping: device int64
 * [num_seqs].  Sequences with length 0 or a length past the table get -1. */
pa_status pa_decode_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t block_size, int64_t* slot_mapping,
                                 pa_stream_t stream);

/* Check a slot mapping before an append.  A slot names one position of one
 * block ([viz] "PagedAttention: the cache in blocks"), so no two tokens of
 * one append may name the same slot: the appends do not detect it (the
 * result is then one of the rows, unspecified which).  Writes *flags
 * (device int32, 4-byte aligned), in stream order: 0 when every slot is
 * negative (a pad) or in [0, pool_slots) and no slot >= 0 repeats; else
 * PA_SLOT_REPEATED (1) if some slot >= 0 repeats, | PA_SLOT_OUTSIDE_POOL (2)
 * if some slot >= pool_slots (the appends skip those).  Two kernels (the
 * flag is zeroed, then the slots are compared); nothing is synchronized and
 * nothing traps: read *flags when convenient.  Cost O(num_tokens^2 / 2)
 * compares.  pool_slots = num_blocks * block_size. */
#define PA_SLOT_REPEATED 1
#define PA_SLOT_OUTSIDE_POOL 2
pa_status pa_check_slot_mapping(const int64_t* slot_mapping, int64_t num_tokens,
                                int64_t pool_slots, int32_t* flags, pa_stream_t stream);

/* ---------------------------------------------------------------- append */

/* Store each new token's K and V rows into the pool at its slot, for every
 * KV head ([notes] step 4 "Append and repeat"; [guide] "How the cache turns
 * the loop cheap").  k_new, v_new: device [num_tokens][Hkv][D] in the cache's
 * format (fp32/fp16/bf16); k_cache, v_cache: device pools, updated in place.
 * Bit-exact copy.  Negative slots are skipped. */
pa_status pa_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                       int64_t num_tokens, void* k_cache, void* v_cache,
                       const pa_cache_desc* cache, pa_stream_t stream);

/* int8 cache ([notes] "How serving systems tame the cost", quantized KV
 * cache; the quantizer is this library's reading): for every (token, head)
 * row of fp16 values x,
 *   a = max |x|,  s = fp16_rne(fp32(a / 127)),
 *   code = clamp(rint_half_even(fp32(x / s)), -127, 127)   (0 when s == 0),
 * with IEEE binary32 divisions.  Codes go to k_cache/v_cache (device int8
 * pools, cache->dtype == PA_I8), s to k_scale/v_scale (device fp16
 * [NB][Hkv][BS]).  k_new, v_new: device fp16 [num_tokens][Hkv][D]. */
pa_status pa_kv_append_int8(const void* k_new, const void* v_new,
                            const int64_t* slot_mapping, int64_t num_tokens,
                            int8_t* k_cache, int8_t* v_cache, void* k_scale,
                            void* v_scale, const pa_cache_desc* cache,
                            pa_stream_t stream);

/* fp8 cache ([viz] "What the page leaves out" names 8- and 4-bit cache
 * quantization; the format and the quantizer are this library's reading):
 * the int8 scheme with OCP E4M3 codes,
 *   a = max |x|,  s = fp16_rne(fp32(a / 448)),
 *   code = the E4M3 value nearest fp32(x / s), ties to even, saturating at
 *          +-448 (0 when s == 0 or x is NaN; the NaN code is never stored).
 * Codes go to k_cache/v_cache (device byte pools, cache->dtype == PA_FP8),
 * s to k_scale/v_scale (device fp16 [NB][Hkv][BS]).  k_new, v_new: device
 * fp16 [num_tokens][Hkv][D]. */
pa_status pa_kv_append_fp8(const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int64_t num_tokens,
                           void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                           const pa_cache_desc* cache, pa_stream_t stream);

/* int4 cache (the 4-bit half of [viz] "What the page leaves out"'s "8-bit or
 * 4-bit"; groups and rounding are this library's reading): for every group of
 * 32 consecutive dims of a (token, head) row of fp16 values x,
 *   a = max |x|,  s = fp16_rne(fp32(a / 7)),
 *   code = clamp(rint_half_even(fp32(x / s)), -7, 7)   (0 when s == 0 or x is
 *   NaN), stored as the nibble code + 8.
 * Codes go to k_cache/v_cache (device bytes [NB][Hkv][BS][D/2],
 * cache->dtype == PA_I4), the group scales to k_scale/v_scale (device fp16
 * [NB][Hkv][BS][D/32]).  k_new, v_new: device fp16 [num_tokens][Hkv][D]. */
pa_status pa_kv_append_int4(const void* k_new, const void* v_new,
                            const int64_t* slot_mapping, int64_t num_tokens,
                            void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                            const pa_cache_desc* cache, pa_stream_t stream);

/* ---------------------------------------------------------------- attention */

/* Workspace the decode entry points need for this shape: fp32 partial
 * results (running max, sum and unnormalized output) of every context
 * partition.  partition_tokens = 0 picks the library's own plan, the one
 * pa_paged_decode_attention uses; pass the same value to the phase entry
 * points below.  Pure host arithmetic; returns 0 for an invalid shape or a
 * single-partition plan (which needs no workspace).  The workspace must be
 * 16-byte aligned (PA_ERR_INVALID_ARG otherwise).  Contents are scratch;
 * calls that overlap on one workspace race. */
size_t pa_decode_workspace_bytes(const pa_cache_desc* cache, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 int32_t partition_tokens);

/* The partition length (tokens) the library's plan picks for this shape,
 * a multiple of the tile length.  Pure host arithmetic; 0 if invalid. */
int32_t pa_decode_partition_tokens(const pa_cache_desc* cache, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_blocks_per_seq);

/* Decode attention for one new token per sequence: for every query head h,
 *   out[s][h] = softmax(q[s][h] . K_s^T * scale) . V_s
 * over the context_lens[s] cached rows of KV head h / G, reached through the
 * block table ([notes] "Concept" and step 3 "Attend against the cache";
 * [viz] "PagedAttention: the cache in blocks").  The softmax runs online
 * over the cache, tile by tile, never forming the score row in memory
 * ([guide] "Flash attention: don't build the giant matrix").  Long contexts
 * are split into partitions whose partials a second launch combines with the
 * log-sum-exp merge (pa_decode_partitions + pa_lse_merge).  q, out: device
 * [S][Hq][D] in the cache's format; fp32 accumulation; out rounded to
 * nearest-even.  A sequence with length 0 gets zeros.  workspace: device,
 * >= pa_decode_workspace_bytes(cache, S, Hq, max_blocks_per_seq, 0) bytes,
 * contents clobbered. */
pa_status pa_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, float scale, void* out,
                                    const pa_cache_desc* cache, void* workspace,
                                    size_t workspace_bytes, pa_stream_t stream);

/* The same over an int8 cache: keys and values are code * scale, with the
 * scales folded into the scores and the weights.  q, out: device fp16. */
pa_status pa_paged_decode_attention_int8(const void* q, const int8_t* k_cache,
                                         const int8_t* v_cache, const void* k_scale,
                                         const void* v_scale, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, float scale, void* out,
                                         const pa_cache_desc* cache, void* workspace,
                                         size_t workspace_bytes, pa_stream_t stream);

/* The same over an fp8 (E4M3) cache: keys and values are decode(code) *
 * scale, exact in binary32; q and out fp16. */
pa_status pa_paged_decode_attention_fp8(const void* q, const void* k_cache,
                                        const void* v_cache, const void* k_scale,
                                        const void* v_scale, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, float scale, void* out,
                                        const pa_cache_desc* cache, void* workspace,
                                        size_t workspace_bytes, pa_stream_t stream);

/* The same over an int4 cache: keys and values are code * (the scale of the
 * code's 32-dim group), exact in binary32; q and out fp16.  Runs on the
 * vector-ALU kernel at any group size. */
pa_status pa_paged_decode_attention_int4(const void* q, const void* k_cache,
                                         const void* v_cache, const void* k_scale,
                                         const void* v_scale, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, float scale, void* out,
                                         const pa_cache_desc* cache, void* workspace,
                                         size_t workspace_bytes, pa_stream_t stream);

/* One decode step for a fp32 / fp16 / bf16 cache: store each
 * sequence's new K and V rows (k_new, v_new: device [S][Hkv][D] in the
 * cache's format) at position context_lens[s] - 1, i.e. at slot
 * block_tables[s][pos / BS] * BS + pos % BS ([notes] steps 2-4: project the
 * new token, attend, append; [guide] "How the cache turns the loop cheap"),
 * and compute the same attention as pa_paged_decode_attention over all
 * context_lens[s] rows, the new one included.  The append happens inside the
 * attention launch (each workgroup whose partition holds the new position
 * stores the rows, then reads them back through the pool); the merge of a
 * multi-partition plan is the second launch.  Equivalent to
 * pa_decode_slot_mapping + pa_kv_append + pa_paged_decode_attention.
 * Sequences of length 0 append nothing.
 * k_cache, v_cache are updated in place; other arguments as above. */
pa_status pa_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         float scale, void* out, const pa_cache_desc* cache, void* workspace,
                         size_t workspace_bytes, pa_stream_t stream);

/* pa_decode_step without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The partials of a multi-partition plan go to a
 * static device array of the library (32 MiB per device, held by every
 * device the library runs on until the process ends); no call allocates or
 * frees memory.  Shapes whose partials exceed it return PA_ERR_WORKSPACE
 * (use pa_decode_step).  Every call on one device shares that device's
 * array: calls that overlap on one device race (enqueue them on one stream,
 * or order the streams).  Nothing in the array needs to start at zero.
 * Arguments, results and errors otherwise as pa_decode_step. */
pa_status pa_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                 void* k_cache, void* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, float scale, void* out,
                                 const pa_cache_desc* cache, pa_stream_t stream);

/* Phase 1 of the above with an explicit partition length, or 0 for the
 * plan's.  The length must be a positive multiple of the tile, which is
 * max(block_size, 1024 / (head_dim * bytes per cache element)) positions
 * (PA_ERR_INVALID_ARG otherwise).  Each workgroup attends
 * over one partition of one sequence's context for one KV head's query
 * heads and writes its partial (max, sum, unnormalized output) into the
 * workspace.  When the partition covers the whole table width
 * (partition_tokens >= max_blocks_per_seq * BS) the result is final and is
 * written to out directly; otherwise pa_lse_merge must follow.  k_scale and
 * v_scale are used only for a quantized (int8, fp8, int4) cache (NULL otherwise). */
pa_status pa_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                               const void* k_scale, const void* v_scale,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, float scale, int32_t partition_tokens,
                               void* out, const pa_cache_desc* cache, void* workspace,
                               size_t workspace_bytes, pa_stream_t stream);

/* Phase 1 of pa_decode_step with an explicit partition length (as for
 * pa_decode_partitions): the append at context_lens[s] - 1 and the
 * partitions' attention, in one launch. */
pa_status pa_decode_step_partitions(const void* q, const void* k_new, const void* v_new,
                                    void* k_cache, void* v_cache, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, float scale,
                                    int32_t partition_tokens, void* out,
                                    const pa_cache_desc* cache, void* workspace,
                                    size_t workspace_bytes, pa_stream_t stream);

/* One decode step for a quantized (int8, fp8 or int4) cache: the
 * quantizing append of pa_kv_append_int8 / _fp8 / _int4 (by cache->dtype) of
 * each sequence's new K and V rows (k_new, v_new: device fp16 [S][Hkv][D])
 * at position context_lens[s] - 1, codes to k_cache/v_cache and scales to
 * k_scale/v_scale in those entry points' layouts, followed by the attention
 * of pa_paged_decode_attention_int8 / _fp8 / _int4 over all context_lens[s]
 * rows, the new one included ([notes] steps 2-4 and "Quantized KV cache";
 * [viz] "What the page leaves out").  As in pa_decode_step, the append
 * happens inside the attention launch, and a multi-partition plan's merge is
 * the second launch.  Stores the same codes and scales, bit for bit, as
 * pa_decode_slot_mapping + the quantizing append, and gives the same output
 * as the attention call after them.  q, out: device fp16.  Caches and
 * scales are updated in place; other arguments as for pa_decode_step. */
pa_status pa_decode_step_quant(const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, float scale, void* out,
                               const pa_cache_desc* cache, void* workspace,
                               size_t workspace_bytes, pa_stream_t stream);

/* Phase 1 of pa_decode_step_quant with an explicit partition length (as for
 * pa_decode_partitions): the quantizing append at context_lens[s] - 1 and the
 * partitions' attention, in one launch; pa_lse_merge (out_dtype PA_F16)
 * follows a multi-partition plan. */
pa_status pa_decode_step_partitions_quant(const void* q, const void* k_new, const void* v_new,
                                          void* k_cache, void* v_cache, void* k_scale,
                                          void* v_scale, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, float scale,
                                          int32_t partition_tokens, void* out,
                                          const pa_cache_desc* cache, void* workspace,
                                          size_t workspace_bytes, pa_stream_t stream);

/* Phase 2: log-sum-exp merge of the partitions' partials into out
 * (max M = max_p m_p; out = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p),
 * which is the same softmax-weighted sum a single pass gives ([guide]
 * "Flash attention": tiling leaves the math unchanged).  Arguments as for
 * pa_decode_partitions with the same partition_tokens; out_dtype is the
 * format of out (PA_F32, PA_F16 or PA_BF16).  workspace and out must be
 * 16-byte aligned (PA_ERR_INVALID_ARG otherwise). */
pa_status pa_lse_merge(const void* workspace, size_t workspace_bytes,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t partition_tokens, int32_t out_dtype, void* out,
                       pa_stream_t stream);

/* ---------------------------------------------------------------- gather */

/* Un-page every sequence to dense rows: a sequence's rows are those of the
 * blocks its table lists, in order, position pos at offset pos % BS of block
 * table[pos / BS] ([viz] "PagedAttention: the cache in blocks").  This is
 * the block-table gather the attention kernels do on the fly, exported so
 * that it can be checked byte for byte.  k_out[s][i][h][:] = row of
 * position i, for i < context_lens[s]; rows at or past the length are left
 * untouched.  k_out, v_out: device [num_seqs][max_blocks_per_seq * BS][Hkv]
 * [row bytes] in the cache's format (int8 / fp8 codes; int4: D/2 bytes of
 * packed codes).  For a quantized cache, k_scale/v_scale (the pools' fp16
 * scales) and k_scale_out/v_scale_out ([S][maxB*BS][Hkv] fp16, int4:
 * [S][maxB*BS][Hkv][D/32]) carry the scales along; the scale outputs may be
 * NULL to gather codes only.  Errors: PA_ERR_INVALID_ARG for a NULL pool,
 * table, length or output pointer or bad sizes.  Rows whose table entry lies
 * outside the pool, and every row of a sequence whose length is negative or
 * past the table, are left untouched (no fault).  num_seqs = 0 is a no-op. */
pa_status pa_gather_kv(const void* k_cache, const void* v_cache, const void* k_scale,
                       const void* v_scale, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t num_seqs, void* k_out, void* v_out, void* k_scale_out,
                       void* v_scale_out, const pa_cache_desc* cache, pa_stream_t stream);

/* ---------------------------------------------------------------- measurement */

/* HBM read-rate probe (a measurement export, not part of attention): src
 * (device, 16-byte aligned, `bytes` a positive multiple of 4096) is read once
 * as 4 KiB chunks -- the size of one fp16 (block, head) tile at block 16 and
 * head_dim 128 -- each by one wave with 16-byte non-temporal loads, in the
 * order chunk_order gives (device int32 [bytes / 4096], a permutation of the
 * chunk indices; entries outside the range are read as chunk 0) or in
 * sequence when chunk_order is NULL.  The loaded words are folded into one
 * value per thread, stored to sink[0] (device uint32) only if it equals a
 * fixed improbable constant, so that the reads cannot be elided.  Timing a
 * launch gives the practical read bandwidth of a sequential stream, or of a
 * random gather of tiles, that the attention kernels' rates can be compared
 * with.  PA_ERR_INVALID_ARG for a NULL src or sink or a bad size. */
pa_status pa_hbm_read_probe(const void* src, size_t bytes, const int32_t* chunk_order,
                            uint32_t* sink, pa_stream_t stream);

/* ---------------------------------------------------------------- sliding window */

/* Sliding-window decode attention ([viz] "What the page leaves out" names
 * sliding-window attention; the reading here: the newest token attends to
 * the last `window` positions of its sequence, [max(0, ctx - window), ctx)).
 * Otherwise as pa_paged_decode_attention, for every cache format: k_scale and
 * v_scale are used for an int8 or fp8 cache (q/out fp16) and ignored
 * otherwise.  window == 0 attends to the whole context; window < 0 is
 * PA_ERR_INVALID_ARG.  Positions before the window are never read, and
 * neither are the table entries of blocks wholly before it: a caller may
 * free those blocks and leave any value in their entries.  The workspace is
 * sized by pa_decode_window_workspace_bytes with the same window (the plan's
 * partitions follow the window's length). */
size_t pa_decode_window_workspace_bytes(const pa_cache_desc* cache, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_blocks_per_seq,
                                        int32_t window);
pa_status pa_paged_decode_attention_window(const void* q, const void* k_cache,
                                           const void* v_cache, const void* k_scale,
                                           const void* v_scale, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, float scale, int32_t window,
                                           void* out, const pa_cache_desc* cache,
                                           void* workspace, size_t workspace_bytes,
                                           pa_stream_t stream);

/* One decode step with a sliding window, for any cache format: the append
 * of pa_decode_step (fp32 / fp16 / bf16 caches: k_new, v_new in the cache's
 * format) or of pa_decode_step_quant (int8, fp8, int4: fp16 rows quantized
 * into codes and scales) at position context_lens[s] - 1, inside the
 * attention launch of pa_paged_decode_attention_window, which then attends
 * over the last `window` positions, the new one included ([notes] steps 2-4;
 * [viz] "What the page leaves out": sliding-window attention).  The merge of
 * a multi-partition plan is the second launch.  workspace: >=
 * pa_decode_window_workspace_bytes; k_scale, v_scale: NULL for unquantized
 * caches.  Other arguments and errors as for those entry points. */
pa_status pa_decode_step_window(const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, float scale, int32_t window, void* out,
                                const pa_cache_desc* cache, void* workspace,
                                size_t workspace_bytes, pa_stream_t stream);

/* ---------------------------------------------------------------- prefill */

/* Causal attention of several query tokens per sequence over the paged cache:
 * prefill, which takes a whole prompt at once, and chunked prefill, which
 * takes it in pieces ([viz] "Without vs with the cache", "Prefill and decode
 * feel different").  Sequence s brings T_s = query_start[s+1] - query_start[s]
 * query tokens whose K and V rows are already stored as its last T_s cached
 * positions (append first, e.g. pa_kv_append with pa_slot_mapping), so its
 * query token i sits at position p = context_lens[s] - T_s + i and attends to
 * positions 0..p: a token never looks ahead ([viz] "The idea").  Tiles of the
 * score matrix stay on chip ([guide] "Flash attention").
 *   q, out         : device [query_start[num_seqs]][num_q_heads][head_dim],
 *                    fp16 or bf16, the cache's format; out fully written for
 *                    every token of a chunk no longer than max_query_len
 *   query_start    : device int32 [num_seqs + 1], non-decreasing, from 0
 *   context_lens   : device int32 [num_seqs], each >= its chunk length
 *   max_query_len  : host bound on every T_s (sizes the grid); tokens of a
 *                    longer chunk are not computed
 * Only fp16 and bf16 caches (head_dim 64 or 128, any supported block size);
 * PA_ERR_UNSUPPORTED when max_query_len * (num_q_heads / num_kv_heads) query
 * rows need more than 65535 row tiles of 256 (16.7 M rows).
 * A sequence whose context length is below its chunk length or above
 * max_blocks_per_seq * block_size gets NaN rows, as does one whose needed
 * table entries name a block outside the pool. */
pa_status pa_paged_prefill_attention(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* query_start, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t max_query_len,
                                     int32_t num_q_heads, float scale, void* out,
                                     const pa_cache_desc* cache, pa_stream_t stream);

/* ---------------------------------------------------------------- block pool */

/* Host-side owner of one block pool: which pool block holds which positions
 * of which sequence.  It produces the block tables, context lengths and slot
 * numbers the calls above consume, following the paging rules of [viz]
 * "PagedAttention: the cache in blocks" and [guide] "Paging":
 *   - a sequence takes a new block only when its last block is full, so at
 *     most one of its blocks is partly filled;
 *   - a freed sequence returns its blocks to the pool at once;
 *   - a fork shares its parent's blocks for a prefix, by reference count;
 *   - a block held by more than one sequence is copied only when one of them
 *     writes into it: the writer moves onto a fresh block, and the append
 *     reports the (source, destination) pair, which the caller must copy with
 *     pa_copy_blocks in every layer's pool before appending to the slots.
 * The manager lives in host memory only and makes no HIP call.  One manager
 * serves all layers of a model (they share the tables).  It is not
 * thread-safe: calls on one manager must not overlap.  Sequence ids are small
 * integers chosen by the manager; the id of a freed sequence may be reused.
 * Which free block is handed out is unspecified. */
typedef struct pa_block_manager pa_block_manager;

/* A pool of num_blocks blocks of block_size slots (block_size in {4, 8, 16,
 * 32}).  *out receives the manager, or NULL on failure. */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);  /* NULL is ignored */

/* A new, empty sequence; its id goes to *seq. */
pa_status pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq);

/* A new sequence holding the first prefix_tokens positions of parent (all of
 * them when prefix_tokens < 0): it shares the parent's first
 * ceil(prefix_tokens / block_size) blocks and takes no block of its own. */
pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t prefix_tokens,
                     int32_t* child);

/* Ends a sequence; every block it alone held is free again. */
pa_status pa_bm_free_sequence(pa_block_manager* bm, int32_t seq);

/* Reserves num_tokens[r] new positions at the end of sequence seqs[r], for
 * each request r (host arrays; a sequence at most once).  slots (host int64,
 * capacity max_slots) receives the slot of every new position, request by
 * request, in position order -- the slot_mapping of the append that follows.
 * copies (host int32 [max_copies][2]) receives (source, destination) block
 * pairs to copy before that append, and *num_copies their number (at most one
 * per request).  All or nothing: PA_ERR_OUT_OF_BLOCKS when the free blocks
 * do not cover the request, PA_ERR_INVALID_ARG when a buffer is too small;
 * then nothing changes. */
pa_status pa_bm_append(pa_block_manager* bm, const int32_t* seqs, const int32_t* num_tokens,
                       int32_t num_requests, int64_t* slots, int64_t max_slots,
                       int32_t* copies, int32_t max_copies, int32_t* num_copies);

/* Host int32 block_tables [num_seqs][max_blocks_per_seq] (entries past a
 * sequence's blocks set to -1) and, if context_lens is not NULL, host int32
 * context_lens [num_seqs] of the listed sequences. */
pa_status pa_bm_block_tables(const pa_block_manager* bm, const int32_t* seqs, int32_t num_seqs,
                             int32_t max_blocks_per_seq, int32_t* block_tables,
                             int32_t* context_lens);

int32_t pa_bm_num_free_blocks(const pa_block_manager* bm);           /* -1 if bm is NULL */
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block);  /* -1 out of range */
int32_t pa_bm_sequence_length(const pa_block_manager* bm, int32_t seq); /* -1 if not live */

/* Copies whole blocks inside one pool, for the copy-on-write of shared blocks
 * ([viz] "PagedAttention: the cache in blocks": a shared block is copied when
 * one holder writes into it).  block_pairs: device int32 [num_pairs][2] of
 * (source, destination) block ids; every KV head's rows of the source block
 * are copied to the destination block, in k_cache and v_cache, and for an
 * int8, fp8 or int4 cache also in k_scale and v_scale (NULL otherwise).  Pairs with an id
 * outside [0, num_blocks) are skipped.  A destination must not be the source
 * or the destination of another pair in the same call. */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                         const int32_t* block_pairs, int32_t num_pairs,
                         const pa_cache_desc* cache, pa_stream_t stream);

/* ---------------------------------------------------------------- misc */

const char* pa_status_string(pa_status status); /* static string */
const char* pa_last_error(void);  /* thread-local detail of the last failure */
int32_t pa_abi_version(void);     /* PA_ABI_VERSION */

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
