// api.cpp -- the C ABI of libpagedattn.so: argument checks, the decode plan
// and kernel dispatch.  Declarations and their contracts: include/pagedattn.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pagedattn.h"
#include "decode_dispatch.h"
#include "decode_plan.h"
#include "prefill_dispatch.h"
#include "kv_ops.h"
#include "noalloc.h"
#include "status.h"

namespace pa {

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

}  // namespace pa

namespace {

using pa::fail;
using pa::g_last_error;

pa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

using pa::Plan;
using pa::check_cache;
using pa::elem_bytes;
using pa::make_plan;
using pa::quantized;
using pa::row_bytes;
using pa::scales_per_row;
using pa::supported_block;
using pa::supported_dim;

pa_status run_partitions(const void* q, const void* k_cache, const void* v_cache,
                         const void* k_scale, const void* v_scale, const int32_t* block_tables,
                         int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_q_heads, float scale, void* out, const pa_cache_desc* cache,
                         const Plan& plan, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, const void* k_new = nullptr,
                         const void* v_new = nullptr, int32_t window = 0) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (quantized(cache->dtype) && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARG, "a quantized cache needs k_scale and v_scale");
  if (plan.num_parts > 1 && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes,
                plan.ws_bytes);
  if (plan.num_parts > 1 && ((uintptr_t)workspace & 15) != 0)
    return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  pa::DecodeParams p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = (const uint16_t*)k_scale;
  p.v_scale = (const uint16_t*)v_scale;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.part_ml = plan.num_parts > 1 ? (float*)workspace : nullptr;
  p.part_o = plan.num_parts > 1 ? (float*)((char*)workspace + plan.o_offset) : nullptr;
  p.max_blocks = max_blocks;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cache->num_kv_heads;
  p.num_blocks = cache->num_blocks;
  p.group = num_q_heads / cache->num_kv_heads;
  p.head_chunks = plan.chunks;
  p.part_tokens = plan.part_tokens;
  p.num_parts = plan.num_parts;
  p.scale_log2 = scale * pa::kLog2e;
  p.k_new = k_new;
  p.v_new = v_new;
  p.window = window;
  p.tile = plan.tile;
  p.pair = plan.pair ? 1 : 0;
  p.num_seqs = num_seqs;
  hipError_t e;
  const int D = cache->head_dim, BS = cache->block_size;
  if (plan.mfma) {
    switch (cache->dtype) {
      case PA_F16: e = pa::launch_mfma_f16(p, D, BS, plan.gc, num_seqs, stream); break;
      case PA_BF16: e = pa::launch_mfma_bf16(p, D, BS, plan.gc, num_seqs, stream); break;
      case PA_I8: e = pa::launch_mfma_i8(p, D, BS, plan.gc, num_seqs, stream); break;
      case PA_FP8: e = pa::launch_mfma_fp8(p, D, BS, plan.gc, num_seqs, stream); break;
      case PA_I4: e = pa::launch_mfma_i4(p, D, BS, plan.gc, num_seqs, stream); break;
      default: return fail(PA_ERR_UNSUPPORTED, "dtype %d", cache->dtype);
    }
    return hip_status(e, "decode partitions launch");
  }
  switch (cache->dtype) {
    case PA_F32: e = pa::launch_decode_f32(p, cache->head_dim, cache->block_size, plan.gc, num_seqs, stream); break;
    case PA_F16: e = pa::launch_decode_f16(p, cache->head_dim, cache->block_size, plan.gc, num_seqs, stream); break;
    case PA_BF16: e = pa::launch_decode_bf16(p, cache->head_dim, cache->block_size, plan.gc, num_seqs, stream); break;
    case PA_I8: e = pa::launch_decode_i8(p, cache->head_dim, cache->block_size, plan.gc, num_seqs, stream); break;
    case PA_FP8: e = pa::launch_decode_fp8(p, cache->head_dim, cache->block_size, plan.gc, num_seqs, stream); break;
    case PA_I4: e = pa::launch_decode_i4(p, cache->head_dim, cache->block_size, plan.gc, num_seqs, stream); break;
    default: return fail(PA_ERR_UNSUPPORTED, "dtype %d", cache->dtype);
  }
  return hip_status(e, "decode partitions launch");
}

pa_status run_merge(const Plan& plan, const void* workspace, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_tokens,
                    int32_t out_dtype, void* out, hipStream_t stream, int32_t window = 0) {
  if (((uintptr_t)out & 15) != 0) return fail(PA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  const hipError_t e = pa::launch_lse_merge(
      (const float*)workspace, (const float*)((const char*)workspace + plan.o_offset),
      context_lens, num_seqs, num_q_heads, head_dim, max_tokens, plan.part_tokens,
      plan.num_parts, window, plan.tile, out_dtype, out, stream);
  return hip_status(e, "lse merge launch");
}

pa_status decode_common(const void* q, const void* k_cache, const void* v_cache,
                        const void* k_scale, const void* v_scale, const int32_t* block_tables,
                        int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs,
                        int32_t num_q_heads, float scale, void* out, const pa_cache_desc* cache,
                        void* workspace, size_t workspace_bytes, hipStream_t stream,
                        int32_t want_dtype, const void* k_new = nullptr,
                        const void* v_new = nullptr, int32_t window = 0) {
  Plan plan;
  pa_status st = make_plan(cache, num_seqs, num_q_heads, max_blocks, 0, &plan, window);
  if (st != PA_OK) return st;
  // want_dtype: the quantized format an entry point is for, or -1 for the
  // entry points of unquantized caches.
  if (want_dtype >= 0 ? cache->dtype != want_dtype : quantized(cache->dtype))
    return fail(PA_ERR_UNSUPPORTED,
                want_dtype == PA_I8    ? "the int8 entry point needs an int8 cache"
                : want_dtype == PA_FP8 ? "the fp8 entry point needs an fp8 cache"
                : want_dtype == PA_I4  ? "the int4 entry point needs an int4 cache"
                : cache->dtype == PA_I8 ? "int8 cache: use pa_paged_decode_attention_int8"
                : cache->dtype == PA_FP8 ? "fp8 cache: use pa_paged_decode_attention_fp8"
                                         : "int4 cache: use pa_paged_decode_attention_int4");
  if (num_seqs == 0) return PA_OK;
  st = run_partitions(q, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks,
                      context_lens, num_seqs, num_q_heads, scale, out, cache, plan, workspace,
                      workspace_bytes, stream, k_new, v_new, window);
  if (st != PA_OK || plan.num_parts == 1) return st;
  const int32_t out_dtype = quantized(cache->dtype) ? PA_F16 : cache->dtype;
  return run_merge(plan, workspace, context_lens, num_seqs, num_q_heads, cache->head_dim,
                   max_blocks * cache->block_size, out_dtype, out, stream, window);
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or format";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_HIP: return "HIP error";
    case PA_ERR_OUT_OF_BLOCKS: return "out of pool blocks";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t num_seqs, const int32_t* token_seq, const int32_t* token_pos,
                          int64_t num_tokens, int32_t block_size, int64_t* slot_mapping,
                          pa_stream_t stream) {
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative sizes or empty table");
  if (!supported_block(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported", block_size);
  if (num_tokens == 0) return PA_OK;
  if (!block_tables || !token_seq || !token_pos || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  return hip_status(pa::launch_slot_mapping(block_tables, max_blocks_per_seq, num_seqs, token_seq,
                                            token_pos, num_tokens, block_size, slot_mapping,
                                            (hipStream_t)stream),
                    "slot mapping launch");
}

pa_status pa_decode_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t block_size, int64_t* slot_mapping, pa_stream_t stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative sizes or empty table");
  if (!supported_block(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported", block_size);
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !context_lens || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  return hip_status(pa::launch_decode_slot_mapping(block_tables, max_blocks_per_seq, context_lens,
                                                   num_seqs, block_size, slot_mapping,
                                                   (hipStream_t)stream),
                    "decode slot mapping launch");
}

pa_status pa_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                       int64_t num_tokens, void* k_cache, void* v_cache,
                       const pa_cache_desc* cache, pa_stream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (quantized(cache->dtype))
    return fail(PA_ERR_UNSUPPORTED, "quantized cache: use pa_kv_append_int8 or pa_kv_append_fp8");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %lld < 0", (long long)num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  const int32_t row_bytes = cache->head_dim * elem_bytes(cache->dtype);
  return hip_status(pa::launch_kv_append(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache,
                                         cache->num_kv_heads, cache->block_size, row_bytes,
                                         (int64_t)cache->num_blocks * cache->block_size,
                                         (hipStream_t)stream),
                    "kv_append launch");
}

namespace {

pa_status kv_append_quantized(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                              int64_t num_tokens, void* k_cache, void* v_cache, void* k_scale,
                              void* v_scale, const pa_cache_desc* cache, int32_t want,
                              hipStream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (cache->dtype != want)
    return fail(PA_ERR_UNSUPPORTED, want == PA_I8    ? "pa_kv_append_int8 needs an int8 cache"
                                    : want == PA_FP8 ? "pa_kv_append_fp8 needs an fp8 cache"
                                                     : "pa_kv_append_int4 needs an int4 cache");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %lld < 0", (long long)num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  return hip_status(pa::launch_kv_append_quant(k_new, v_new, slot_mapping, num_tokens, k_cache,
                                               v_cache, k_scale, v_scale, cache->num_kv_heads,
                                               cache->block_size, cache->head_dim,
                                               (int64_t)cache->num_blocks * cache->block_size,
                                               want == PA_I8 ? 0 : want == PA_FP8 ? 1 : 2,
                                               stream),
                    "quantizing append launch");
}

}  // namespace

pa_status pa_kv_append_int8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                            int64_t num_tokens, int8_t* k_cache, int8_t* v_cache, void* k_scale,
                            void* v_scale, const pa_cache_desc* cache, pa_stream_t stream) {
  return kv_append_quantized(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, k_scale,
                             v_scale, cache, PA_I8, (hipStream_t)stream);
}

pa_status pa_kv_append_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                           int64_t num_tokens, void* k_cache, void* v_cache, void* k_scale,
                           void* v_scale, const pa_cache_desc* cache, pa_stream_t stream) {
  return kv_append_quantized(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, k_scale,
                             v_scale, cache, PA_FP8, (hipStream_t)stream);
}

size_t pa_decode_workspace_bytes(const pa_cache_desc* cache, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 int32_t partition_tokens) {
  Plan plan;
  if (make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &plan) != PA_OK)
    return 0;
  return plan.ws_bytes;
}

int32_t pa_decode_partition_tokens(const pa_cache_desc* cache, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_blocks_per_seq) {
  Plan plan;
  if (make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, 0, &plan) != PA_OK) return 0;
  return plan.part_tokens;
}

pa_status pa_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, float scale, void* out,
                                    const pa_cache_desc* cache, void* workspace,
                                    size_t workspace_bytes, pa_stream_t stream) {
  return decode_common(q, k_cache, v_cache, nullptr, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, out, cache, workspace,
                       workspace_bytes, (hipStream_t)stream, -1);
}

pa_status pa_paged_decode_attention_int8(const void* q, const int8_t* k_cache,
                                         const int8_t* v_cache, const void* k_scale,
                                         const void* v_scale, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, float scale, void* out,
                                         const pa_cache_desc* cache, void* workspace,
                                         size_t workspace_bytes, pa_stream_t stream) {
  return decode_common(q, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, out, cache, workspace,
                       workspace_bytes, (hipStream_t)stream, PA_I8);
}

size_t pa_decode_window_workspace_bytes(const pa_cache_desc* cache, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_blocks_per_seq,
                                        int32_t window) {
  Plan plan;
  if (make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, 0, &plan, window) != PA_OK)
    return 0;
  return plan.ws_bytes;
}

pa_status pa_paged_decode_attention_window(const void* q, const void* k_cache,
                                           const void* v_cache, const void* k_scale,
                                           const void* v_scale, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, float scale, int32_t window,
                                           void* out, const pa_cache_desc* cache,
                                           void* workspace, size_t workspace_bytes,
                                           pa_stream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "window %d < 0", window);
  return decode_common(q, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, out, cache, workspace,
                       workspace_bytes, (hipStream_t)stream,
                       quantized(cache->dtype) ? cache->dtype : -1, nullptr, nullptr, window);
}

pa_status pa_kv_append_int4(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                            int64_t num_tokens, void* k_cache, void* v_cache, void* k_scale,
                            void* v_scale, const pa_cache_desc* cache, pa_stream_t stream) {
  return kv_append_quantized(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, k_scale,
                             v_scale, cache, PA_I4, (hipStream_t)stream);
}

pa_status pa_paged_decode_attention_int4(const void* q, const void* k_cache,
                                         const void* v_cache, const void* k_scale,
                                         const void* v_scale, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, float scale, void* out,
                                         const pa_cache_desc* cache, void* workspace,
                                         size_t workspace_bytes, pa_stream_t stream) {
  return decode_common(q, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, out, cache, workspace,
                       workspace_bytes, (hipStream_t)stream, PA_I4);
}

pa_status pa_paged_decode_attention_fp8(const void* q, const void* k_cache,
                                        const void* v_cache, const void* k_scale,
                                        const void* v_scale, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, float scale, void* out,
                                        const pa_cache_desc* cache, void* workspace,
                                        size_t workspace_bytes, pa_stream_t stream) {
  return decode_common(q, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, out, cache, workspace,
                       workspace_bytes, (hipStream_t)stream, PA_FP8);
}

pa_status pa_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                               const void* k_scale, const void* v_scale,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, float scale, int32_t partition_tokens,
                               void* out, const pa_cache_desc* cache, void* workspace,
                               size_t workspace_bytes, pa_stream_t stream) {
  Plan plan;
  pa_status st = make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &plan);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  return run_partitions(q, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                        context_lens, num_seqs, num_q_heads, scale, out, cache, plan, workspace,
                        workspace_bytes, (hipStream_t)stream);
}

pa_status pa_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         float scale, void* out, const pa_cache_desc* cache, void* workspace,
                         size_t workspace_bytes, pa_stream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (quantized(cache->dtype))
    return fail(PA_ERR_UNSUPPORTED,
                "quantized cache: use pa_decode_step_quant");
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_INVALID_ARG, "NULL k_new / v_new");
  return decode_common(q, k_cache, v_cache, nullptr, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, out, cache, workspace,
                       workspace_bytes, (hipStream_t)stream, -1, k_new, v_new);
}

pa_status pa_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                 void* k_cache, void* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, float scale, void* out,
                                 const pa_cache_desc* cache, pa_stream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (quantized(cache->dtype))
    return fail(PA_ERR_UNSUPPORTED, "quantized cache: pa_decode_step_noalloc takes 16/32-bit caches");
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_INVALID_ARG, "NULL k_new / v_new");
  Plan plan;
  st = make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, 0, &plan);
  if (st != PA_OK) return st;
  if (plan.ws_bytes > pa::kNoAllocScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "this shape's partials need %zu bytes, above the %zu-byte static scratch of "
                "pa_decode_step_noalloc: use pa_decode_step with a workspace",
                plan.ws_bytes, pa::kNoAllocScratchBytes);
  void* ws = nullptr;
  if (num_seqs > 0 && plan.num_parts > 1) {
    const hipError_t e = pa::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "static scratch address");
  }
  return decode_common(q, k_cache, v_cache, nullptr, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, out, cache, ws,
                       ws ? pa::kNoAllocScratchBytes : 0, (hipStream_t)stream, -1, k_new, v_new);
}

pa_status pa_decode_step_partitions(const void* q, const void* k_new, const void* v_new,
                                    void* k_cache, void* v_cache, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, float scale,
                                    int32_t partition_tokens, void* out,
                                    const pa_cache_desc* cache, void* workspace,
                                    size_t workspace_bytes, pa_stream_t stream) {
  Plan plan;
  pa_status st = make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &plan);
  if (st != PA_OK) return st;
  if (quantized(cache->dtype))
    return fail(PA_ERR_UNSUPPORTED,
                "quantized cache: use pa_decode_step_partitions_quant");
  if (num_seqs == 0) return PA_OK;
  if (!k_new || !v_new) return fail(PA_ERR_INVALID_ARG, "NULL k_new / v_new");
  return run_partitions(q, k_cache, v_cache, nullptr, nullptr, block_tables, max_blocks_per_seq,
                        context_lens, num_seqs, num_q_heads, scale, out, cache, plan, workspace,
                        workspace_bytes, (hipStream_t)stream, k_new, v_new);
}

pa_status pa_decode_step_quant(const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, float scale, void* out,
                               const pa_cache_desc* cache, void* workspace,
                               size_t workspace_bytes, pa_stream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (!quantized(cache->dtype))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_step_quant needs an int8, fp8 or int4 cache");
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_INVALID_ARG, "NULL k_new / v_new");
  return decode_common(q, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, out, cache, workspace,
                       workspace_bytes, (hipStream_t)stream, cache->dtype, k_new, v_new);
}

pa_status pa_decode_step_partitions_quant(const void* q, const void* k_new, const void* v_new,
                                          void* k_cache, void* v_cache, void* k_scale,
                                          void* v_scale, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, float scale,
                                          int32_t partition_tokens, void* out,
                                          const pa_cache_desc* cache, void* workspace,
                                          size_t workspace_bytes, pa_stream_t stream) {
  Plan plan;
  pa_status st = make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &plan);
  if (st != PA_OK) return st;
  if (!quantized(cache->dtype))
    return fail(PA_ERR_UNSUPPORTED,
                "pa_decode_step_partitions_quant needs an int8, fp8 or int4 cache");
  if (num_seqs == 0) return PA_OK;
  if (!k_new || !v_new) return fail(PA_ERR_INVALID_ARG, "NULL k_new / v_new");
  return run_partitions(q, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                        context_lens, num_seqs, num_q_heads, scale, out, cache, plan, workspace,
                        workspace_bytes, (hipStream_t)stream, k_new, v_new);
}

pa_status pa_lse_merge(const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                       int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_tokens,
                       int32_t out_dtype, void* out, pa_stream_t stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || partition_tokens <= 0)
    return fail(PA_ERR_INVALID_ARG, "bad sizes");
  if (!supported_dim(head_dim)) return fail(PA_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (!supported_block(block_size)) return fail(PA_ERR_UNSUPPORTED, "block_size %d", block_size);
  if (out_dtype != PA_F32 && out_dtype != PA_F16 && out_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "block table width x block size exceeds 2^31 positions");
  Plan plan;
  plan.part_tokens = partition_tokens;
  const int64_t max_tok = (int64_t)max_blocks_per_seq * block_size;
  plan.num_parts = (int32_t)((max_tok + partition_tokens - 1) / partition_tokens);
  if (plan.num_parts <= 1)
    return fail(PA_ERR_INVALID_ARG, "a single partition is final already; nothing to merge");
  size_workspace(plan, num_seqs, num_q_heads, head_dim);
  if (num_seqs == 0) return PA_OK;
  if (!workspace || !context_lens || !out) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  if (workspace_bytes < plan.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, plan.ws_bytes);
  if (((uintptr_t)workspace & 15) != 0)
    return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return run_merge(plan, workspace, context_lens, num_seqs, num_q_heads, head_dim, (int32_t)max_tok,
                   out_dtype, out, (hipStream_t)stream);
}

pa_status pa_check_slot_mapping(const int64_t* slot_mapping, int64_t num_tokens,
                                int64_t pool_slots, int32_t* flags, pa_stream_t stream) {
  if (num_tokens < 0 || pool_slots <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_tokens %lld < 0 or pool_slots %lld <= 0",
                (long long)num_tokens, (long long)pool_slots);
  if (!flags || (num_tokens > 0 && !slot_mapping)) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  if (((uintptr_t)flags & 3) != 0) return fail(PA_ERR_INVALID_ARG, "flags must be 4-byte aligned");
  if ((uint64_t)(num_tokens + 255) / 256 > 0x7fffffffu)
    return fail(PA_ERR_UNSUPPORTED, "%lld tokens: too many for one check", (long long)num_tokens);
  return hip_status(pa::launch_check_slots(slot_mapping, num_tokens, pool_slots, flags,
                                           (hipStream_t)stream),
                    "slot check launch");
}

pa_status pa_gather_kv(const void* k_cache, const void* v_cache, const void* k_scale,
                       const void* v_scale, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                       void* k_out, void* v_out, void* k_scale_out, void* v_scale_out,
                       const pa_cache_desc* cache, pa_stream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "bad sizes");
  if (num_seqs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_tables || !context_lens || !k_out || !v_out)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  const int32_t rbytes = row_bytes(cache);
  const bool i8 = quantized(cache->dtype);
  return hip_status(pa::launch_gather_kv(k_cache, v_cache, i8 ? k_scale : nullptr,
                                         i8 ? v_scale : nullptr, block_tables, max_blocks_per_seq,
                                         context_lens, num_seqs, k_out, v_out,
                                         i8 ? k_scale_out : nullptr, i8 ? v_scale_out : nullptr,
                                         cache->num_blocks, cache->num_kv_heads,
                                         cache->block_size, rbytes, scales_per_row(cache),
                                         (hipStream_t)stream),
                    "gather launch");
}

pa_status pa_hbm_read_probe(const void* src, size_t bytes, const int32_t* chunk_order,
                            uint32_t* sink, pa_stream_t stream) {
  if (!src || !sink) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  if (bytes == 0 || bytes % 4096 != 0 || ((uintptr_t)src & 15) != 0)
    return fail(PA_ERR_INVALID_ARG, "probe buffer of %zu bytes must be a positive multiple of 4096, "
                "16-byte aligned", bytes);
  return hip_status(pa::launch_hbm_read_probe(src, bytes, chunk_order, sink, (hipStream_t)stream),
                    "read probe launch");
}

pa_status pa_decode_step_window(const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, float scale, int32_t window, void* out,
                                const pa_cache_desc* cache, void* workspace,
                                size_t workspace_bytes, pa_stream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "window %d < 0", window);
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_INVALID_ARG, "NULL k_new / v_new");
  return decode_common(q, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, out, cache, workspace,
                       workspace_bytes, (hipStream_t)stream,
                       quantized(cache->dtype) ? cache->dtype : -1, k_new, v_new, window);
}

pa_status pa_paged_prefill_attention(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* query_start, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t max_query_len,
                                     int32_t num_q_heads, float scale, void* out,
                                     const pa_cache_desc* cache, pa_stream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (cache->dtype != PA_F16 && cache->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "prefill attention takes fp16 or bf16 caches (dtype %d)",
                cache->dtype);
  if (num_seqs < 0 || max_query_len < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "bad sizes (seqs %d, max_query_len %d, max_blocks %d, "
                "q heads %d)", num_seqs, max_query_len, max_blocks_per_seq, num_q_heads);
  if (num_q_heads % cache->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "%d query heads do not divide over %d KV heads",
                num_q_heads, cache->num_kv_heads);
  if (!(scale > 0.0f))
    return fail(PA_ERR_INVALID_ARG, "prefill scale must be positive (got %g)", (double)scale);
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (num_seqs > 65535 || cache->num_kv_heads > 65535)
    return fail(PA_ERR_UNSUPPORTED, "more than 65535 sequences or KV heads in one launch");
  if (!q || !k_cache || !v_cache || !block_tables || !query_start || !context_lens || !out)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  pa::PrefillParams p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.query_start = query_start;
  p.context_lens = context_lens;
  p.out = out;
  p.max_blocks = max_blocks_per_seq;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cache->num_kv_heads;
  p.num_blocks = cache->num_blocks;
  p.group = num_q_heads / cache->num_kv_heads;
  p.scale_log2 = scale * pa::kLog2e;
  // 256 query rows per workgroup once the chunk fills them; 64 for short
  // chunks, whose rows would otherwise mostly be padding.
  const int64_t rows = (int64_t)max_query_len * p.group;
  const pa::PrefillShape shape = pa::prefill_shape(cache->head_dim, rows);
  const int64_t row_tiles = (rows + shape.rows() - 1) / shape.rows();
  if (row_tiles > 65535)
    return fail(PA_ERR_UNSUPPORTED, "chunk of %d tokens x %d heads per KV head needs %lld row "
                "tiles, more than 65535", max_query_len, p.group, (long long)row_tiles);
  const hipError_t e =
      cache->dtype == PA_F16
          ? pa::launch_prefill_f16(p, cache->head_dim, cache->block_size, shape, (int)row_tiles,
                                   num_seqs, (hipStream_t)stream)
          : pa::launch_prefill_bf16(p, cache->head_dim, cache->block_size, shape,
                                    (int)row_tiles, num_seqs, (hipStream_t)stream);
  return hip_status(e, "prefill launch");
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                         const int32_t* block_pairs, int32_t num_pairs,
                         const pa_cache_desc* cache, pa_stream_t stream) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  const bool i8 = quantized(cache->dtype);
  if (!k_cache || !v_cache || !block_pairs || (i8 && (!k_scale || !v_scale)))
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  const int32_t rbytes = row_bytes(cache);
  if ((int64_t)cache->num_kv_heads * cache->block_size * rbytes > ((int64_t)1 << 29))
    return fail(PA_ERR_UNSUPPORTED, "blocks above 512 MiB per tensor");
  return hip_status(pa::launch_copy_blocks(k_cache, v_cache, i8 ? k_scale : nullptr,
                                           i8 ? v_scale : nullptr, block_pairs, num_pairs,
                                           cache->num_blocks, cache->num_kv_heads,
                                           cache->block_size, rbytes, scales_per_row(cache),
                                           (hipStream_t)stream),
                    "copy_blocks launch");
}

}  // extern "C"
