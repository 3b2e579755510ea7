// kv_ops.h -- launchers of the slot, append and gather kernels (internal).
#pragma once

#include "device.h"

namespace pa {

hipError_t launch_slot_mapping(const int32_t* tables, int32_t max_blocks, int32_t num_seqs,
                               const int32_t* token_seq, const int32_t* token_pos,
                               int64_t num_tokens, int32_t block_size, int64_t* slots,
                               hipStream_t stream);
hipError_t launch_decode_slot_mapping(const int32_t* tables, int32_t max_blocks,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t block_size, int64_t* slots, hipStream_t stream);
// Flags of a slot mapping (bit 0 repeated slot, bit 1 slot >= pool_slots)
// into a device int32, zeroed first by the same launch sequence.
hipError_t launch_check_slots(const int64_t* slots, int64_t num_tokens, int64_t pool_slots,
                              int32_t* flags, hipStream_t stream);
hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slots,
                            int64_t num_tokens, void* k_cache, void* v_cache,
                            int32_t num_kv_heads, int32_t block_size, int32_t row_bytes,
                            int64_t pool_slots, hipStream_t stream);
// Quantizing append into an int8 (kind 0), fp8 E4M3 (1) or int4 (2) cache.
hipError_t launch_kv_append_quant(const void* k_new, const void* v_new, const int64_t* slots,
                                  int64_t num_tokens, void* k_cache, void* v_cache,
                                  void* k_scale, void* v_scale, int32_t num_kv_heads,
                                  int32_t block_size, int32_t head_dim, int64_t pool_slots,
                                  int kind, hipStream_t stream);
hipError_t launch_gather_kv(const void* k_cache, const void* v_cache, const void* k_scale,
                            const void* v_scale, const int32_t* tables, int32_t max_blocks,
                            const int32_t* context_lens, int32_t num_seqs, void* k_out,
                            void* v_out, void* k_scale_out, void* v_scale_out,
                            int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                            int32_t row_bytes, int32_t scales_per_row, hipStream_t stream);
hipError_t launch_hbm_read_probe(const void* src, size_t bytes, const int32_t* chunk_order,
                                 uint32_t* sink, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                              const int32_t* pairs, int32_t num_pairs, int32_t num_blocks,
                              int32_t num_kv_heads, int32_t block_size, int32_t row_bytes,
                              int32_t scales_per_row, hipStream_t stream);

// Log-sum-exp merge of partition partials (lse_merge.hip).
// window > 0: partials are stored by window slot (slot 0 starts at the tile,
// of `tile` positions, holding the window's first position).
hipError_t launch_lse_merge(const float* part_ml, const float* part_o,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t head_dim, int32_t max_tokens, int32_t part_tokens,
                            int32_t num_parts, int32_t window, int32_t tile, int32_t out_fmt,
                            void* out, hipStream_t stream);

}  // namespace pa
