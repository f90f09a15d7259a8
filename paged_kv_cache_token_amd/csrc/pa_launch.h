// pa_launch.h -- host-side entry points of the kernel files, called by the
// C ABI (pa_api.hip).  Kept apart from pa_internal.h, which holds what the
// kernels themselves are built from.
#pragma once

#include "pa_internal.h"

namespace pa {

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* cu_seqlens,
                               const int32_t* context_offsets, const int32_t* block_tables,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_tokens,
                               hipStream_t stream);

hipError_t launch_swap_blocks(void* dst, const void* src, const int64_t* pairs, int64_t num_pairs,
                              int64_t block_bytes, int64_t dst_blocks, int64_t src_blocks,
                              hipStream_t stream);

hipError_t launch_varlen_rows(int32_t* row_seq, int32_t* row_ctx, const int32_t* cu_seqlens,
                              const int32_t* context_offsets, int32_t num_seqs, int32_t q_rows,
                              hipStream_t stream);

hipError_t launch_write_kv(const void* key, const void* value, void* k_cache, void* v_cache,
                           const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                           int32_t head_dim, int64_t num_blocks, int32_t elem_bytes,
                           hipStream_t stream);

// Waves per workgroup and partition length for a decode call, from shapes only
// (so a call's result never depends on where its blocks live).
void decode_config(int num_seqs, int num_kv_heads, int max_context_len, int* waves,
                   int* part_tokens, int* buffers, int* grid_mode, int* oversub);
// whether a work-list launch derives its list in every workgroup (no plan kernel)
bool decode_inline_plan(int num_seqs, int waves);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// rows per prefill work item and bound on the number of items
int prefill_tile_tokens(int group);
int prefill_work_capacity(int num_seqs, int total_q_tokens, int num_kv_heads, int group);
// bytes of the work list (header and one record per item) in the workspace
size_t prefill_work_bytes(int num_seqs, int total_q_tokens, int num_kv_heads, int group);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// the common-prefix pass: `splits` items per (row tile, kv head)
hipError_t launch_cascade_prefix(const PrefillArgs& a, int splits, hipStream_t stream);

}  // namespace pa
