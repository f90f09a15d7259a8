// pa_internal.h -- device helpers and launcher declarations shared by the
// library's kernel files (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;        // tokens per physical block
constexpr int kDecodeWaves = 4;       // waves per decode workgroup
constexpr int kPartitionTokens = 512; // split-K partition (multiple of kBlockSize)

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

// bf16 <-> fp32.  Widening is exact (the bf16 pattern is the top half of the
// fp32 one); narrowing rounds to nearest-even through the compiler's __bf16
// conversion (a hardware convert on gfx950).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}

// ---------------------------------------------------------------------------
// wavefront reductions
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// All-reduce sum over aligned groups of W consecutive lanes (W = 8, 16, 32, 64);
// every lane of a group ends with the group's sum.  Within a 16-lane DPP row:
// quad_perm swaps of neighbours and pairs, then the half-row mirror (lane i
// <-> 7-i joins the two quads of each half), then the row mirror (i <-> 15-i
// joins the two halves).  Beyond 16 lanes a cross-row exchange follows.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  if constexpr (W >= 16) x += dpp_f32<0x140>(x);  // row_mirror
  if constexpr (W >= 32) x += __shfl_xor(x, 16);
  if constexpr (W >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// launch arguments
// ---------------------------------------------------------------------------

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;     // decode mode: tokens per sequence
  const int32_t* cu_seqlens;       // varlen mode: packed query rows
  const int32_t* context_offsets;  // varlen mode: cached tokens before the row
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int64_t num_blocks;
  float scale;
  int32_t dtype;                   // PA_F32 / PA_BF16
  bool varlen;                     // rows come from cu_seqlens; only q_len == 1 seqs
  float* ws;                       // partials (may be null if max_parts == 1)
  int32_t max_parts;
};

// Split-K partial layout in the workspace:
//   ml  [num_seqs][num_q_heads][max_parts][2]   (running max in log2 units, sum)
//   acc [num_seqs][num_q_heads][max_parts][head_dim]
inline size_t decode_ws_floats(int num_seqs, int num_q_heads, int head_dim, int max_parts) {
  if (max_parts <= 1) return 0;
  return (size_t)num_seqs * num_q_heads * max_parts * (head_dim + 2);
}
inline int decode_max_parts(int max_context_len) {
  return max_context_len <= 0 ? 1 : ceil_div(max_context_len, kPartitionTokens);
}

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_seqlens;
  const int32_t* context_offsets;
  const int32_t* block_tables;
  int32_t num_seqs;
  int32_t total_q_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int64_t num_blocks;
  float scale;
  int32_t* work;       // work list in the workspace
  int32_t work_cap;    // capacity in items
};

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* cu_seqlens,
                               const int32_t* context_offsets, const int32_t* block_tables,
                               int32_t num_seqs, int32_t max_blocks_per_seq, hipStream_t stream);

hipError_t launch_write_kv(const void* key, const void* value, void* k_cache, void* v_cache,
                           const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                           int32_t head_dim, int64_t num_blocks, int32_t elem_bytes,
                           hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// rows per prefill work item and bound on the number of items
int prefill_tile_tokens(int group);
int prefill_work_capacity(int num_seqs, int total_q_tokens, int group);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
