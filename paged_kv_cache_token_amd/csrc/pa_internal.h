// pa_internal.h -- device helpers and launcher declarations shared by the
// library's kernel files (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;           // tokens per physical block
constexpr int kDecodeMaxWaves = 4;       // waves per decode workgroup (1, 2 or 4)
constexpr int kMinPartitionTokens = 256; // smallest split-K partition; sizes the workspace
constexpr int kMaxEntriesPerWave = 64;   // table entries a wave holds (one per lane)

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
// x rounded to the nearest bf16, as fp32 (exact in either format)
__device__ __forceinline__ float round_to_bf16(float x) {
  return __uint_as_float((uint32_t)f32_to_bf16_bits(x) << 16);
}

// ---------------------------------------------------------------------------
// vector types, LDS and buffer helpers
// ---------------------------------------------------------------------------

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// two fp32 -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_f32_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

#define PA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// 16 bytes per lane from a buffer straight into LDS: lane i's chunk (at
// byte offset voff of the buffer) lands at lds_base + 16 i (lds_base is
// wave-uniform); a chunk at or past num_records bytes reads as zeros.  AUX:
// the load's cache-policy bits (2: non-temporal).
template <int AUX = 0>
__device__ __forceinline__ void dma16(const void* base, int num_records, int voff, uint4* lds_base) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_records, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, PA_LDS(void, lds_base), 16, voff, 0, 0, AUX);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane s supplies the address of 4 consecutive bf16; lane j = 4q + c of the
// group receives element c of the chunks of lanes q, 4 + q, 8 + q, 12 + q.
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(PA_LDS(i16x4_t, p)));
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

// The same all-reduce applied to N independent values, one DPP step at a time
// across all of them, so consecutive DPP operations never depend on each other.
template <int W, int N>
__device__ __forceinline__ void group_sum_n(float (&x)[N]) {
  static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f32<0xB1>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f32<0x4E>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f32<0x141>(x[i]);
  if constexpr (W >= 16) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f32<0x140>(x[i]);
  }
  if constexpr (W >= 32) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], 16);
  }
  if constexpr (W >= 64) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], 32);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// launch arguments
// ---------------------------------------------------------------------------

// Decode workspace (used only when some context spans several partitions):
//   ml       float [num_seqs][num_q_heads][max_parts][2]  (running max in log2 units, sum)
//   acc      float [num_seqs][num_q_heads][max_parts][head_dim]
//   count    int   [1]                       (work items in the list)
//   items    int2  [num_seqs * max_parts]    ((sequence, partition) work list)
struct DecodeWorkspace {
  float* ml;
  float* acc;
  int32_t* count;
  int2* items;
};

inline int decode_max_parts(int max_context_len, int partition_tokens = kMinPartitionTokens) {
  return max_context_len <= 0 ? 1 : ceil_div(max_context_len, partition_tokens);
}

inline size_t decode_ws_bytes(int num_seqs, int num_q_heads, int head_dim, int max_parts) {
  if (max_parts <= 1) return 0;
  const size_t rows = (size_t)num_seqs * num_q_heads * max_parts;
  size_t bytes = rows * 2 * sizeof(float);                    // ml
  bytes += rows * (size_t)head_dim * sizeof(float);           // acc
  bytes += 2 * sizeof(int32_t);                               // count (+ pad to 8 bytes)
  bytes += (size_t)num_seqs * max_parts * sizeof(int2);       // items
  return bytes;
}

inline DecodeWorkspace decode_ws_layout(void* base, int num_seqs, int num_q_heads, int head_dim,
                                        int max_parts) {
  DecodeWorkspace w{};
  char* p = static_cast<char*>(base);
  const size_t rows = (size_t)num_seqs * num_q_heads * max_parts;
  w.ml = reinterpret_cast<float*>(p);
  p += rows * 2 * sizeof(float);
  w.acc = reinterpret_cast<float*>(p);
  p += rows * (size_t)head_dim * sizeof(float);
  w.count = reinterpret_cast<int32_t*>(p);
  p += 2 * sizeof(int32_t);
  w.items = reinterpret_cast<int2*>(p);
  return w;
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* table_rows;       // varlen mode, rows one by one: block-table row of each
                                   // packed row (null: single-token sequences only)
  const int32_t* context_lens;     // decode mode: tokens per sequence; rows one by one: per row
  const int32_t* cu_seqlens;       // varlen mode: packed query rows
  const int32_t* context_offsets;  // varlen mode: cached tokens before the row
  int32_t num_seqs;
  int32_t q_rows;                  // rows of q / out (num_seqs, or total packed rows)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int64_t num_blocks;
  float scale;
  int32_t dtype;                   // PA_F32 / PA_BF16
  bool varlen;                     // rows come from cu_seqlens (only q_len == 1 seqs), or
                                   // every row on its own through table_rows
  const void* key_new;             // fused step: the new token's K [num_seqs][Hkv][d], or null
  const void* value_new;           // fused step: the new token's V
  void* k_cache_w;                 // fused step: caches to store the new token into
  void* v_cache_w;
  DecodeWorkspace ws;              // valid when max_parts > 1
  int32_t max_parts;               // partitions of the longest context
  int32_t part_tokens;             // split-K partition length (a multiple of 16 tokens)
  int32_t waves;                   // waves per workgroup
  int32_t buffers;                 // K/V register buffers per wave (2..4)
  int32_t grid_mode;               // multi-partition: 1 = (seq, kvh, part) grid, 0 = work list
  int32_t oversub;                 // persistent grid = oversub x resident workgroups
  int32_t key_start;               // keys [0, key_start) of every context are attended
                                   // elsewhere (a common prefix); partitions start there
  int32_t inline_plan;             // work list mode: each workgroup derives the item list
                                   // itself (no plan kernel); needs num_seqs <= 2048
  int32_t prefix_parts;            // partial slots [0, prefix_parts) of every (seq, q head)
                                   // hold that prefix's partials; this call's partitions
                                   // follow them, and the merge takes all of them
  int32_t mfma;                    // bf16 at head_dim 128: the matrix-core item code
                                   // (set at launch)
};

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
  float scale;         // > 0: the kernels fold it into exp2 with a running max in raw
                       // score units, which only orders scores correctly for scale > 0
  int32_t q_sign;      // how the call's scale reaches that form: 1 = q as is (scale > 0),
                       // -1 = q negated, scale = |call scale| (s * scale unchanged),
                       // 0 = q zeroed, scale = 1 (every visible key weighs the same)
  int32_t* work;       // work list in the workspace
  int32_t work_cap;    // capacity in items
  // common-prefix pass of a decode call (the rows are the sequences' single
  // query rows; the keys are the first prefix_tokens of block-table row 0)
  const int32_t* context_lens;
  float* part_ml;      // decode partial slots: (max in log2 units, sum) ...
  float* part_acc;     // ... and unnormalised accumulators, max_parts per (seq, q head)
  int32_t max_parts;
  int32_t prefix_tokens;
  int32_t split_tiles; // 64-key tiles per item; item x of a row tile fills partial slot x
};

}  // namespace pa
