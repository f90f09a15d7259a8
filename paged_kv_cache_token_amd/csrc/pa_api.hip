// pa_api.hip -- the C ABI: host-side argument checks, workspace sizing and
// dispatch to the kernels.  Nothing here touches the GPU before every check
// has passed, so a call that returns an error has enqueued nothing.

#include <stdlib.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/pa.h"
#include "pa_launch.h"

using namespace pa;

namespace {

bool dtype_ok(int32_t dt) { return dt == PA_F32 || dt == PA_BF16; }
int elem_bytes(int32_t dt) { return dt == PA_BF16 ? 2 : 4; }
bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }
bool heads_ok(int32_t hq, int32_t hkv) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return false;
  const int g = hq / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}
int32_t from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }
// a softmax scale the kernels can use: finite (NaN or an infinity would give
// no defined weights)
bool scale_ok(float scale) { return std::isfinite(scale); }

// The matrix-core kernels fold a positive scale into their exponentials; any
// finite scale reaches that form exactly: scale < 0 as (-q, |scale|), 0 as
// (q = 0, 1), both giving the same scale * <q, k> for every key.
void set_prefill_scale(PrefillArgs& p, float scale) {
  if (scale > 0.f) {
    p.scale = scale;
    p.q_sign = 1;
  } else if (scale < 0.f) {
    p.scale = -scale;
    p.q_sign = -1;
  } else {
    p.scale = 1.f;
    p.q_sign = 0;
  }
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// varlen workspace = [decode partials][prefill work list]
size_t varlen_decode_part_bytes(int32_t num_seqs, int32_t hq, int32_t d, int32_t max_ctx) {
  return align_up(decode_ws_bytes(num_seqs, hq, d, decode_max_parts(max_ctx)));
}
// Chunks run on the matrix-core kernel for bf16 at head_dim 128; otherwise
// every packed row goes through the decode kernels as a row of its own.
bool varlen_matrix_path(int32_t dtype, int32_t head_dim) {
  return dtype == PA_BF16 && head_dim == 128;
}
// row path workspace = [row -> sequence][row -> context][decode partials of every row]
size_t varlen_rows_bytes(int32_t total_q) {
  return align_up((size_t)total_q * sizeof(int32_t));
}
size_t varlen_work_bytes(int32_t num_seqs, int32_t total_q, int32_t hkv, int32_t group) {
  return align_up(prefill_work_bytes(num_seqs, total_q, hkv, group));
}

// The common-prefix pass runs on the matrix-core kernel: bf16 at head_dim 128.
bool cascade_matrix_path(int32_t dtype, int32_t head_dim) {
  return dtype == PA_BF16 && head_dim == 128;
}
constexpr int kCascadeKeyTile = 64;  // keys per tile of the matrix-core kernel
// Tiles per prefix item: enough items to give every compute unit one (256
// items) but at least two tiles each, so the per-item start-up (query and
// first tiles in flight) is paid over several tiles.  Shapes only.
int cascade_split_tiles(int num_seqs, int num_kv_heads, int group, int prefix_tokens) {
  const int tiles = ceil_div(prefix_tokens, kCascadeKeyTile);
  const int pairs = ceil_div(num_seqs, prefill_tile_tokens(group)) * num_kv_heads;
  int st = std::max(2, (int)(((int64_t)tiles * pairs + 255) / 256));
  const char* e = getenv("PA_CASCADE_SPLIT_TILES");  // tuning override (>= 1)
  if (e && *e) {
    const int v = atoi(e);
    if (v >= 1) st = v;
  }
  return std::min(st, std::max(tiles, 1));
}
// The private rest of every context in one partition (one item per
// (sequence, kv head), on the single-partition kernel with its streaming
// loads) when it fits one item and the pairs alone give the chip enough
// items.  Measured with a 4096-token common prompt and private parts of
// U[16, 1024] tokens: 128 sequences (1024 pairs) 96 us against 101 split
// into 512-token partitions, 256 sequences 147 against 167; at 512 pairs
// and fewer, splitting was faster (64 sequences 67 against 72).
// PA_CASCADE_DIRECT=0/1 forces it off/on (if the rest fits one item).
bool cascade_single_rest(int num_seqs, int num_kv_heads, int rest, int waves) {
  if (rest <= 0 || rest > PA_BLOCK_SIZE * kMaxEntriesPerWave * waves) return false;
  const char* e = getenv("PA_CASCADE_DIRECT");
  if (e && *e) return atoi(e) != 0;
  return (int64_t)num_seqs * num_kv_heads >= 1024;
}
// Partial slots per (seq, q head): the prefix splits (at most one per tile),
// then the partitions of the rest of the longest context.
int cascade_max_parts(int32_t max_context_len, int32_t prefix_blocks, int part_tokens,
                      int splits) {
  const int prefix_tokens = prefix_blocks * PA_BLOCK_SIZE;
  if (splits <= 0) splits = std::max(1, ceil_div(prefix_tokens, kCascadeKeyTile));
  return splits + decode_max_parts(std::max(max_context_len - prefix_tokens, 0), part_tokens);
}


// Host checks shared by pa_decode and pa_decode_noalloc (PA_OK: go on).
int32_t decode_checks(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                      int32_t max_context_len, int64_t num_blocks, float scale, int32_t dtype) {
  if (!dtype_ok(dtype) || !head_dim_ok(head_dim) || block_size != PA_BLOCK_SIZE ||
      !heads_ok(num_q_heads, num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks <= 0 ||
      !scale_ok(scale))
    return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_NULL_POINTER;
  return PA_OK;
}

// A plain decode call's launch arguments and shape-based launch choice (the
// workspace layout is the caller's to add when max_parts > 1).
DecodeArgs decode_args(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                       int64_t num_blocks, float scale, int32_t dtype) {
  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.q_rows = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_blocks = num_blocks;
  a.scale = scale;
  a.dtype = dtype;
  a.varlen = false;
  decode_config(num_seqs, num_kv_heads, max_context_len, &a.waves, &a.part_tokens, &a.buffers,
                &a.grid_mode, &a.oversub);
  a.max_parts = decode_max_parts(max_context_len, a.part_tokens);
  return a;
}

}  // namespace

// ---------------------------------------------------------------------------
// Fixed device scratch of pa_decode_noalloc: the split-K partials and the work
// list of a decode call, for callers that cannot allocate.  Every GPU the
// library runs on holds one copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: the kernels get
// the address hipGetSymbolAddress returns for the device, kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;  // device ordinals served by pa_decode_noalloc

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kScratchDevices];

// The device `stream` runs on (the current device for the null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
  if (stream == nullptr) return hipGetDevice(dev);
  hipDevice_t d = 0;
  const hipError_t e = hipStreamGetDevice(stream, &d);
  *dev = static_cast<int>(d);
  return e;
}

// This device's copy of `scratch`, looked up once per device with that
// device current (the current device is restored afterwards).
hipError_t scratch_on(int dev, void** ptr) {
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s, dev] {
    int cur = -1;
    s.err = hipGetDevice(&cur);
    if (s.err == hipSuccess && cur != dev) s.err = hipSetDevice(dev);
    if (s.err == hipSuccess) s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (s.err == hipSuccess) s.err = r;
    }
    if (s.err == hipSuccess && s.ptr == nullptr) s.err = hipErrorInvalidSymbol;
    if (s.err != hipSuccess) (void)hipGetLastError();
  });
  *ptr = s.ptr;
  return s.err;
}

}  // namespace

extern "C" {

int32_t pa_version(void) { return PA_VERSION; }

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case PA_ERR_UNSUPPORTED:
      return "unsupported dtype, head_dim, block_size or query/kv head ratio";
    case PA_ERR_INVALID_ARGUMENT:
      return "negative or inconsistent size argument, or a non-finite softmax scale";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the size query returned";
    case PA_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case PA_ERR_NO_FREE_BLOCKS: return "not enough free blocks in the pool";
    case PA_ERR_HOST_MEMORY: return "a host memory allocation failed";
    case PA_ERR_SCRATCH_TOO_SMALL:
      return "the call needs more than the fixed device scratch of pa_decode_noalloc";
    default: return "unknown status";
  }
}

int32_t pa_build_slot_mapping(int64_t* slot_mapping, const int32_t* cu_seqlens,
                              const int32_t* context_offsets, const int32_t* block_tables,
                              int32_t num_seqs, int64_t num_tokens, int32_t max_blocks_per_seq,
                              int32_t block_size, void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARGUMENT;
  if (block_size != PA_BLOCK_SIZE) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!slot_mapping || !cu_seqlens || !context_offsets || !block_tables) return PA_ERR_NULL_POINTER;
  if (max_blocks_per_seq == 0) return PA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_slot_mapping(slot_mapping, cu_seqlens, context_offsets, block_tables,
                                      num_seqs, max_blocks_per_seq, num_tokens,
                                      static_cast<hipStream_t>(stream)));
}

int32_t pa_write_kv(const void* key, const void* value, void* k_cache, void* v_cache,
                    const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                    void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(head_dim) || block_size != PA_BLOCK_SIZE)
    return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL_POINTER;
  return from_hip(launch_write_kv(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                  num_kv_heads, head_dim, num_blocks, elem_bytes(dtype),
                                  static_cast<hipStream_t>(stream)));
}

// The address a kernel uses for p: device memory as is, pinned host memory
// through its device mapping; nullptr for memory the runtime does not know
// (pageable host memory would fault the kernel, so it is refused here).
static void* device_view(const void* p) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error the failed query leaves
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) return const_cast<void*>(p);
  if (attr.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return d;
  }
  return nullptr;
}

int32_t pa_swap_blocks(void* dst, const void* src, const int64_t* block_pairs, int64_t num_pairs,
                       int64_t block_bytes, int64_t dst_num_blocks, int64_t src_num_blocks,
                       void* stream) {
  if (num_pairs < 0 || block_bytes <= 0 || block_bytes % 16 != 0 || dst_num_blocks < 0 ||
      src_num_blocks < 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (num_pairs == 0) return PA_OK;
  if (!dst || !src || !block_pairs) return PA_ERR_NULL_POINTER;
  void* d = device_view(dst);
  void* s = device_view(src);
  void* pr = device_view(block_pairs);
  if (!d || !s || !pr) return PA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_swap_blocks(d, s, static_cast<const int64_t*>(pr), num_pairs, block_bytes,
                                     dst_num_blocks, src_num_blocks,
                                     static_cast<hipStream_t>(stream)));
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || !head_dim_ok(head_dim) || !dtype_ok(dtype)) return 0;
  return decode_ws_bytes(num_seqs, num_q_heads, head_dim, decode_max_parts(max_context_len));
}

int32_t pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
                  int64_t num_blocks, float scale, int32_t dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  const int32_t st = decode_checks(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                                   num_q_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, max_context_len, num_blocks, scale, dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  const size_t need =
      pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, dtype);
  if (workspace_bytes < need) return PA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && !workspace) return PA_ERR_NULL_POINTER;
  DecodeArgs a = decode_args(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                             num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                             max_context_len, num_blocks, scale, dtype);
  if (a.max_parts > 1)
    a.ws = decode_ws_layout(workspace, num_seqs, num_q_heads, head_dim, a.max_parts);
  return from_hip(launch_decode(a, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t max_context_len, int64_t num_blocks, float scale, int32_t dtype,
                          void* stream) {
  const int32_t st = decode_checks(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                                   num_q_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, max_context_len, num_blocks, scale, dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  DecodeArgs a = decode_args(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                             num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                             max_context_len, num_blocks, scale, dtype);
  if (a.max_parts > 1) {
    // what this launch uses (its own partition length, not the size query's
    // shortest one), refused before anything is enqueued when it exceeds the
    // fixed buffer
    const size_t need = decode_ws_bytes(num_seqs, num_q_heads, head_dim, a.max_parts);
    if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH_TOO_SMALL;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    int dev = -1;
    void* base = nullptr;
    if (stream_device(hs, &dev) != hipSuccess || scratch_on(dev, &base) != hipSuccess) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    a.ws = decode_ws_layout(base, num_seqs, num_q_heads, head_dim, a.max_parts);
  }
  return from_hip(launch_decode(a, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_step(void* out, const void* q, const void* key, const void* value,
                       void* k_cache, void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                       float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(head_dim) || block_size != PA_BLOCK_SIZE ||
      !heads_ok(num_q_heads, num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks <= 0 ||
      !scale_ok(scale))
    return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !key || !value || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_NULL_POINTER;
  const size_t need =
      pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, dtype);
  if (workspace_bytes < need) return PA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && !workspace) return PA_ERR_NULL_POINTER;

  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.q_rows = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_blocks = num_blocks;
  a.scale = scale;
  a.dtype = dtype;
  a.varlen = false;
  a.key_new = key;
  a.value_new = value;
  a.k_cache_w = k_cache;
  a.v_cache_w = v_cache;
  decode_config(num_seqs, num_kv_heads, max_context_len, &a.waves, &a.part_tokens, &a.buffers,
                &a.grid_mode, &a.oversub);
  a.max_parts = decode_max_parts(max_context_len, a.part_tokens);
  if (a.max_parts > 1)
    a.ws = decode_ws_layout(workspace, num_seqs, num_q_heads, head_dim, a.max_parts);
  return from_hip(launch_decode(a, static_cast<hipStream_t>(stream)));
}

size_t pa_cascade_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t num_common_prefix_blocks, int32_t dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || !head_dim_ok(head_dim) || !dtype_ok(dtype) ||
      num_common_prefix_blocks < 0)
    return 0;
  const size_t plain =
      pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, dtype);
  if (num_common_prefix_blocks == 0 || !cascade_matrix_path(dtype, head_dim)) return plain;
  const size_t split = decode_ws_bytes(num_seqs, num_q_heads, head_dim,
                                       cascade_max_parts(max_context_len, num_common_prefix_blocks,
                                                         kMinPartitionTokens, 0));
  return split > plain ? split : plain;
}

int32_t pa_cascade_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t max_context_len, int64_t num_blocks,
                          int32_t num_common_prefix_blocks, float scale, int32_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(head_dim) || block_size != PA_BLOCK_SIZE ||
      !heads_ok(num_q_heads, num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks <= 0 ||
      num_common_prefix_blocks < 0 || num_common_prefix_blocks > max_blocks_per_seq ||
      !scale_ok(scale))
    return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_NULL_POINTER;
  const size_t need = pa_cascade_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                max_context_len, num_common_prefix_blocks, dtype);
  if (workspace_bytes < need) return PA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && !workspace) return PA_ERR_NULL_POINTER;
  if (num_common_prefix_blocks == 0 || !cascade_matrix_path(dtype, head_dim))
    return pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len,
                     num_blocks, scale, dtype, workspace, workspace_bytes, stream);

  const int group = num_q_heads / num_kv_heads;
  const int prefix_tokens = num_common_prefix_blocks * PA_BLOCK_SIZE;
  const int split_tiles = cascade_split_tiles(num_seqs, num_kv_heads, group, prefix_tokens);
  const int splits = ceil_div(ceil_div(prefix_tokens, kCascadeKeyTile), split_tiles);

  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.q_rows = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_blocks = num_blocks;
  a.scale = scale;
  a.dtype = dtype;
  a.varlen = false;
  decode_config(num_seqs, num_kv_heads, max_context_len, &a.waves, &a.part_tokens, &a.buffers,
                &a.grid_mode, &a.oversub);
  a.key_start = prefix_tokens;
  a.prefix_parts = splits;
  if (cascade_single_rest(num_seqs, num_kv_heads, max_context_len - prefix_tokens, a.waves))
    a.part_tokens = std::max(a.part_tokens, ceil_div(max_context_len - prefix_tokens, PA_BLOCK_SIZE) *
                                                PA_BLOCK_SIZE);
  a.max_parts = cascade_max_parts(max_context_len, num_common_prefix_blocks, a.part_tokens, splits);
  a.ws = decode_ws_layout(workspace, num_seqs, num_q_heads, head_dim, a.max_parts);

  PrefillArgs p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.total_q_tokens = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.num_blocks = num_blocks;
  set_prefill_scale(p, scale);
  p.part_ml = a.ws.ml;
  p.part_acc = a.ws.acc;
  p.max_parts = a.max_parts;
  p.prefix_tokens = prefix_tokens;
  p.split_tiles = split_tiles;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t err = launch_cascade_prefix(p, splits, st);
  if (err != hipSuccess) return from_hip(err);
  return from_hip(launch_decode(a, st));
}

size_t pa_varlen_workspace_size(int32_t num_seqs, int32_t total_q_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                                int32_t dtype) {
  if (num_seqs <= 0 || total_q_tokens < 0 || !head_dim_ok(head_dim) || !dtype_ok(dtype) ||
      !heads_ok(num_q_heads, num_kv_heads))
    return 0;
  if (!varlen_matrix_path(dtype, head_dim))
    return 2 * varlen_rows_bytes(total_q_tokens) +
           varlen_decode_part_bytes(total_q_tokens, num_q_heads, head_dim, max_context_len);
  return varlen_decode_part_bytes(num_seqs, num_q_heads, head_dim, max_context_len) +
         varlen_work_bytes(num_seqs, total_q_tokens, num_kv_heads, num_q_heads / num_kv_heads);
}

int32_t pa_varlen_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* cu_seqlens, const int32_t* context_offsets,
                          const int32_t* block_tables, int32_t num_seqs, int32_t total_q_tokens,
                          int32_t max_q_len, int32_t max_context_len, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                          int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return pa_varlen_prefill_ex(out, q, k_cache, v_cache, cu_seqlens, context_offsets,
                              block_tables, num_seqs, total_q_tokens, max_q_len, max_context_len,
                              num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                              num_blocks, scale, dtype, -1, workspace, workspace_bytes, stream);
}

int32_t pa_varlen_prefill_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* cu_seqlens, const int32_t* context_offsets,
                             const int32_t* block_tables, int32_t num_seqs,
                             int32_t total_q_tokens, int32_t max_q_len, int32_t max_context_len,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                             float scale, int32_t dtype, int32_t num_decode_rows,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(head_dim) || block_size != PA_BLOCK_SIZE ||
      !heads_ok(num_q_heads, num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || total_q_tokens < 0 || max_q_len < 0 || max_context_len < 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || !scale_ok(scale))
    return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0 || total_q_tokens == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !cu_seqlens || !context_offsets || !block_tables)
    return PA_ERR_NULL_POINTER;
  const size_t need = pa_varlen_workspace_size(num_seqs, total_q_tokens, num_q_heads,
                                               num_kv_heads, head_dim, max_context_len, dtype);
  if (workspace_bytes < need) return PA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return PA_ERR_NULL_POINTER;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);

  if (!varlen_matrix_path(dtype, head_dim)) {
    // every row on its own through the decode kernels: row r of sequence i
    // attends i's keys 0 .. context_offsets[i] + j
    int32_t* row_seq = reinterpret_cast<int32_t*>(ws);
    int32_t* row_ctx = reinterpret_cast<int32_t*>(ws + varlen_rows_bytes(total_q_tokens));
    hipError_t err = launch_varlen_rows(row_seq, row_ctx, cu_seqlens, context_offsets, num_seqs,
                                        total_q_tokens, s);
    if (err != hipSuccess) return PA_ERR_HIP;
    DecodeArgs r{};
    r.out = out;
    r.q = q;
    r.k_cache = k_cache;
    r.v_cache = v_cache;
    r.block_tables = block_tables;
    r.table_rows = row_seq;
    r.context_lens = row_ctx;
    r.num_seqs = total_q_tokens;
    r.q_rows = total_q_tokens;
    r.num_q_heads = num_q_heads;
    r.num_kv_heads = num_kv_heads;
    r.head_dim = head_dim;
    r.max_blocks_per_seq = max_blocks_per_seq;
    r.max_context_len = max_context_len;
    r.num_blocks = num_blocks;
    r.scale = scale;
    r.dtype = dtype;
    r.varlen = true;
    decode_config(total_q_tokens, num_kv_heads, max_context_len, &r.waves, &r.part_tokens,
                  &r.buffers, &r.grid_mode, &r.oversub);
    r.max_parts = decode_max_parts(max_context_len, r.part_tokens);
    if (r.max_parts > 1)
      r.ws = decode_ws_layout(ws + 2 * varlen_rows_bytes(total_q_tokens), total_q_tokens,
                              num_q_heads, head_dim, r.max_parts);
    return from_hip(launch_decode(r, s));
  }

  const size_t dec_bytes =
      varlen_decode_part_bytes(num_seqs, num_q_heads, head_dim, max_context_len);

  // single-token rows: the decode kernels in varlen mode
  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.cu_seqlens = cu_seqlens;
  a.context_offsets = context_offsets;
  a.num_seqs = num_seqs;
  a.q_rows = total_q_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_blocks = num_blocks;
  a.scale = scale;
  a.dtype = dtype;
  a.varlen = true;
  decode_config(num_seqs, num_kv_heads, max_context_len, &a.waves, &a.part_tokens, &a.buffers,
                &a.grid_mode, &a.oversub);
  a.max_parts = decode_max_parts(max_context_len, a.part_tokens);
  if (a.max_parts > 1) a.ws = decode_ws_layout(ws, num_seqs, num_q_heads, head_dim, a.max_parts);
  if (num_decode_rows != 0) {
    const hipError_t err = launch_decode(a, s);
    if (err != hipSuccess) return PA_ERR_HIP;
  }
  if (max_q_len <= 1) return PA_OK;

  // multi-token chunks: the matrix-core prefill kernel
  PrefillArgs p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.cu_seqlens = cu_seqlens;
  p.context_offsets = context_offsets;
  p.block_tables = block_tables;
  p.num_seqs = num_seqs;
  p.total_q_tokens = total_q_tokens;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.num_blocks = num_blocks;
  set_prefill_scale(p, scale);
  p.work = reinterpret_cast<int32_t*>(ws + dec_bytes);
  p.work_cap =
      prefill_work_capacity(num_seqs, total_q_tokens, num_kv_heads, num_q_heads / num_kv_heads);
  return from_hip(launch_prefill(p, s));
}

}  // extern "C"
