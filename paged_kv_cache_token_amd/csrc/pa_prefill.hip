// pa_prefill.hip -- causal attention of the multi-token chunks of a packed
// super-sequence over the paged cache, on the CDNA4 matrix cores.
//
// "vLLM изнутри: как устроен движок для быстрого инференса LLM", forward-pass
// paragraph: all sequences of a step are packed into one super-sequence whose
// masks and positions keep each sequence on its own tokens; the paragraph on
// the stages of a step: prefill works on every prompt token and is bound by
// compute.  "vLLM：颠覆大模型推理的高效API服务引擎深度解析", §1.3: the keys and
// values come from physical blocks gathered through the block table.  The
// tiled online softmax is the chunked-attention idea of the flash-attention
// paragraph in "vLLMつかったら、ベクトル検索サーバーが高速化して安定性も向上した".
//
// Work decomposition (gfx950, wave64, head_dim 128, bf16):
//   * a work item is (sequence, tile of 256/g query tokens) for one kv head; its
//     256 rows are the g query heads of that kv head times the tile's tokens,
//     32 rows per wave, 8 waves (two per SIMD, so one wave's softmax overlaps
//     the other's matrix products), and each K/V tile read serves all g heads;
//   * keys stream in tiles of 64 (4 physical blocks), gathered through the
//     block table straight from HBM into four LDS buffers (K and V alike as
//     [block][16-byte chunk][key], keys swizzled by chunk; V is read back with
//     the transposing LDS read).  One barrier per tile: tile t is computed
//     while tile t+1 waits in LDS and the loads of tile t+2 are in flight;
//   * the work list is ordered longest first (key tiles per item), built by
//     every workgroup in LDS (or, for very large calls, by a plan kernel); one
//     workgroup per CU walks its share in snake order, and while an item runs
//     its last steps the next item's record, first two key tiles and query
//     rows are already being loaded, so items follow each other without a
//     cold start;
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = the wave's 32 query rows
//     held in registers), so a lane holds 16 scores of one query row and the
//     softmax statistics are per lane (one exchange with lane^32 per tile);
//   * O^T += V^T P^T with the same instruction: the B operand (P^T) is taken
//     straight from the S^T accumulators, rounded to bf16, with the key order
//     inside each 16-key step permuted to match the accumulator layout; the A
//     operand reads V^T rows from LDS in that same key order;
//   * the causal mask (key <= context_offset + row) is applied only on tiles
//     that cross the diagonal; V of keys past the chunk's last key is zeroed
//     on the way into LDS (p = 0 times a stale NaN would poison the sum);
//   * the same item code serves the common-prefix pass of a cascade decode:
//     rows are the single query rows of 256/g sequences, keys a range of the
//     shared prefix, and the item writes partial results for the decode merge.

#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "pa_launch.h"

namespace pa {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPrefillD = 128;
constexpr int kPrefillWaves = 8;             // two waves per SIMD share every K/V tile
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr int kPrefillRows = 32 * kPrefillWaves;  // (head, token) rows per item
constexpr int kKeyTile = 64;                 // keys per tile = 4 physical blocks
constexpr int kSortBuckets = 1024;           // work-list order: key tiles per item (capped)

int prefill_tile_tokens(int group) { return kPrefillRows / group; }

int prefill_work_capacity(int num_seqs, int total_q_tokens, int num_kv_heads, int group) {
  const int t = prefill_tile_tokens(group);
  return (total_q_tokens / t + num_seqs + 1) * num_kv_heads;
}

// Work list in the workspace: a 64-byte header (int32 item count), then one
// 128-byte record per item, int32 words:
//   [0] sequence  [1] query tile * num_kv_heads + kv head  [2] first packed row
//   [3] query rows of the sequence  [4] its cached tokens  [5..7] unused
//   [8 + 4j + b]  table entry of block b of key tile j, j < 3 (clamped into
//                 the table row), so a workgroup can start the item's first
//                 tile loads without reading the table itself
constexpr int kRecWords = 32;
constexpr int kWorkHeaderWords = 16;

__device__ __forceinline__ int32_t* prefill_rec(int32_t* work, int idx) {
  return work + kWorkHeaderWords + (int64_t)idx * kRecWords;
}

size_t prefill_work_bytes(int num_seqs, int total_q_tokens, int num_kv_heads, int group) {
  return (kWorkHeaderWords +
          (size_t)kRecWords * prefill_work_capacity(num_seqs, total_q_tokens, num_kv_heads, group)) *
         sizeof(int32_t);
}

// One workgroup lists the (sequence, query tile, kv head) items of every
// sequence with two or more query rows, ordered by the number of 64-key tiles
// they stream, most first (a counting sort in LDS), so the persistent
// workgroups start the longest items first, on every CU at once.  It serves
// the calls too large for the list each workgroup builds itself (below).  The
// order among equal counts is arbitrary: items are independent and each
// writes only its own rows.  The work is spread over (sequence, query tile) pairs, so a
// few long chunks do not leave one thread per sequence walking its tiles.
constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxSeqs = 2048;  // sequences held in LDS (two per thread)

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillArgs a,
                                                                    int tile_tokens) {
  __shared__ int count[kSortBuckets];
  __shared__ int wave_tot[kPlanThreads / 64];
  __shared__ int pair0[kPlanMaxSeqs];  // first (sequence, query tile) pair of each sequence
  __shared__ int slen[kPlanMaxSeqs], sctx[kPlanMaxSeqs];
  const int n = a.num_seqs;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int maxk = max(0, min(a.max_context_len, a.max_blocks_per_seq * kBlockSize));
  for (int i = t; i < kSortBuckets; i += kPlanThreads) count[i] = 0;

  // exclusive scan over the block of one value per thread; returns the
  // thread's offset, and the sum in `total`
  auto block_scan = [&](int v, int& total) -> int {
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int up = __shfl_up(inc, off);
      if (lane >= off) inc += up;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      const int x = wave_tot[w];
      base += w < wave ? x : 0;
      total += x;
    }
    __syncthreads();  // wave_tot is reused by the next scan
    return base + inc - v;
  };
  auto bucket = [&](int len, int c, int q) {
    const int qn = min(tile_tokens, len - q * tile_tokens);
    const int kend = max(0, min(c + q * tile_tokens + qn, maxk));
    return min(ceil_div(kend, kKeyTile), kSortBuckets - 1);
  };

  // each thread: sequences 2t, 2t+1 (metadata into LDS) and their query tiles
  const bool fits = n <= kPlanMaxSeqs;
  int npairs = 0;
  if (fits) {
    int nt[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int sq = 2 * t + j;
      if (sq < n) {
        const int lo = a.cu_seqlens[sq];
        const int len = a.cu_seqlens[sq + 1] - lo;
        slen[sq] = len;
        sctx[sq] = a.context_offsets[sq];
        nt[j] = len >= 2 ? ceil_div(len, tile_tokens) : 0;
      }
    }
    const int first = block_scan(nt[0] + nt[1], npairs);
    if (2 * t < n) pair0[2 * t] = first;
    if (2 * t + 1 < n) pair0[2 * t + 1] = first + nt[0];
  }
  __syncthreads();
  // the sequence of pair p: the last s with pair0[s] <= p (sequences without
  // tiles repeat their successor's start and are passed over)
  auto seq_of = [&](int p) -> int {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pair0[mid] <= p) lo = mid;
      else hi = mid;
    }
    return lo;
  };
  auto seq_meta = [&](int sq, int& len, int& c) {
    len = a.cu_seqlens[sq + 1] - a.cu_seqlens[sq];
    c = a.context_offsets[sq];
  };

  if (fits) {
    for (int p = t; p < npairs; p += kPlanThreads) {
      const int sq = seq_of(p);
      atomicAdd(&count[bucket(slen[sq], sctx[sq], p - pair0[sq])], a.num_kv_heads);
    }
  } else {
    for (int sq = t; sq < n; sq += kPlanThreads) {
      int len, c;
      seq_meta(sq, len, c);
      if (len < 2) continue;
      const int nt = ceil_div(len, tile_tokens);
      for (int q = 0; q < nt; ++q) atomicAdd(&count[bucket(len, c, q)], a.num_kv_heads);
    }
  }
  __syncthreads();
  // exclusive offsets, largest bucket first: thread t owns bucket 1023 - t
  static_assert(kSortBuckets == kPlanThreads, "one bucket per thread");
  int total = 0;
  const int off = block_scan(count[kSortBuckets - 1 - t], total);
  count[kSortBuckets - 1 - t] = off;
  if (t == 0) a.work[0] = min(total, a.work_cap);
  __syncthreads();
  auto place = [&](int sq, int q, int len, int c) {
    const int pos = atomicAdd(&count[bucket(len, c, q)], a.num_kv_heads);
    const int32_t* table = a.block_tables + (int64_t)sq * a.max_blocks_per_seq;
    int e[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) e[i] = table[min(i, a.max_blocks_per_seq - 1)];
    const int lo = a.cu_seqlens[sq];
    for (int h = 0; h < a.num_kv_heads; ++h) {
      if (pos + h >= a.work_cap) break;
      int4* r = reinterpret_cast<int4*>(prefill_rec(a.work, pos + h));
      r[0] = make_int4(sq, q * a.num_kv_heads + h, lo, len);
      r[1] = make_int4(c, 0, 0, 0);
      r[2] = make_int4(e[0], e[1], e[2], e[3]);
      r[3] = make_int4(e[4], e[5], e[6], e[7]);
      r[4] = make_int4(e[8], e[9], e[10], e[11]);
    }
  };
  if (fits) {
    for (int p = t; p < npairs; p += kPlanThreads) {
      const int sq = seq_of(p);
      place(sq, p - pair0[sq], slen[sq], sctx[sq]);
    }
  } else {
    for (int sq = t; sq < n; sq += kPlanThreads) {
      int len, c;
      seq_meta(sq, len, c);
      if (len < 2) continue;
      const int nt = ceil_div(len, tile_tokens);
      for (int q = 0; q < nt; ++q) place(sq, q, len, c);
    }
  }
}

// LDS tiles: 64 keys x 128 dims of bf16, as [block of 16 keys][16-byte chunk
// of 8 dims][key in block], the key position XOR-swizzled by the chunk:
// key k16 of chunk c sits at position k16 ^ 4 (c % 4).  The direct HBM->LDS
// loads write each wave instruction's 1 KiB contiguously (4 chunks x 16 keys
// of one block); the 16-byte K reads of 16 keys at one chunk, and the
// transposing 8-byte V reads of 4 keys x 4 chunks, hit distinct banks.
struct __attribute__((aligned(16))) PrefillShared {
  uint4 k[4][4][16][16];
  uint4 v[4][4][16][16];
};

// A prefill work item's metadata, and the table entries of its first three
// key tiles (one per lane, lane i: block i & 3 of the tile).
struct ItemMeta {
  int seq, qtile, kvh;  // cascade: key split, row tile, kv head
  int lo_row, len, c;   // first packed row, query rows, cached tokens
  int e0, e1, e2;
};

// An item's record as loaded (vector registers), turned into ItemMeta only
// where it is used, so the load is waited for there and not at issue.
struct RecRaw {
  int4 m;  // seq, tile * num_kv_heads + kv head, first row, query rows
  int c, e0, e1, e2;
};

// A workgroup's own items when it builds the work list itself: its k-th item
// (rank k of the snake order) in entry k, the same fields as words 0..4 of a
// record in the workspace list.
constexpr int kListCap = 256;
struct ItemList {
  int4 m[kListCap];
  int c[kListCap];
};

// Item idx's record: from the workspace list (idx is the item's rank), or,
// when the workgroup built its own list (INL), entry idx of `list` (in LDS),
// whose table entries are read from the block table here.
template <bool INL>
__device__ __forceinline__ RecRaw load_rec(const PrefillArgs& a, int idx, const ItemList* list) {
  const int lane = threadIdx.x & 63;
  RecRaw x;
  if constexpr (INL) {
    const auto* e = PA_LDS(const int, &list->m[idx]);
    x.m = make_int4(e[0], e[1], e[2], e[3]);
    x.c = *PA_LDS(const int, &list->c[idx]);
    const int32_t* table = a.block_tables + (int64_t)x.m.x * a.max_blocks_per_seq;
    const int last = a.max_blocks_per_seq - 1;
    x.e0 = table[min(lane & 3, last)];
    x.e1 = table[min(4 + (lane & 3), last)];
    x.e2 = table[min(8 + (lane & 3), last)];
    return x;
  }
  const int32_t* r = prefill_rec(a.work, idx);
  x.m = *reinterpret_cast<const int4*>(r);
  x.c = r[4];
  x.e0 = r[8 + (lane & 3)];
  x.e1 = r[12 + (lane & 3)];
  x.e2 = r[16 + (lane & 3)];
  return x;
}

__device__ __forceinline__ ItemMeta meta_of(const PrefillArgs& a, const RecRaw& x) {
  ItemMeta im;
  im.seq = __builtin_amdgcn_readfirstlane(x.m.x);
  const int y = __builtin_amdgcn_readfirstlane(x.m.y);
  im.qtile = y / a.num_kv_heads;
  im.kvh = y - im.qtile * a.num_kv_heads;
  im.lo_row = __builtin_amdgcn_readfirstlane(x.m.z);
  im.len = __builtin_amdgcn_readfirstlane(x.m.w);
  im.c = __builtin_amdgcn_readfirstlane(x.c);
  im.e0 = x.e0;
  im.e1 = x.e1;
  im.e2 = x.e2;
  return im;
}

// Keys [0, kend) that any row of a (non-cascade) item sees, clamped to the
// declared maxima.
template <int G>
__device__ __forceinline__ int item_kend(const PrefillArgs& a, const ItemMeta& x) {
  constexpr int BMT = kPrefillRows / G;
  const int q0 = x.qtile * BMT;
  const int qn = min(BMT, x.len - q0);
  const int kmax = min(a.max_context_len, a.max_blocks_per_seq * kBlockSize);
  return max(0, min(x.c + q0 + qn, kmax));
}

// The query fragments of item x (B operand of S^T = K Q^T): lane n = lane & 31
// of wave w holds row rho = 32w + n (head kvh*G + rho / (256/G), token
// q0 + rho % (256/G)), dims ks*16 + hi*8 .. +8 in qf[ks].  Rows past the tile
// or outside the packed arrays read as zeros.  A call with scale < 0 runs on
// -q and |scale| (negating a bf16 flips its sign bit: exact), one with scale 0
// on q = 0 (all scores 0: uniform weights).
template <int G, bool CASCADE>
__device__ __forceinline__ void load_query(const PrefillArgs& a, const ItemMeta& x,
                                           bf16x8_t (&qf)[8]) {
  constexpr int D = kPrefillD;
  constexpr int BMT = kPrefillRows / G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, hi = lane >> 5;
  const int lo_row = CASCADE ? 0 : x.lo_row;
  const int len = CASCADE ? a.num_seqs : x.len;
  const int q0 = x.qtile * BMT;
  const int qn = min(BMT, len - q0);
  const int rho = wave * 32 + n;
  const int head = x.kvh * G + rho / BMT;
  const int tok = rho % BMT;
  const bool valid =
      tok < qn && lo_row >= 0 && (int64_t)lo_row + q0 + tok < (int64_t)a.total_q_tokens;
  const uint4* qrow = static_cast<const uint4*>(a.q) +
                      ((int64_t)(valid ? lo_row + q0 + tok : 0) * a.num_q_heads + head) * (D / 8);
  const uint32_t flip = a.q_sign < 0 ? 0x80008000u : 0u;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    uint4 v = qrow[ks * 2 + hi];
    v.x ^= flip;
    v.y ^= flip;
    v.z ^= flip;
    v.w ^= flip;
    if (!valid || a.q_sign == 0) v = make_uint4(0u, 0u, 0u, 0u);
    qf[ks] = __builtin_bit_cast(bf16x8_t, v);
  }
}

// What a workgroup carries from one item to the next.
struct PipeState {
  bf16x8_t qf[8];  // the query fragments of the item about to run, when q_ready
  int tb;          // key tiles this workgroup has streamed: tile t of the
                   // running item sits in LDS buffer (tb + t) & 3
  int pre;         // leading key tiles (0..2) of the item about to run whose
                   // loads the previous item already issued
  bool q_ready;
};

// One work item.  Prefill (CASCADE = false): sequence `seq`, query tile
// `qtile`, kv head `kvh`; rows are (q head, token) of the tile.  Common-prefix
// pass (CASCADE = true): `seq` is the key split (tiles split*split_tiles ..),
// the rows are (q head, sequence) for sequences qtile*256/G ..; every row
// sees the prefix keys below its own context length, and the item writes
// unnormalised partials instead of the output.
//
// Items run back to back in a workgroup overlap their start-up with the end
// of the previous item: given the next item's index (its rank in the
// workspace list, or its entry in the workgroup's own `list`), the running one
// loads its record with its own first key tile, starts the next item's first two
// key tiles into the LDS buffers its own last two steps leave free, and loads
// the next item's queries during its own last step (which skips the discarded
// score products that would read them).  On return `next` holds the next
// item and `pipe` what was started for it.
template <int G, bool CASCADE, bool INL = false>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, const ItemMeta& im,
                                             PrefillShared& sm, PipeState& pipe, int next_idx,
                                             const ItemList* list, ItemMeta& next) {
  const int seq = im.seq, qtile = im.qtile, kvh = im.kvh;
  constexpr int D = kPrefillD;
  constexpr int BMT = kPrefillRows / G;  // query tokens per item
  constexpr float kNegInf = -INFINITY;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;             // this lane's query row within the wave
  const int hi = lane >> 5;            // which half of each 16-element k step

  // per-item metadata, wave-uniform
  int lo_row, len, c;
  if constexpr (CASCADE) {
    lo_row = 0;
    len = a.num_seqs;
    c = 0;
  } else {
    lo_row = im.lo_row;
    len = im.len;
    c = im.c;
  }
  const int tile0 = CASCADE ? seq * a.split_tiles : 0;  // first key tile of the item
  const int q0 = qtile * BMT;
  const int qn = min(BMT, len - q0);   // valid query tokens of this tile (>= 1)
  const int rho = wave * 32 + n;       // row of the item: (head_local, token)
  const int head = kvh * G + rho / BMT;
  const int tok = rho % BMT;
  // rows outside the packed q / out arrays (inconsistent metadata) are skipped
  const bool valid_q =
      tok < qn && lo_row >= 0 && (int64_t)lo_row + q0 + tok < (int64_t)a.total_q_tokens;
  const int kmax = min(a.max_context_len, a.max_blocks_per_seq * kBlockSize);
  int kend, row_lim, full_lim;
  if constexpr (CASCADE) {
    // keys of the split; a row sees those below its context length
    kend = max(0, min(min((tile0 + a.split_tiles) * kKeyTile, a.prefix_tokens), kmax));
    const int ctx = valid_q ? max(0, min(a.context_lens[q0 + tok], kmax)) : 0;
    row_lim = min(ctx, kend);
    // keys every valid row of this wave sees (masking is decided per wave)
    int lim = valid_q ? row_lim : 0x7fffffff;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lim = min(lim, __shfl_xor(lim, off));
    full_lim = __builtin_amdgcn_readfirstlane(lim);
  } else {
    const int qpos = c + q0 + tok;       // absolute position of this row
    // keys any row of the item sees, clamped to the declared maxima
    kend = max(0, min(c + q0 + qn, kmax));
    row_lim = valid_q ? min(qpos + 1, kend) : 0;  // keys [0, row_lim) are visible
    full_lim = min(c + q0 + 1, kend);  // keys every row of the item sees
  }
  const int ntiles = max(0, ceil_div(kend, kKeyTile) - tile0);
  const int hkv = a.num_kv_heads;
  const int hq = a.num_q_heads;
  const int32_t* table = a.block_tables + (CASCADE ? 0 : (int64_t)seq * a.max_blocks_per_seq);

  // B operand of S^T = K Q^T: this item's query rows (already loaded when the
  // previous item prefetched them)
  bf16x8_t (&qf)[8] = pipe.qf;
  if (!pipe.q_ready) load_query<G, CASCADE>(a, im, qf);
  const int tb = pipe.tb;
  const bool has_next = !CASCADE && next_idx >= 0;
  RecRaw nraw{};
  int next_pre = 0;       // leading tiles of the next item started here
  bool next_q = false;    // the next item's queries loaded here

  // Table entries of a tile, one per lane (lane i & 3: block i & 3 of the
  // tile), loaded one step ahead with vector loads that land with that step's
  // tile loads; read back as wave-uniform values, so no scalar load waits on
  // the in-flight tile loads.  Entries past the table's end are clamped (their
  // keys lie past the item's end).
  auto entries = [&](int t) -> int {
    return table[min((tile0 + t) * 4 + (lane & 3), a.max_blocks_per_seq - 1)];
  };
  auto phys_of = [&](int e, int blk) -> int {
    const int phys = __builtin_amdgcn_readlane(e, blk);
    return (phys >= 0 && (int64_t)phys < a.num_blocks) ? phys : -1;
  };
  // bit b: block b of the tile is outside the pool (its keys take no part)
  auto bad_mask = [&](int e) -> int {
    int bad = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) bad |= (phys_of(e, b) < 0 ? 1 : 0) << b;
    return bad;
  };
  // Loads of tile t into LDS buffer b: wave instruction j = 2*wave + r (of 16
  // per tensor) moves block j/4 of the tile, chunks 4(j%4) .. +3; lane i takes
  // chunk +i/16 at key position i%16.  Each instruction reads one block of
  // one kv head as a buffer of its valid keys only: keys past the item's end,
  // and every key of a block outside the pool, arrive as zeros (V must be
  // finite there: p = 0 times a stale NaN would poison the sum; K is masked).
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  constexpr int kRowBytes = D * 2;
  int dma_off[2];  // this lane's byte offset within the block, per instruction
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int ch = 4 * ((2 * wave + r) & 3) + (lane >> 4);
    dma_off[r] = ((lane & 15) ^ (4 * (ch & 3))) * kRowBytes + ch * 16;
  }
  // key tile `tile` (absolute) of an item with keys [0, kend_x) of kv head
  // kvh_x, into LDS buffer b
  auto issue_for = [&](int kend_x, int kvh_x, int tile, int b, int e) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int j = 2 * wave + r;
      const int blk = j >> 2, c0 = 4 * (j & 3);
      const int phys = phys_of(e, blk);              // wave-uniform
      // (readfirstlane: a buffer descriptor must be scalar)
      const int nvalid = __builtin_amdgcn_readfirstlane(
          phys < 0 ? 0 : min(max(kend_x - (tile * kKeyTile + blk * kBlockSize), 0), kBlockSize));
      const int64_t off = ((int64_t)max(phys, 0) * hkv + kvh_x) * (kBlockSize * kRowBytes);
      dma16(kc + off, nvalid * kRowBytes, dma_off[r], &sm.k[b][blk][c0][0]);
      dma16(vc + off, nvalid * kRowBytes, dma_off[r], &sm.v[b][blk][c0][0]);
    }
  };
  auto issue = [&](int t, int b, int e) { issue_for(kend, kvh, tile0 + t, b, e); };

  const float sl2 = a.scale * 1.4426950408889634f;
  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = kNegInf, lsum = 0.f;

  // S^T of a tile's two 32-key halves from LDS buffer b
  auto scores = [&](int b, f32x16_t(&sc)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[u][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int ch = 2 * ks + hi;
        const bf16x8_t kf = __builtin_bit_cast(
            bf16x8_t, sm.k[b][2 * u + (n >> 4)][ch][(n & 15) ^ (4 * (ch & 3))]);
        sc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sc[u], 0, 0, 0);
      }
    }
  };

  // V^T fragment of k step kb (a multiple of 16) and dims dt*32 .. +32: lane
  // l = 16g + s supplies dims dt*32 + 16(g%2) + 4(s%4) .. +3 of key
  // kb + 4(g/2) + s/4 (then of that key + 8); the transposing read hands lane
  // l the 4 keys of its dim dt*32 + l%32.
  const int vg = lane >> 4, vs = lane & 15;
  const int vch = 2 * (vg & 1) + ((vs & 3) >> 1);       // chunk within a 32-dim span
  int v_off[2];  // byte offsets within a V buffer of this lane's two reads at kb = 0, dt = 0
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k16 = 4 * (vg >> 1) + (vs >> 2) + 8 * h;
    v_off[h] = vch * 256 + (k16 ^ (4 * vch)) * 16 + 8 * (vs & 1);
  }
  const char* v_lds = reinterpret_cast<const char*>(&sm.v[0][0][0][0]);
  auto v_frag = [&](int b, int kb, int dt) -> bf16x8_t {
    uint2 w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[h] = lds_read_tr(reinterpret_cast<const uint16_t*>(
          v_lds + v_off[h] + b * (int)sizeof(sm.v[0]) + (kb >> 4) * 4096 + dt * 1024));
    return __builtin_bit_cast(bf16x8_t, make_uint4(w[0].x, w[0].y, w[1].x, w[1].y));
  };

  // Row maxima: mrun is the running maximum of the raw scores seen so far;
  // m is the reference the exponentials use, p = 2^((s - m) * scale * log2e).
  // m follows mrun lazily: only when some row's maximum has risen by more
  // than 2^kLazyRescale over its reference are the accumulators rescaled, so
  // p stays below 2^kLazyRescale and most tiles skip the 64 products.
  constexpr float kLazyRescale = 8.f;
  float mrun = kNegInf;

  // One key tile.  Its scores `cur` were computed one step earlier; this
  // step issues the products of tile t+1 into `nxt` (independent of the
  // softmax work on `cur`, so the matrix cores run while the vector ALUs do
  // the exponentials), then O += V^T P^T for tile t.
  //
  // The two waves of a SIMD (w and w+4) run the same steps half a step
  // apart: waves 0-3 meet the step's barrier after the PV products, waves
  // 4-7 between the score products and the PV products.  So while one does
  // the exponentials the other feeds the matrix core.  Between barriers t-1
  // and t, waves 0-3 do softmax(t), scores(t+1) and PV(t); waves 4-7 do
  // PV(t-1), softmax(t) and scores(t+1).
  //
  // Four LDS buffers, tile t in t%4: the loads of tile t+2 go out at the
  // start of step t into the buffer of tile t-2, whose last readers (PV(t-2):
  // waves 0-3 before barrier t-2, waves 4-7 before barrier t-1) are done, and
  // land before barrier t, after which scores(t+2) read them.  e2 holds the
  // table entries of tile t+2; bq the bad-block masks of tiles t, t+1 (and
  // t+2 once added) in 4-bit fields.
  const bool late = wave >= 4;
  int e2 = 0, bq = 0;
  auto step = [&](auto with_scores, int t, f32x16_t(&cur)[2], f32x16_t(&nxt)[2]) {
    constexpr bool kScores = decltype(with_scores)::value;
    const int bc = (tb + t) & 3;
    const int bn = (tb + t + 1) & 3;
    const int bs = (tb + t + 2) & 3;
    bq |= bad_mask(e2) << 8;  // (read e2 before the tile loads go out)
    if (t + 2 < ntiles) {
      issue(t + 2, bs, e2);
    } else if (has_next && t + 2 - ntiles == next_pre) {
      // the next item's tile next_pre into the buffer this item's tile t + 2
      // would take: its last readers (tile t - 2) passed barrier t - 1
      next = meta_of(a, nraw);
      const int kend_n = item_kend<G>(a, next);
      if (kend_n > 0) {
        issue_for(kend_n, next.kvh, next_pre, bs, next_pre == 0 ? next.e0 : next.e1);
        ++next_pre;
      }
    }
    if (!kScores && has_next) {
      // the last step: no score products, so the query registers are free
      // for the next item's rows
      next = meta_of(a, nraw);
      load_query<G, CASCADE>(a, next, qf);
      next_q = true;
    }
    e2 = entries(t + 3);
    const int bad = bq & 15;
    // cur[u][4i+j] is the raw score of key t*64 + 32u + 8i + 4hi + j for this
    // row; the running max m is kept in raw units (scale > 0 here: the host
    // turns other scales into that form through q_sign) and the scale is
    // folded into the exponent: p = 2^(s*scale*log2e - m*scale*log2e)
    const int kt0 = (tile0 + t) * kKeyTile;
    // every key of the tile visible to every row: no masking
    const bool full = bad == 0 && kt0 + kKeyTile <= full_lim;
    if (!full) {
      // keeps this block a real (uniform) branch instead of 32 selects on
      // every tile
      asm volatile("" ::: "memory");
      const int lim = row_lim - kt0 - 4 * hi;  // first masked offset of this lane
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // key kt0 + 32u + 8(r/4) + 4hi + r%4, in block 2u + r/8 of the tile
          if (32 * u + 8 * (r >> 2) + (r & 3) >= lim || ((bad >> (2 * u + (r >> 3))) & 1))
            cur[u][r] = kNegInf;
        }
    }
    float mm[4] = {kNegInf, kNegInf, kNegInf, kNegInf};  // independent chains
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        mm[(r >> 1) & 3] = __builtin_elementwise_maximum(
            mm[(r >> 1) & 3], __builtin_elementwise_maximum(cur[u][r], cur[u][r + 1]));
    const float mloc = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mm[0], mm[1]),
                                                     __builtin_elementwise_maximum(mm[2], mm[3]));
    // the row's other 32 keys sit in lane ^ 32
    const auto mx = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc),
                                                     false, false);
    mrun = __builtin_elementwise_maximum(
        mrun, __builtin_elementwise_maximum(__uint_as_float(mx[0]), __uint_as_float(mx[1])));
    if (__any((mrun - m) * sl2 > kLazyRescale)) {
      // kept a real branch so tiles that move no reference skip the products
      asm volatile("" ::: "memory");
      // 0 while m = -inf; 1 for a row that has seen no key yet (all of its
      // keys so far masked: nothing accumulated, and -inf - -inf is NaN)
      const float alpha = fast_exp2(mrun == kNegInf ? 0.f : (m - mrun) * sl2);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m = mrun;
    }
    // The next tile's score products (past the last tile they read a stale
    // buffer and are discarded), interleaved one for one with this tile's
    // exponentials so the matrix core and the vector ALU work at once; the
    // K reads run three products ahead.  sched_barrier keeps this order.
    const float moff = -((m == kNegInf) ? 0.f : m) * sl2;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};  // partial row sums (independent chains)
    uint32_t pf[16];  // P^T pairs: pf[8u + 4t2 + e/2] = scores 8t2 + e, +1 of half u
    auto kread = [&](int i) -> bf16x8_t {
      const int u = i >> 3, ch = 2 * (i & 7) + hi;
      return __builtin_bit_cast(bf16x8_t,
                                sm.k[bn][2 * u + (n >> 4)][ch][(n & 15) ^ (4 * (ch & 3))]);
    };
    bf16x8_t kq[4];
    if constexpr (kScores) {
      kq[0] = kread(0);
      kq[1] = kread(1);
      kq[2] = kread(2);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int u = i >> 3, ks = i & 7;
      if constexpr (kScores) {
        if (i + 3 < 16) kq[(i + 3) % 4] = kread(i + 3);
        if (ks == 0)
#pragma unroll
          for (int r = 0; r < 16; ++r) nxt[u][r] = 0.f;
        nxt[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[i % 4], qf[ks], nxt[u], 0, 0, 0);
      }
      const int r = 2 * (i & 7);
      const float p0 = fast_exp2(fmaf(cur[u][r], sl2, moff));
      const float p1 = fast_exp2(fmaf(cur[u][r + 1], sl2, moff));
      ps[i & 3] += p0 + p1;
      pf[i] = pack_f32_bf16(p0, p1);
      __builtin_amdgcn_sched_barrier(0);
    }
    lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // (the last step has no barrier: what it would publish -- the next
    // item's first tiles -- the next item's prologue waits for, and every
    // buffer the next item refills was last read before barrier t - 1)
    if (kScores && late) {
      // this wave's loads of tile t+2 (and the entries of tile t+3) have
      // landed; the barrier publishes them
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }

    // O^T += V^T P^T; k step ut = 2u + t2 covers keys 16ut + {8(e/4) + 4hi + e%4};
    // the V reads run three products ahead
    auto vread = [&](int j) -> bf16x8_t { return v_frag(bc, 16 * (j >> 2), j & 3); };
    bf16x8_t vq[4];
    vq[0] = vread(0);
    vq[1] = vread(1);
    vq[2] = vread(2);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j + 3 < 16) vq[(j + 3) % 4] = vread(j + 3);
      const int ut = j >> 2, dt = j & 3;
      const bf16x8_t pb = __builtin_bit_cast(
          bf16x8_t, make_uint4(pf[4 * ut], pf[4 * ut + 1], pf[4 * ut + 2], pf[4 * ut + 3]));
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[j % 4], pb, o[dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    bq >>= 4;
    if (kScores && !late) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  };

  // Tiles 0 and 1 go to buffers tb & 3 and (tb + 1) & 3, which the previous
  // item's last two tiles (the only ones it may still read after its final
  // barrier) do not use; the barrier below orders everything after that.
  if (ntiles > 0) {
    const int e0 = CASCADE ? entries(0) : im.e0;
    if (pipe.pre < 1) issue(0, tb & 3, e0);
    bq = bad_mask(e0);
    const int e1 = CASCADE ? entries(1) : im.e1;
    if (pipe.pre < 2 && ntiles > 1) issue(1, (tb + 1) & 3, e1);
    bq |= bad_mask(e1) << 4;
    e2 = CASCADE ? entries(2) : im.e2;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16_t sa[2], sb[2];
    scores(tb & 3, sa);
    // the next item's record, loaded beside this item's third tile
    if (has_next) nraw = load_rec<INL>(a, next_idx, list);
    for (int t = 0; t + 1 < ntiles; ++t) {
      step(std::true_type{}, t, sa, sb);
      sa[0] = sb[0];
      sa[1] = sb[1];
    }
    step(std::false_type{}, ntiles - 1, sa, sb);
  } else if (has_next) {
    nraw = load_rec<INL>(a, next_idx, list);
  }
  if (has_next) next = meta_of(a, nraw);
  pipe.tb = tb + max(ntiles, 0);
  pipe.pre = next_pre;
  pipe.q_ready = next_q;

  // this lane summed 32 of each tile's 64 keys; its partner lane^32 the rest
  const auto ls = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                   false, false);
  const float ltot = __uint_as_float(ls[0]) + __uint_as_float(ls[1]);
  if constexpr (CASCADE) {
    // partial slot `seq` (the split) of (sequence q0 + tok, head): the
    // reference the exponentials used, in log2 units, the sum and the
    // unnormalised accumulators
    if (valid_q) {
      const int64_t pidx = ((int64_t)(q0 + tok) * hq + head) * a.max_parts + seq;
      float* acc = a.part_acc + pidx * D;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(acc + dt * 32 + 8 * i + 4 * hi) =
              make_float4(o[dt][4 * i], o[dt][4 * i + 1], o[dt][4 * i + 2], o[dt][4 * i + 3]);
      if (hi == 0) {
        a.part_ml[pidx * 2] = m == kNegInf ? kNegInf : m * sl2;
        a.part_ml[pidx * 2 + 1] = ltot;
      }
    }
    return;
  }
  if (valid_q) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    uint16_t* out = static_cast<uint16_t*>(a.out) + ((int64_t)(lo_row + q0 + tok) * hq + head) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // dims dt*32 + 8i + 4hi + 0..3
        const int d = dt * 32 + 8 * i + 4 * hi;
        uint2 w;
        w.x = pack_f32_bf16(o[dt][4 * i + 0] * inv, o[dt][4 * i + 1] * inv);
        w.y = pack_f32_bf16(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(out + d) = w;
      }
  }
}

// Persistent workgroups, one per resident slot, walk the longest-first list
// in snake order (workgroup i takes ranks i, 2G-1-i, 2G+i, ... for G
// workgroups), which pairs long items with short ones, each item's start-up
// overlapped with the end of the one before.
// The work list built inside every workgroup (no plan launch): the same
// (sequence, query tile, kv head) items as the plan kernel lists, ordered by
// key tiles, most first, and within one count by (sequence, query tile) --
// a stable counting sort, so every workgroup derives the same order -- of
// which the workgroup keeps only the items of its own snake ranks, in `list`.
// Scratch: the tile buffers `w`, before any tile is loaded.  Returns the item
// count (every thread).  Needs num_seqs <= kInlineMaxSeqs, at most
// kInlineMaxPairs (sequence, query tile) pairs (more are dropped, as are
// items past work_cap: the host bounds both) and work_cap <= kListCap x grid.
constexpr int kInlineMaxSeqs = 4096;   // a pair's sequence takes 12 bits of its word
constexpr int kInlineMaxPairs = 7168;

// Exclusive scan over the workgroup of one value per thread: the thread's
// offset, and the sum in `total` (wt: one word per wave of scratch).
__device__ __forceinline__ int inline_scan(int v, int& total, int* wt) {
  constexpr int NW = kPrefillThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(inc, off);
    if (lane >= off) inc += up;
  }
  if (lane == 63) wt[wave] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = wt[w];
    base += w < wave ? x : 0;
    total += x;
  }
  __syncthreads();  // wt is reused by the next scan
  return base + inc - v;
}

__device__ int plan_inline(const PrefillArgs& a, int tile_tokens, int* w, ItemList& list) {
  constexpr int NT = kPrefillThreads, NW = NT / 64;
  constexpr int B = kSortBuckets;
  int* cnt = w;                            // [B] pairs per bucket, then first pair
  int* cw = cnt + B;                       // [NW][B] per-wave counts, then offsets
  int* scu = cw + NW * B;                  // [n + 1] first packed row of each sequence
  int* sctx = scu + kInlineMaxSeqs + 1;    // [n] cached tokens
  int* psq = sctx + kInlineMaxSeqs;        // [pairs] sequence | query tile << 12
  int* pkey = psq + kInlineMaxPairs;       // [pairs] bucket | rank among its wave's equals << 10
  int* wt = pkey + kInlineMaxPairs;        // [NW] scan scratch
  static_assert(kInlineMaxSeqs <= 4096, "sequence index in 12 bits");
  static_assert((NW + 1) * B + 2 * kInlineMaxSeqs + 1 + 2 * kInlineMaxPairs + NW <=
                    (int)(sizeof(PrefillShared) / sizeof(int)),
                "inline plan scratch fits the tile buffers");
  static_assert(B == 2 * NT, "two buckets per thread");
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = a.num_seqs, hkv = a.num_kv_heads;
  const int maxk = max(0, min(a.max_context_len, a.max_blocks_per_seq * kBlockSize));
  for (int i = t; i < (NW + 1) * B; i += NT) w[i] = 0;

  // sequences [s0, s0 + C) of this thread: lengths and cached counts into LDS,
  // and their query tiles (sequences of one row have none)
  const int C = ceil_div(n, NT);
  const int s0 = t * C;
  int mine = 0;
  for (int j = 0; j < C; ++j) {
    const int s = s0 + j;
    if (s >= n) break;
    const int lo = a.cu_seqlens[s], hi = a.cu_seqlens[s + 1];
    scu[s] = lo;
    sctx[s] = a.context_offsets[s];
    if (s == n - 1) scu[n] = hi;
    mine += hi - lo >= 2 ? ceil_div(hi - lo, tile_tokens) : 0;
  }
  int npairs = 0;
  int p = inline_scan(mine, npairs, wt);  // barrier: scu complete
  npairs = min(npairs, kInlineMaxPairs);
  for (int j = 0; j < C; ++j) {
    const int s = s0 + j;
    if (s >= n) break;
    const int len = scu[s + 1] - scu[s];
    const int nt = len >= 2 ? ceil_div(len, tile_tokens) : 0;
    for (int q = 0; q < nt && p < kInlineMaxPairs; ++q, ++p) psq[p] = s | (q << 12);
  }
  __syncthreads();

  auto bucket = [&](int s, int q) {
    const int len = scu[s + 1] - scu[s], c = sctx[s];
    const int qn = min(tile_tokens, len - q * tile_tokens);
    const int kend = max(0, min(c + q * tile_tokens + qn, maxk));
    return min(ceil_div(kend, kKeyTile), B - 1);
  };
  for (int i = t; i < npairs; i += NT) {
    const int b = bucket(psq[i] & 4095, psq[i] >> 12);
    pkey[i] = b;
    atomicAdd(&cnt[b], 1);
  }
  __syncthreads();
  // first pair of each bucket, largest bucket first: thread t owns buckets
  // B-1-2t and B-2-2t
  {
    const int b0 = B - 1 - 2 * t, b1 = b0 - 1;
    const int x0 = cnt[b0], x1 = cnt[b1];
    int unused;
    const int off = inline_scan(x0 + x1, unused, wt);
    cnt[b0] = off;
    cnt[b1] = off + x0;
  }
  // stable rank among equal buckets: wave v walks pairs [v S, (v + 1) S) 64 at
  // a time; the lanes holding one bucket find each other by ballots over its
  // bits, and the lowest of them advances the wave's count for that bucket
  const int S = ceil_div(npairs, NW);
  {
    int* mycw = cw + wave * B;
    const int end = min(npairs, (wave + 1) * S);
    for (int base = wave * S; base < end; base += 64) {
      const int i = base + lane;
      const bool valid = i < end;
      const int b = valid ? pkey[i] : 0;
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 10; ++bit) {
        const bool on = (b >> bit) & 1;
        const uint64_t m = __ballot(valid && on);
        peers &= on ? m : ~m;
      }
      const int below = __popcll(peers & ((1ull << lane) - 1ull));
      const int old = valid ? mycw[b] : 0;
      if (valid && below == 0) mycw[b] = old + __popcll(peers);
      if (valid) pkey[i] = b | ((old + below) << 10);
    }
  }
  __syncthreads();
  // per bucket: the waves' counts -> each wave's first rank
  for (int b = t; b < B; b += NT) {
    int pre = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int x = cw[v * B + b];
      cw[v * B + b] = pre;
      pre += x;
    }
  }
  __syncthreads();
  // place: pair i's items are pos*hkv + h; keep those of this workgroup's
  // snake ranks (rank k*G + j belongs to workgroup j for even k, G-1-j odd)
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int total = min(npairs * hkv, a.work_cap);
  for (int i = t; i < npairs; i += NT) {
    const int key = pkey[i];
    const int b = key & (B - 1);
    const int pos = cnt[b] + cw[(i / S) * B + b] + (key >> 10);
    const int s = psq[i] & 4095, q = psq[i] >> 12;
    const int lo = scu[s], len = scu[s + 1] - lo, c = sctx[s];
    for (int h = 0; h < hkv; ++h) {
      const int idx = pos * hkv + h;
      if (idx >= total) break;
      const int k = idx / nwg, j = idx - k * nwg;
      if (((k & 1) ? nwg - 1 - j : j) == wg && k < kListCap) {
        list.m[k] = make_int4(s, q * hkv + h, lo, len);
        list.c[k] = c;
      }
    }
  }
  __syncthreads();  // the list is complete and the scratch free for tiles
  return total;
}

template <int G, bool INL>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillArgs a) {
  __shared__ PrefillShared sm;
  __shared__ std::conditional_t<INL, ItemList, int> own;  // this workgroup's items (INL)
  const ItemList* list = nullptr;
  int total;
  if constexpr (INL) {
    total = plan_inline(a, kPrefillRows / G, reinterpret_cast<int*>(&sm), own);
    list = &own;
  } else {
    total = a.work[0];
  }
  const int nwg = gridDim.x, wg = blockIdx.x;
  auto rank = [&](int k) { return k * nwg + ((k & 1) ? nwg - 1 - wg : wg); };
  if (rank(0) >= total) return;
  PipeState ps;
  ps.tb = 0;
  ps.pre = 0;
  ps.q_ready = false;
  ItemMeta cur = meta_of(a, load_rec<INL>(a, INL ? 0 : rank(0), list));
  for (int k = 0;; ++k) {
    const int nidx = rank(k + 1);  // ranks grow with k: past the end, done
    ItemMeta next;
    prefill_item<G, false, INL>(a, cur, sm, ps, nidx < total ? (INL ? k + 1 : nidx) : -1, list,
                                next);
    if (nidx >= total) break;
    cur = next;
  }
}

// Common-prefix pass: item (split, row tile, kv head) = (x, y, z).
template <int G>
__global__ __launch_bounds__(kPrefillThreads) void cascade_prefix_kernel(PrefillArgs a) {
  __shared__ PrefillShared sm;
  ItemMeta im{};
  im.seq = blockIdx.x;
  im.qtile = blockIdx.y;
  im.kvh = blockIdx.z;
  PipeState ps;
  ps.tb = 0;
  ps.pre = 0;
  ps.q_ready = false;
  ItemMeta none;
  prefill_item<G, true>(a, im, sm, ps, -1, nullptr, none);
}

static int prefill_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

template <int G>
static hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t stream) {
  // resident workgroups per CU (computed once; concurrent first calls compute
  // the same value)
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(&prefill_kernel<G, true>), kPrefillThreads, 0) !=
            hipSuccess ||
        nb <= 0)
      nb = 1;
    per_cu = nb;
    per_cu_cache.store(nb, std::memory_order_relaxed);
  }
  // one workgroup per resident slot, each walking its share of the list
  // (tuning override PA_PREFILL_GRID)
  int64_t want = (int64_t)per_cu * prefill_cus();
  const char* eg = getenv("PA_PREFILL_GRID");
  if (eg && *eg && atoi(eg) >= 1) want = atoi(eg);
  const int gx = (int)std::max<int64_t>(1, std::min<int64_t>(a.work_cap, want));
  // the work list: built inside every workgroup where its bounds allow
  // (sequences, (sequence, query tile) pairs -- each sequence of two or more
  // rows has at most rows / tile + 1 of them, and at most rows / 2 -- and
  // items per workgroup), else by the one-workgroup plan kernel
  // (PA_PREFILL_INLINE_PLAN=0 forces the plan kernel)
  const int tile = prefill_tile_tokens(G);
  const int64_t multi = std::min<int64_t>(a.num_seqs, a.total_q_tokens / 2);
  const int64_t pairs_bound = std::min<int64_t>((int64_t)a.total_q_tokens / tile + multi + 1,
                                                (int64_t)a.total_q_tokens / 2 + 1);
  const char* ei = getenv("PA_PREFILL_INLINE_PLAN");
  const bool inline_plan = (!ei || atoi(ei) != 0) && a.num_seqs <= kInlineMaxSeqs &&
                           pairs_bound <= kInlineMaxPairs && ceil_div(a.work_cap, gx) <= kListCap;
  if (!inline_plan) {
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a, tile);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (inline_plan)
    hipLaunchKernelGGL((prefill_kernel<G, true>), dim3(gx), dim3(kPrefillThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<G, false>), dim3(gx), dim3(kPrefillThreads), 0, stream, a);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_cascade_g(const PrefillArgs& a, int splits, hipStream_t stream) {
  const dim3 grid(splits, ceil_div(a.num_seqs, prefill_tile_tokens(G)), a.num_kv_heads);
  hipLaunchKernelGGL((cascade_prefix_kernel<G>), grid, dim3(kPrefillThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_cascade_prefix(const PrefillArgs& a, int splits, hipStream_t stream) {
  if (a.head_dim != kPrefillD || splits <= 0) return hipErrorInvalidValue;
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_cascade_g<1>(a, splits, stream);
    case 2: return launch_cascade_g<2>(a, splits, stream);
    case 4: return launch_cascade_g<4>(a, splits, stream);
    case 8: return launch_cascade_g<8>(a, splits, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.head_dim != kPrefillD) return hipErrorInvalidValue;
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_prefill_g<1>(a, stream);
    case 2: return launch_prefill_g<2>(a, stream);
    case 4: return launch_prefill_g<4>(a, stream);
    case 8: return launch_prefill_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
