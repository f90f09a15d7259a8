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
//     block table into double-buffered LDS: K row-major [key][dim], V
//     transposed [dim][key].  One barrier per tile: tile t is computed while
//     tile t+1 is staged and the loads of tile t+2 are in flight;
//   * the work list is ordered longest first (key tiles per item);
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
//     on the way into LDS (p = 0 times a stale NaN would poison the sum).

#include <math.h>

#include <algorithm>

#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPrefillD = 128;
constexpr int kPrefillWaves = 8;             // two waves per SIMD share every K/V tile
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr int kPrefillRows = 32 * kPrefillWaves;  // (head, token) rows per item
constexpr int kKeyTile = 64;                 // keys per tile = 4 physical blocks
constexpr int kSortBuckets = 1024;           // work-list order: key tiles per item (capped)
constexpr int kKRow = kPrefillD + 8;         // LDS row of K, bf16 elements (padded)
constexpr int kVRow = kKeyTile + 4;          // LDS row of V^T, bf16 elements (padded)

int prefill_tile_tokens(int group) { return kPrefillRows / group; }

int prefill_work_capacity(int num_seqs, int total_q_tokens, int num_kv_heads, int group) {
  const int t = prefill_tile_tokens(group);
  return (total_q_tokens / t + num_seqs + 1) * num_kv_heads;
}

// Work list in the workspace: int32 count, int32 pad, then int2
// (seq, tile * num_kv_heads + kv head).
__device__ __forceinline__ int2* prefill_items(int32_t* work) {
  return reinterpret_cast<int2*>(work + 2);
}

// One workgroup lists the (sequence, query tile, kv head) items of every
// sequence with two or more query rows, ordered by the number of 64-key tiles
// they stream, most first (a counting sort in LDS), so the persistent
// workgroups start the longest items first, on every CU at once.  The order
// among equal counts is arbitrary: items are independent and each writes only
// its own rows.
__global__ __launch_bounds__(1024) void prefill_plan_kernel(PrefillArgs a, int tile_tokens) {
  __shared__ int count[kSortBuckets];
  const int n = a.num_seqs;
  const int t = threadIdx.x;
  const int maxk = max(0, min(a.max_context_len, a.max_blocks_per_seq * kBlockSize));
  for (int i = t; i < kSortBuckets; i += blockDim.x) count[i] = 0;
  __syncthreads();
  auto bucket = [&](int s, int q) {
    const int len = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
    const int qn = min(tile_tokens, len - q * tile_tokens);
    const int kend = max(0, min(a.context_offsets[s] + q * tile_tokens + qn, maxk));
    return min(ceil_div(kend, kKeyTile), kSortBuckets - 1);
  };
  for (int s = t; s < n; s += blockDim.x) {
    const int len = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
    if (len < 2) continue;
    const int nt = ceil_div(len, tile_tokens);
    for (int q = 0; q < nt; ++q) atomicAdd(&count[bucket(s, q)], a.num_kv_heads);
  }
  __syncthreads();
  // exclusive offsets, largest bucket first: thread t owns bucket 1023 - t and
  // the counts are scanned over t
  static_assert(kSortBuckets == 1024, "one bucket per thread");
  __shared__ int scan[kSortBuckets];
  const int mine = count[kSortBuckets - 1 - t];
  scan[t] = mine;
  __syncthreads();
  for (int off = 1; off < kSortBuckets; off <<= 1) {
    const int add = t >= off ? scan[t - off] : 0;
    __syncthreads();
    scan[t] += add;
    __syncthreads();
  }
  count[kSortBuckets - 1 - t] = scan[t] - mine;
  if (t == kSortBuckets - 1) a.work[0] = min(scan[t], a.work_cap);
  __syncthreads();
  int2* items = prefill_items(a.work);
  for (int s = t; s < n; s += blockDim.x) {
    const int len = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
    if (len < 2) continue;
    const int nt = ceil_div(len, tile_tokens);
    for (int q = 0; q < nt; ++q) {
      const int pos = atomicAdd(&count[bucket(s, q)], a.num_kv_heads);
      for (int h = 0; h < a.num_kv_heads; ++h)
        if (pos + h < a.work_cap) items[pos + h] = make_int2(s, q * a.num_kv_heads + h);
    }
  }
}

// LDS tiles typed by their access width (16-byte K pieces, 4-byte key pairs
// of V^T) so that every access is provably aligned.
struct __attribute__((aligned(16))) PrefillShared {
  uint4 k[2][kKeyTile][kKRow / 8];      // double-buffered K tile [key][dim / 8]
  uint32_t vt[2][kPrefillD][kVRow / 2];  // double-buffered V^T tile [dim][key / 2]
};

// pack the low (or high) bf16 halves of two words: (lo of a) | (lo of b) << 16
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ uint32_t word(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_f32_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <int G>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, int seq, int qtile, int kvh,
                                             PrefillShared& sm) {
  constexpr int D = kPrefillD;
  constexpr int BMT = kPrefillRows / G;  // query tokens per item
  constexpr float kNegInf = -INFINITY;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;             // this lane's query row within the wave
  const int hi = lane >> 5;            // which half of each 16-element k step

  const int lo_row = a.cu_seqlens[seq];
  const int len = a.cu_seqlens[seq + 1] - lo_row;
  const int c = a.context_offsets[seq];
  const int q0 = qtile * BMT;
  const int qn = min(BMT, len - q0);   // valid query tokens of this tile (>= 1)
  const int rho = wave * 32 + n;       // row of the item: (head_local, token)
  const int head = kvh * G + rho / BMT;
  const int tok = rho % BMT;
  // rows outside the packed q / out arrays (inconsistent metadata) are skipped
  const bool valid_q =
      tok < qn && lo_row >= 0 && (int64_t)lo_row + q0 + tok < (int64_t)a.total_q_tokens;
  const int qpos = c + q0 + tok;       // absolute position of this row
  // keys any row of the item sees, clamped to the declared maxima
  const int kend = max(0, min(c + q0 + qn, min(a.max_context_len, a.max_blocks_per_seq * kBlockSize)));
  const int row_lim = valid_q ? min(qpos + 1, kend) : 0;  // keys [0, row_lim) are visible
  const int full_lim = min(c + q0 + 1, kend);  // keys every row of the item sees
  const int ntiles = ceil_div(kend, kKeyTile);
  const int hkv = a.num_kv_heads;
  const int hq = a.num_q_heads;
  const int32_t* table = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;

  // B operand of S^T = K Q^T: this lane's query row, dims ks*16 + hi*8 .. +8
  bf16x8_t qf[8];
  {
    const uint4* qrow = static_cast<const uint4*>(a.q) +
                        ((int64_t)(valid_q ? lo_row + q0 + tok : 0) * hq + head) * (D / 8);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 v = qrow[ks * 2 + hi];
      if (!valid_q) v = make_uint4(0u, 0u, 0u, 0u);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // tile staging (512 threads): thread tid holds K pieces tid and tid + 512 of
  // the tile's 4 blocks (a block tile is 256 pieces of 16 bytes), and V of keys
  // 2*(tid/16), +1 at dims (tid%16)*8 .. +8
  const uint4* kc = static_cast<const uint4*>(a.k_cache);
  const uint4* vc = static_cast<const uint4*>(a.v_cache);
  constexpr int kTilePieces = kBlockSize * D / 8;  // 16-byte pieces per block tile
  uint4 k0, k1, v0, v1;  // the next tile's K and V pieces, in flight
  auto block_of = [&](int logical) -> int {
    const int lb = min(logical, a.max_blocks_per_seq - 1);
    const int phys = table[lb];
    return (phys >= 0 && (int64_t)phys < a.num_blocks) ? phys : -1;
  };
  auto k_piece = [&](int tile, int piece) -> uint4 {
    const int phys = block_of(tile * 4 + piece / kTilePieces);
    const int64_t base = ((int64_t)max(phys, 0) * hkv + kvh) * kTilePieces;
    return kc[base + piece % kTilePieces];
  };
  auto fetch = [&](int tile) {
    k0 = k_piece(tile, tid);
    k1 = k_piece(tile, tid + kPrefillThreads);
    const int key0 = 2 * (tid >> 4);                 // first of this thread's 2 keys
    const int phys = block_of(tile * 4 + key0 / kBlockSize);
    const int64_t base = ((int64_t)max(phys, 0) * hkv + kvh) * kTilePieces +
                         (key0 % kBlockSize) * (D / 8) + (tid & 15);
    v0 = vc[base];
    v1 = vc[base + D / 8];
    // V of keys past the chunk's end (or in an unusable block) must not reach
    // the products (p = 0 times a stale NaN is NaN): select zero instead
    const int key = tile * kKeyTile + key0;
    if (phys < 0 || key >= kend) v0 = make_uint4(0u, 0u, 0u, 0u);
    if (phys < 0 || key + 1 >= kend) v1 = make_uint4(0u, 0u, 0u, 0u);
  };
  auto stage_k = [&](int buf, int piece, uint4 v) {
    const int key = (piece / kTilePieces) * kBlockSize + (piece % kTilePieces) / 16;
    sm.k[buf][key][piece & 15] = v;
  };
  auto stage = [&](int buf) {
    stage_k(buf, tid, k0);
    stage_k(buf, tid + kPrefillThreads, k1);
    const int key0 = 2 * (tid >> 4);
    const int d0 = (tid & 15) * 8;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dims d0 + 2w (low halves) and d0 + 2w + 1 (high halves) of the 2 keys
      const uint32_t a0 = word(v0, w), a1 = word(v1, w);
      sm.vt[buf][d0 + 2 * w][key0 / 2] = pack_lo(a0, a1);
      sm.vt[buf][d0 + 2 * w + 1][key0 / 2] = pack_hi(a0, a1);
    }
  };

  const float sl2 = a.scale * 1.4426950408889634f;
  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = kNegInf, lsum = 0.f;

  // Double-buffered LDS tiles, one barrier per tile: tile t is computed from
  // LDS buffer t%2 while tile t+1 (already in registers) is staged into the
  // other buffer and the loads of tile t+2 go out.
  if (ntiles > 0) {
    fetch(0);
    stage(0);
    if (ntiles > 1) fetch(1);
  }
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    // blocks of this tile outside the pool take no part (bit b: block b of 4)
    int bad = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) bad |= (block_of(tile * 4 + b) < 0 ? 1 : 0) << b;
    // S^T for the tile's two 32-key halves
    f32x16_t s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[u][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, sm.k[buf][32 * u + n][ks * 2 + hi]);
        s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[u], 0, 0, 0);
      }
    }
    // s[u][4i+j] is the raw score of key tile*64 + 32u + 8i + 4hi + j for this
    // row; the running max m is kept in raw units (scale > 0) and the scale
    // is folded into the exponent: p = 2^(s*scale*log2e - m*scale*log2e)
    const int kt0 = tile * kKeyTile;
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
            s[u][r] = kNegInf;
        }
    }
    float mloc = kNegInf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mloc = fmaxf(mloc, fmaxf(s[u][r], s[u][r + 1]));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mn = fmaxf(m, mloc);
    if (__any(mn != m)) {
      // some row's max moved: rescale (rows whose max did not move get 1);
      // kept a real branch so tiles that move no max skip the 64 products
      asm volatile("" ::: "memory");
      const float alpha = fast_exp2((m - ((mn == kNegInf) ? 0.f : mn)) * sl2);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m = mn;
    }
    const float moff = -((m == kNegInf) ? 0.f : m) * sl2;
    float psum = 0.f;
    uint32_t pf[2][2][4];  // P^T fragments: [half u][16-key step t2][packed pairs]
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = fast_exp2(fmaf(s[u][8 * t2 + e], sl2, moff));
          const float p1 = fast_exp2(fmaf(s[u][8 * t2 + e + 1], sl2, moff));
          psum += p0 + p1;
          pf[u][t2][e / 2] = pack_f32_bf16(p0, p1);
        }
    lsum += psum;

    // O^T += V^T P^T; k step (u, t2) covers keys 32u + 16t2 + {8(e/4) + 4hi + e%4}
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const bf16x8_t pb = __builtin_bit_cast(
            bf16x8_t, make_uint4(pf[u][t2][0], pf[u][t2][1], pf[u][t2][2], pf[u][t2][3]));
        const int kb = 32 * u + 16 * t2 + 4 * hi;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint32_t* vrow = &sm.vt[buf][dt * 32 + n][kb / 2];
          const bf16x8_t vf =
              __builtin_bit_cast(bf16x8_t, make_uint4(vrow[0], vrow[1], vrow[4], vrow[5]));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[dt], 0, 0, 0);
        }
      }
    if (tile + 1 < ntiles) {
      stage(buf ^ 1);
      if (tile + 2 < ntiles) fetch(tile + 2);
    }
    __syncthreads();  // tile+1 staged for all; everyone is done with buffer `buf`
  }

  // this lane summed 32 of each tile's 64 keys; its partner lane^32 the rest
  const float ltot = lsum + __shfl_xor(lsum, 32);
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

template <int G>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillArgs a) {
  __shared__ PrefillShared sm;
  const int total = a.work[0];
  const int2* items = prefill_items(a.work);
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int2 w = items[it];
    prefill_item<G>(a, w.x, w.y / a.num_kv_heads, w.y % a.num_kv_heads, sm);
  }
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
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, stream, a, prefill_tile_tokens(G));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  static int per_cu = 0;
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(&prefill_kernel<G>), kPrefillThreads, 0) !=
            hipSuccess ||
        nb <= 0)
      nb = 1;
    per_cu = nb;
  }
  const int64_t want = (int64_t)2 * per_cu * prefill_cus();
  const int gx = (int)std::max<int64_t>(1, std::min<int64_t>(a.work_cap, want));
  hipLaunchKernelGGL((prefill_kernel<G>), dim3(gx), dim3(kPrefillThreads), 0, stream, a);
  return hipGetLastError();
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
