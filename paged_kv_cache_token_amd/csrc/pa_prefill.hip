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
//   * a work item is (sequence, tile of 128/g query tokens) for one kv head; its
//     128 rows are the g query heads of that kv head times the tile's tokens,
//     32 rows per wave, so each K/V tile read serves all g heads;
//   * keys stream in tiles of 64 (4 physical blocks), gathered through the
//     block table into LDS: K row-major [key][dim], V transposed [dim][key].
//     The next tile's global loads are in flight while the current one is
//     computed;
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
constexpr int kKeyTile = 64;                 // keys per tile = 4 physical blocks
constexpr int kKRow = kPrefillD + 8;         // LDS row of K, bf16 elements (padded)
constexpr int kVRow = kKeyTile + 4;          // LDS row of V^T, bf16 elements (padded)

int prefill_tile_tokens(int group) { return 128 / group; }

int prefill_work_capacity(int num_seqs, int total_q_tokens, int group) {
  const int t = prefill_tile_tokens(group);
  return total_q_tokens / t + num_seqs + 1;
}

// Work list in the workspace: int32 count, int32 pad, then int2 (seq, tile).
__device__ __forceinline__ int2* prefill_items(int32_t* work) {
  return reinterpret_cast<int2*>(work + 2);
}

// One workgroup lists the (sequence, query tile) items of every sequence with
// two or more query rows, in sequence order, each sequence's tiles from the
// last (most keys) to the first.
__global__ __launch_bounds__(1024) void prefill_plan_kernel(PrefillArgs a, int tile_tokens) {
  __shared__ int scan[1024];
  const int n = a.num_seqs;
  const int t = threadIdx.x;
  const int chunk = ceil_div(n, (int)blockDim.x);
  const int s0 = min(n, t * chunk);
  const int s1 = min(n, s0 + chunk);
  int mine = 0;
  for (int s = s0; s < s1; ++s) {
    const int len = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
    if (len >= 2) mine += ceil_div(len, tile_tokens);
  }
  scan[t] = mine;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    const int add = t >= off ? scan[t - off] : 0;
    __syncthreads();
    scan[t] += add;
    __syncthreads();
  }
  int pos = scan[t] - mine;
  int2* items = prefill_items(a.work);
  for (int s = s0; s < s1; ++s) {
    const int len = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
    if (len < 2) continue;
    const int nt = ceil_div(len, tile_tokens);
    for (int q = nt - 1; q >= 0; --q, ++pos)
      if (pos < a.work_cap) items[pos] = make_int2(s, q);
  }
  if (t == (int)blockDim.x - 1) a.work[0] = min(scan[t], a.work_cap);
}

struct PrefillShared {
  uint16_t k[kKeyTile][kKRow];
  uint16_t vt[kPrefillD][kVRow];
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
__device__ __forceinline__ uint32_t pack_f32_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

template <int G>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, int seq, int qtile, int kvh,
                                             PrefillShared& sm) {
  constexpr int D = kPrefillD;
  constexpr int BMT = 128 / G;         // query tokens per item
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
  const int row_lim = valid_q ? qpos + 1 : 0;  // keys [0, row_lim) are visible
  // keys any row of the item sees, clamped to the declared maxima
  const int kend = max(0, min(c + q0 + qn, min(a.max_context_len, a.max_blocks_per_seq * kBlockSize)));
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

  // tile staging: thread tid holds K piece tid of each of the 4 blocks, and V
  // of keys 4*(tid/16) .. +3 at dims (tid%16)*8 .. +8
  const uint4* kc = static_cast<const uint4*>(a.k_cache);
  const uint4* vc = static_cast<const uint4*>(a.v_cache);
  uint4 kreg[4], vreg[4];
  auto block_of = [&](int logical) -> int {
    const int lb = min(logical, a.max_blocks_per_seq - 1);
    const int phys = table[lb];
    return (phys >= 0 && (int64_t)phys < a.num_blocks) ? phys : -1;
  };
  auto fetch = [&](int tile) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int phys = block_of(tile * 4 + p);
      const int64_t base = ((int64_t)max(phys, 0) * hkv + kvh) * (kBlockSize * D / 8);
      kreg[p] = kc[base + tid];
      if (phys < 0) kreg[p] = make_uint4(0u, 0u, 0u, 0u);
    }
    const int key0 = 4 * (tid >> 4);                 // first of this thread's 4 keys
    const int phys = block_of(tile * 4 + key0 / kBlockSize);
    const int64_t base = ((int64_t)max(phys, 0) * hkv + kvh) * (kBlockSize * D / 8) +
                         (key0 % kBlockSize) * (D / 8) + (tid & 15);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      vreg[kk] = vc[base + kk * (D / 8)];
      // keys past the chunk's end (or in an unusable block) must not reach the
      // products: zero them here
      if (phys < 0 || tile * kKeyTile + key0 + kk >= kend) vreg[kk] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int p = 0; p < 4; ++p)
      *reinterpret_cast<uint4*>(&sm.k[p * kBlockSize + (tid >> 4)][(tid & 15) * 8]) = kreg[p];
    const int key0 = 4 * (tid >> 4);
    const int d0 = (tid & 15) * 8;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dims d0 + 2w (low halves) and d0 + 2w + 1 (high halves) of the 4 keys
      const uint32_t a0 = word(vreg[0], w), a1 = word(vreg[1], w);
      const uint32_t a2 = word(vreg[2], w), a3 = word(vreg[3], w);
      uint2 even = make_uint2(pack_lo(a0, a1), pack_lo(a2, a3));
      uint2 odd = make_uint2(pack_hi(a0, a1), pack_hi(a2, a3));
      *reinterpret_cast<uint2*>(&sm.vt[d0 + 2 * w][key0]) = even;
      *reinterpret_cast<uint2*>(&sm.vt[d0 + 2 * w + 1][key0]) = odd;
    }
  };

  const float sl2 = a.scale * 1.4426950408889634f;
  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = kNegInf, lsum = 0.f;

  fetch(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();  // the previous tile's LDS reads are done
    stage();
    __syncthreads();
    if (tile + 1 < ntiles) fetch(tile + 1);

    // S^T for the tile's two 32-key halves
    f32x16_t s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[u][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t*>(&sm.k[32 * u + n][ks * 16 + hi * 8]);
        s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[u], 0, 0, 0);
      }
    }
    // s[u][4i+j] is the score of key tile*64 + 32u + 8i + 4hi + j for this row
    const int kt0 = tile * kKeyTile;
    const bool full = kt0 + kKeyTile <= c + q0 + 1;  // every key visible to every row
    float mloc = kNegInf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[u][r] * sl2;
        if (!full) {
          const int key = kt0 + 32 * u + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= row_lim) x = kNegInf;
        }
        s[u][r] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mn = fmaxf(m, mloc);
    const float mref = (mn == kNegInf) ? 0.f : mn;
    const float alpha = fast_exp2(m - mref);
    m = mn;
    float psum = 0.f;
    uint32_t pf[2][2][4];  // P^T fragments: [half u][16-key step t2][packed pairs]
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = fast_exp2(s[u][8 * t2 + e] - mref);
          const float p1 = fast_exp2(s[u][8 * t2 + e + 1] - mref);
          psum += p0 + p1;
          pf[u][t2][e / 2] = pack_f32_bf16(p0, p1);
        }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

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
          const uint2 v0 = *reinterpret_cast<const uint2*>(&sm.vt[dt * 32 + n][kb]);
          const uint2 v1 = *reinterpret_cast<const uint2*>(&sm.vt[dt * 32 + n][kb + 8]);
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[dt], 0, 0, 0);
        }
      }
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
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  __shared__ PrefillShared sm;
  const int total = a.work[0];
  const int2* items = prefill_items(a.work);
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int2 w = items[it];
    prefill_item<G>(a, w.x, w.y, blockIdx.y, sm);
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
            &nb, reinterpret_cast<const void*>(&prefill_kernel<G>), 256, 0) != hipSuccess ||
        nb <= 0)
      nb = 1;
    per_cu = nb;
  }
  const int64_t want = (int64_t)2 * per_cu * prefill_cus();
  const int gx = (int)std::max<int64_t>(
      1, std::min<int64_t>(a.work_cap, (want + a.num_kv_heads - 1) / a.num_kv_heads));
  hipLaunchKernelGGL((prefill_kernel<G>), dim3(gx, a.num_kv_heads), dim3(256), 0, stream, a);
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
