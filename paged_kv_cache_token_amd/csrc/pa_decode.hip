// pa_decode.hip -- paged decode attention: split-K over fixed partitions of the
// context, online softmax, and a cross-partition combine.
//
// "vLLM：颠覆大模型推理的高效API服务引擎深度解析", §1.3 (attention reads the
// blocks scattered over the pool through the block table) and §2.2 (one fused
// kernel reads the KV cache straight from the physical blocks);
// "vLLM изнутри: как устроен движок для быстрого инференса LLM", the paragraph on
// the stages of a step (decode reads every cached K/V for one query token and
// is bound by memory bandwidth).  The split of the softmax over partitions with
// a later rescaled merge is the chunked-attention idea named in
// "vLLMつかったら、ベクトル検索サーバーが高速化して安定性も向上した" (the
// flash-attention paragraph: attention computed in small pieces in on-chip
// memory).
//
// Work decomposition (gfx950, wave64):
//   * one workgroup = one (sequence, kv head, partition of kPartitionTokens
//     tokens); it serves all g query heads that share the kv head, so every K/V
//     tile is read from HBM once per step;
//   * 4 waves per workgroup take the partition's 16-token blocks round-robin;
//     each wave keeps the next block's K and V in registers while it computes
//     the current one;
//   * a (block, kv head) tile is 16 * head_dim contiguous elements, so one
//     wave-wide 16-byte-per-lane load reads 1 KB of consecutive memory; lane l
//     holds the 16-byte piece (l % LPT) of token row (l / LPT) + k * (64 / LPT);
//   * q.k partial sums over a lane's piece are finished with DPP all-reduces
//     inside the LPT-lane group that holds one token row (LPT = 16 for bf16 at
//     head_dim 128: exactly one DPP row);
//   * each lane group keeps its own running (max, sum, accumulator) over the
//     token rows it holds; groups are merged once at the end, first across the
//     wave with lane exchanges, then across the 4 waves in LDS;
//   * a partition's result goes straight to `out` when the sequence has a
//     single partition; otherwise (max, sum, accumulator) go to the workspace
//     and a second kernel merges the partitions in fixed order.
// The order of every sum depends only on logical token positions, never on the
// physical block ids, so the output is bit-identical under any placement or
// sharing of blocks.

#include <math.h>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot_piece(uint4 q, uint4 k, std::true_type /*bf16*/) {
  float s = 0.f;
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x),
                                      __builtin_bit_cast(bf16x2_t, k.x), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y),
                                      __builtin_bit_cast(bf16x2_t, k.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z),
                                      __builtin_bit_cast(bf16x2_t, k.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w),
                                      __builtin_bit_cast(bf16x2_t, k.w), s, false);
  return s;
}

__device__ __forceinline__ float dot_piece(uint4 q, uint4 k, std::false_type /*f32*/) {
  float s = __uint_as_float(q.x) * __uint_as_float(k.x);
  s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
  s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
  s = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
  return s;
}

// element e of a 16-byte piece as fp32
template <bool BF16>
__device__ __forceinline__ float piece_elem(const uint4& v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (BF16) {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  } else {
    return __uint_as_float(w[e]);
  }
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float x) {
  if constexpr (BF16) {
    static_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(x);
  } else {
    static_cast<float*>(base)[idx] = x;
  }
}

// Resolve the row of q/out and the attended length for workgroup's sequence.
// Returns false when this sequence is not handled by the decode kernels.
template <bool VARLEN>
__device__ __forceinline__ bool decode_row(const DecodeArgs& a, int seq, int& qrow, int& ctx) {
  if constexpr (VARLEN) {
    const int lo = a.cu_seqlens[seq];
    if (a.cu_seqlens[seq + 1] - lo != 1) return false;
    qrow = lo;
    ctx = a.context_offsets[seq] + 1;
  } else {
    qrow = seq;
    ctx = a.context_lens[seq];
  }
  ctx = max(0, min(ctx, min(a.max_context_len, a.max_blocks_per_seq * kBlockSize)));
  return true;
}

template <bool BF16, int D, int G, bool VARLEN>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeArgs a) {
  using IsBF16 = std::integral_constant<bool, BF16>;
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int EPL = 16 / EB;              // elements in a lane's 16-byte piece
  constexpr int LPT = D / EPL;              // lanes holding one token row
  constexpr int TPL = 64 / LPT;             // token rows per wave-wide load
  constexpr int NLD = kBlockSize / TPL;     // wave-wide loads per 16-token tile
  constexpr int TILE_PIECES = kBlockSize * LPT;
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "piece layout");
  constexpr float kNegInf = -INFINITY;

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  int qrow, ctx;
  if (!decode_row<VARLEN>(a, seq, qrow, ctx)) return;
  const int nparts = max(1, ceil_div(ctx, kPartitionTokens));
  if (part >= nparts) return;

  const int tok0 = part * kPartitionTokens;
  const int tok1 = min(ctx, tok0 + kPartitionTokens);
  const int nblk = tok1 > tok0 ? ceil_div(tok1 - tok0, kBlockSize) : 0;
  const int32_t* table =
      a.block_tables + (int64_t)seq * a.max_blocks_per_seq + tok0 / kBlockSize;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane / LPT;
  const int col = lane % LPT;
  const int hq = a.num_q_heads;
  const int hkv = a.num_kv_heads;

  // this lane's piece of the g query heads that read kv head `kvh`
  uint4 qv[G];
  {
    const uint4* qb = static_cast<const uint4*>(a.q) + ((int64_t)qrow * hq + kvh * G) * LPT + col;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = qb[h * LPT];
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const float sl2 = a.scale * 1.4426950408889634f;  // scores in log2 units
  const uint4* kc = static_cast<const uint4*>(a.k_cache);
  const uint4* vc = static_cast<const uint4*>(a.v_cache);

  auto load = [&](int b, uint4* kr, uint4* vr) -> bool {
    const int phys = table[b];
    if (phys < 0 || (int64_t)phys >= a.num_blocks) return false;
    const int64_t base = ((int64_t)phys * hkv + kvh) * TILE_PIECES + lane;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      kr[j] = kc[base + j * 64];
      vr[j] = vc[base + j * 64];
    }
    return true;
  };

  auto consume = [&](int b, const uint4* kr, const uint4* vr, bool ok) {
    const int t_base = tok0 + b * kBlockSize;
    const bool tail = !ok || (t_base + kBlockSize > tok1);
    float s[NLD][G];
#pragma unroll
    for (int j = 0; j < NLD; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) s[j][h] = group_sum<LPT>(dot_piece(qv[h], kr[j], IsBF16{})) * sl2;
    uint4 vv[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) vv[j] = vr[j];
    if (tail) {
      // select, never multiply: stale slots may hold NaN
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const bool valid = ok && (t_base + row + j * TPL < tok1);
        if (!valid) {
          vv[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
          for (int h = 0; h < G; ++h) s[j][h] = kNegInf;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mb = s[0][h];
#pragma unroll
      for (int j = 1; j < NLD; ++j) mb = fmaxf(mb, s[j][h]);
      const float mn = fmaxf(m[h], mb);
      const float mref = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - mref);
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const float p = fast_exp2(s[j][h] - mref);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, piece_elem<BF16>(vv[j], e), acc[h][e]);
      }
      m[h] = mn;
    }
  };

  // blocks wave, wave+4, ...; the next block is in flight while one is consumed
  {
    uint4 kb[NLD], vb[NLD];
    int b = wave;
    bool ok = false;
    if (b < nblk) ok = load(b, kb, vb);
    for (; b < nblk; b += kDecodeWaves) {
      uint4 kn[NLD], vn[NLD];
      bool okn = false;
      const int bn = b + kDecodeWaves;
      if (bn < nblk) okn = load(bn, kn, vn);
      consume(b, kb, vb, ok);
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        kb[j] = kn[j];
        vb[j] = vn[j];
      }
      ok = okn;
    }
  }

  // merge the lane groups of this wave (token rows) pairwise
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float mref = (mn == kNegInf) ? 0.f : mn;
      const float wa = fast_exp2(m[h] - mref);
      const float wb = fast_exp2(mo - mref);
      l[h] = l[h] * wa + lo * wb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * wa + __shfl_xor(acc[h][e], off) * wb;
      m[h] = mn;
    }
  }

  // merge the waves in LDS
  __shared__ float sm_ml[kDecodeWaves][G][2];
  __shared__ float sm_acc[kDecodeWaves][G][D];
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][h][col * EPL + e] = acc[h][e];
      if (col == 0) {
        sm_ml[wave][h][0] = m[h];
        sm_ml[wave][h][1] = l[h];
      }
    }
  }
  __syncthreads();

  const int64_t part_base = (int64_t)seq * hq + kvh * G;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int d = idx - h * D;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) mx = fmaxf(mx, sm_ml[w][h][0]);
    const float mref = (mx == kNegInf) ? 0.f : mx;
    float lsum = 0.f, asum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float wt = fast_exp2(sm_ml[w][h][0] - mref);
      lsum += wt * sm_ml[w][h][1];
      asum += wt * sm_acc[w][h][d];
    }
    if (nparts == 1) {
      const float o = lsum > 0.f ? asum / lsum : 0.f;
      store_elem<BF16>(a.out, ((int64_t)qrow * hq + kvh * G + h) * D + d, o);
    } else {
      const int64_t pidx = (part_base + h) * a.max_parts + part;
      float* ws_ml = a.ws;
      float* ws_acc = a.ws + (int64_t)a.num_seqs * hq * a.max_parts * 2;
      ws_acc[pidx * D + d] = asum;
      if (d == 0) {
        ws_ml[pidx * 2 + 0] = mx;
        ws_ml[pidx * 2 + 1] = lsum;
      }
    }
  }
}

// Merge the partitions of one (sequence, q head): weights 2^(m_p - max m) in
// ascending partition order.
template <bool BF16, int D, bool VARLEN>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeArgs a) {
  constexpr float kNegInf = -INFINITY;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  int qrow, ctx;
  if (!decode_row<VARLEN>(a, seq, qrow, ctx)) return;
  const int nparts = max(1, ceil_div(ctx, kPartitionTokens));
  if (nparts <= 1) return;
  const int hq = a.num_q_heads;
  const int d = threadIdx.x;
  const int64_t pbase = ((int64_t)seq * hq + h) * a.max_parts;
  const float* ws_ml = a.ws + pbase * 2;
  const float* ws_acc = a.ws + (int64_t)a.num_seqs * hq * a.max_parts * 2 + pbase * D;
  float mx = kNegInf;
  for (int p = 0; p < nparts; ++p) mx = fmaxf(mx, ws_ml[2 * p]);
  const float mref = (mx == kNegInf) ? 0.f : mx;
  float lsum = 0.f, asum = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float wt = fast_exp2(ws_ml[2 * p] - mref);
    lsum += wt * ws_ml[2 * p + 1];
    asum += wt * ws_acc[p * D + d];
  }
  const float o = lsum > 0.f ? asum / lsum : 0.f;
  store_elem<BF16>(a.out, ((int64_t)qrow * hq + h) * D + d, o);
}

template <bool BF16, int D, int G, bool VARLEN>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<BF16, D, G, VARLEN>), grid, dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.max_parts <= 1) return err;
  hipLaunchKernelGGL((decode_reduce_kernel<BF16, D, VARLEN>), dim3(a.num_q_heads, a.num_seqs),
                     dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16, int D, int G>
static hipError_t launch_mode(const DecodeArgs& a, hipStream_t s) {
  return a.varlen ? launch_decode_t<BF16, D, G, true>(a, s) : launch_decode_t<BF16, D, G, false>(a, s);
}

template <bool BF16, int D>
static hipError_t launch_group(const DecodeArgs& a, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_mode<BF16, D, 1>(a, s);
    case 2: return launch_mode<BF16, D, 2>(a, s);
    case 4: return launch_mode<BF16, D, 4>(a, s);
    case 8: return launch_mode<BF16, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
static hipError_t launch_dim(const DecodeArgs& a, hipStream_t s) {
  switch (a.head_dim) {
    case 64: return launch_group<BF16, 64>(a, s);
    case 128: return launch_group<BF16, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  return a.dtype == PA_BF16 ? launch_dim<true>(a, stream) : launch_dim<false>(a, stream);
}

}  // namespace pa
