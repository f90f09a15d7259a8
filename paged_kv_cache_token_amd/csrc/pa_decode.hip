// pa_decode.hip -- paged decode attention: split-K over fixed partitions of the
// context, online softmax, and a cross-partition merge.
//
// "vLLM：颠覆大模型推理的高效API服务引擎深度解析", §1.3 (attention reads the
// blocks scattered over the pool through the block table) and §2.2 (one fused
// kernel reads the KV cache straight from the physical blocks);
// "vLLM изнутри: как устроен движок для быстрого инференса LLM", the paragraph on
// the stages of a step (decode reads every cached K/V for one query token and
// is bound by memory bandwidth).  Splitting the softmax over pieces of the
// context and merging them with a rescale is the chunked-attention idea of the
// flash-attention paragraph in "vLLMつかったら、ベクトル検索サーバーが高速化して
// 安定性も向上した".
//
// Work decomposition (gfx950, wave64):
//   * a work item is one (sequence, partition of the context) for one kv head;
//     a workgroup of 1, 2 or 4 waves serves all g query heads of that kv head,
//     so each K/V tile is read from HBM once per step;
//   * the waves take the partition's 16-token blocks round-robin.  A wave
//     reads its block-table entries once (one entry per lane, issued together
//     with the context length and the query) and broadcasts them with
//     readlane, so the only vector loads in its loop are K and V;
//   * a (block, kv head) tile is 16 * head_dim contiguous elements, so one
//     wave-wide 16-byte-per-lane load reads 1 KB of consecutive memory; the
//     single-partition and work-list kernels read the tiles as streaming
//     (non-temporal) data;
//   * bf16 at head_dim 128 runs the matrix-core item code (decode_item_mfma):
//     the tiles go HBM -> LDS and the block's score and value products are
//     two matrix products with the g query heads as columns; the next block's
//     loads are issued as soon as the current block's operands are read;
//   * fp32 and head_dim 64 run the vector item code (decode_item): lane l
//     holds the 16-byte piece (l % LPT) of token row (l / LPT) + k * (64 / LPT)
//     in registers (the next block's K and V in flight while the current one
//     is computed); q.k partial sums over a lane's piece are finished with DPP
//     all-reduces inside the LPT-lane group that holds one token row; each
//     lane group keeps its own running (max, sum, accumulator) over the token
//     rows it holds, merged at the end of the item across the wave with lane
//     exchanges;
//   * the waves of an item are merged in LDS;
//   * an item whose sequence has one partition writes `out` directly.  Otherwise
//     it stores (max, sum, accumulator) in the workspace, and a merge kernel
//     combines the sequence's partitions in ascending order and writes `out`
//     (a separate launch: the kernel boundary publishes the partials to every
//     XCD, which inside one kernel would take an L2 write-back per item);
//   * when every context fits one partition the grid is (sequence, kv head),
//     kv head fastest; otherwise a persistent grid sized to the chip walks the
//     (sequence, partition) list, full partitions first, which each workgroup
//     derives from the lengths at its start (a one-workgroup plan kernel
//     writes it instead past 2048 sequences);
//   * a cascade decode's common prefix arrives as partials written by the
//     matrix-core pass: the partitions start after it (key_start) and their
//     slots follow its slots (prefix_parts), so the merge combines all; when
//     every private rest fits one partition, the (sequence, kv head) grid
//     writes its one partial per pair and the merge follows it.
// The order of every sum depends only on logical token positions, never on the
// physical block ids, so the output is
// bit-identical under any placement or sharing of blocks and between runs.

#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>

#include "../../include/pa.h"
#include "pa_launch.h"

namespace pa {

__device__ __forceinline__ float dot_piece(uint4 q, uint4 k, std::true_type /*bf16*/) {
  // the first product with a literal zero accumulator (the compiler would
  // otherwise clear a register for the accumulating form)
  float s;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(q.x), "v"(k.x));
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

// An empty asm that reads x: the compiler must have x loaded here.  Used once
// before a loop so that loads issued ahead of it are not waited for inside it
// (the wait counter is in-order: a wait for an old load inside the loop would
// also wait for the prefetch issued in the same iteration).
__device__ __forceinline__ void loaded(uint32_t x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void loaded(const uint4& x) {
  loaded(x.x);
  loaded(x.y);
  loaded(x.z);
  loaded(x.w);
}

// element e of a 16-byte piece as fp32 (e is a compile-time index after unrolling)
template <bool BF16>
__device__ __forceinline__ float piece_elem(const uint4& v, int e) {
  const uint32_t w = e < (BF16 ? 2 : 1) ? v.x : e < (BF16 ? 4 : 2) ? v.y : e < (BF16 ? 6 : 3) ? v.z : v.w;
  if constexpr (BF16) {
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  } else {
    return __uint_as_float(w);
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

// ---------------------------------------------------------------------------
// DPP row (16-lane) helpers for the one-score-per-lane softmax
// ---------------------------------------------------------------------------

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// one halving step of a reduce-scatter across lane pairs that differ in BIT
template <int CTRL, int BIT, int L, int NS>
__device__ __forceinline__ void rs_step(float (&x)[NS], int c) {
  if constexpr (L >= 2) {
    constexpr int H = L / 2;
    const bool hi = (c & BIT) != 0;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float send = hi ? x[i] : x[i + H];
      const float keep = hi ? x[i + H] : x[i];
      x[i] = keep + dpp_f32<CTRL>(send);
    }
  } else {
    x[0] += dpp_f32<CTRL>(x[0]);
  }
}

// Reduce-scatter inside each 16-lane DPP row.  On entry x[0..NS) are a lane's
// partial sums; on exit x[0..V), V = max(1, NS/16), are complete sums, and lane
// c of the row holds index c*V + u (NS >= 16) or c / (16/NS) (NS < 16, each
// index then held by 16/NS lanes).  Partners: row mirror (c <-> 15-c) splits
// on bit 3, half-row mirror on bit 2, quad swaps on bits 1 and 0.
template <int NS>
__device__ __forceinline__ void row_reduce_scatter(float (&x)[NS], int c) {
  rs_step<0x140, 8, NS, NS>(x, c);
  rs_step<0x141, 4, (NS / 2 > 1 ? NS / 2 : 1), NS>(x, c);
  rs_step<0x4E, 2, (NS / 4 > 1 ? NS / 4 : 1), NS>(x, c);
  rs_step<0xB1, 1, (NS / 8 > 1 ? NS / 8 : 1), NS>(x, c);
}

// value of lane LANE of the caller's 16-lane row (every lane has a source,
// so the destination's old value is never kept and needs no clearing)
template <int LANE>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + LANE, 0xF, 0xF, false));
}

// max / sum over the 4 lanes {c, c+4, c+8, c+12} (mod 16) of a row
__device__ __forceinline__ float row_max4(float x) {
  x = fmaxf(x, dpp_f32<0x124>(x));  // row_ror:4
  return fmaxf(x, dpp_f32<0x128>(x));  // row_ror:8
}
__device__ __forceinline__ float row_sum4(float x) {
  x += dpp_f32<0x124>(x);
  return x + dpp_f32<0x128>(x);
}

// The row of q/out and the attended length of a sequence.  Returns false when
// the sequence is not served by the decode kernels (a multi-token chunk of a
// packed batch).
template <bool VARLEN>
__device__ __forceinline__ bool decode_row(const DecodeArgs& a, int seq, int& qrow, int& ctx) {
  if constexpr (VARLEN) {
    if (a.table_rows) {
      // every packed row on its own: item `seq` is query row `seq`, with its
      // own context (its table row comes through table_rows)
      if (seq >= a.q_rows) return false;
      qrow = seq;
      ctx = a.context_lens[seq];
    } else {
      const int lo = a.cu_seqlens[seq];
      if (a.cu_seqlens[seq + 1] - lo != 1) return false;
      if (lo < 0 || lo >= a.q_rows) return false;  // outside q / out: skipped
      qrow = lo;
      ctx = a.context_offsets[seq] + 1;
    }
  } else {
    qrow = seq;
    ctx = a.context_lens[seq];
  }
  ctx = max(0, min(ctx, min(a.max_context_len, a.max_blocks_per_seq * kBlockSize)));
  return true;
}

// partitions of `keys` keys (one, possibly empty, when keys <= 0)
__device__ __forceinline__ int parts_of(int keys, int part_tokens) {
  return max(1, ceil_div(keys, part_tokens));
}

template <int G, int D>
struct DecodeShared {
  float ml[kDecodeMaxWaves][G][2];
  float acc[kDecodeMaxWaves][G][D];
};

// The item's waves have written their (max, sum, accumulator) per head to
// sm: combine them and write the output row, or the partition's partial.
template <bool BF16, int D, int G>
__device__ __forceinline__ void finish_item(const DecodeArgs& a, const DecodeShared<G, D>& sm,
                                            int seq, int qrow, int kvh, int part, int nparts) {
  constexpr float kNegInf = -INFINITY;
  __syncthreads();
  const int hq = a.num_q_heads;
  const int nwaves = a.waves;
  const int64_t row_base = (int64_t)seq * hq + kvh * G;  // (seq, first q head) partial row
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int d = idx - h * D;
    float mx = kNegInf;
    for (int w = 0; w < nwaves; ++w) mx = fmaxf(mx, sm.ml[w][h][0]);
    const float mref = (mx == kNegInf) ? 0.f : mx;
    float lsum = 0.f, asum = 0.f;
    for (int w = 0; w < nwaves; ++w) {
      const float wt = fast_exp2(sm.ml[w][h][0] - mref);
      lsum += wt * sm.ml[w][h][1];
      asum += wt * sm.acc[w][h][d];
    }
    if (nparts == 1 && a.prefix_parts == 0) {
      store_elem<BF16>(a.out, ((int64_t)qrow * hq + kvh * G + h) * D + d,
                       lsum > 0.f ? asum / lsum : 0.f);
    } else {
      const int64_t pidx = (row_base + h) * a.max_parts + a.prefix_parts + part;
      a.ws.acc[pidx * D + d] = asum;
      if (d == 0) {
        a.ws.ml[pidx * 2 + 0] = mx;
        a.ws.ml[pidx * 2 + 1] = lsum;
      }
    }
  }
}

// One work item: partition `part` of sequence `seq`, kv head `kvh`.  NB
// register buffers per wave: NB - 1 blocks stay in flight while one is
// consumed.  STREAM: the K/V tiles are read as streaming data (see load()).
template <bool BF16, int D, int G, bool VARLEN, int NB, bool STREAM = false>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int seq, int part, int kvh,
                                            DecodeShared<G, D>& sm) {
  using IsBF16 = std::integral_constant<bool, BF16>;
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int EPL = 16 / EB;              // elements in a lane's 16-byte piece
  constexpr int LPT = D / EPL;              // lanes holding one token row
  constexpr int TPL = 64 / LPT;             // token rows per wave-wide load
  constexpr int NLD = kBlockSize / TPL;     // wave-wide loads per 16-token tile
  constexpr int TILE_PIECES = kBlockSize * LPT;
  constexpr int NS = NLD * G;               // scores per lane per tile
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "piece layout");
  constexpr float kNegInf = -INFINITY;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = a.waves;
  const int row = lane / LPT;
  const int col = lane % LPT;
  const int hq = a.num_q_heads;
  const int hkv = a.num_kv_heads;
  const int pt = a.part_tokens;
  const int tok0 = a.key_start + part * pt;

  // Three independent loads go out together: the context length (scalar), this
  // wave's table entries (lane i: the wave's i-th block of the partition; the
  // index is clamped into the table row, so entries past the context are
  // in-bounds garbage that is never used) and the query pieces.
  // (rows of a packed call taken one by one name their sequence's table row)
  int tseq = seq;
  if constexpr (VARLEN) {
    if (a.table_rows) tseq = a.table_rows[seq];
  }
  const int32_t* table = a.block_tables + (int64_t)tseq * a.max_blocks_per_seq + tok0 / kBlockSize;
  const int row_left = a.max_blocks_per_seq - tok0 / kBlockSize;  // >= 1 for a live item
  const int my_entry = table[min(wave + nwaves * lane, row_left - 1)];
  int qrow, ctx;
  if (!decode_row<VARLEN>(a, seq, qrow, ctx)) return;
  const int nparts = parts_of(ctx - a.key_start, pt);
  if (part >= nparts) return;
  uint4 qv[G];
  // the new token's K/V (fused step) travel with the query pieces
  uint4 knew = make_uint4(0u, 0u, 0u, 0u), vnew = knew;
  if (a.key_new != nullptr) {
    const int64_t src = ((int64_t)seq * hkv + kvh) * LPT + col;
    knew = static_cast<const uint4*>(a.key_new)[src];
    vnew = static_cast<const uint4*>(a.value_new)[src];
  }
  {
    const uint4* qb = static_cast<const uint4*>(a.q) + ((int64_t)qrow * hq + kvh * G) * LPT + col;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = qb[h * LPT];
#pragma unroll
    for (int h = 0; h < G; ++h) loaded(qv[h]);
    loaded((uint32_t)my_entry);
    loaded(knew);
    loaded(vnew);
  }

  const int tok1 = min(ctx, tok0 + pt);
  const int nblk = tok1 > tok0 ? ceil_div(tok1 - tok0, kBlockSize) : 0;
  const int nmine = nblk > wave ? ceil_div(nblk - wave, nwaves) : 0;  // <= 64

  // Fused step: the new token sits at position context_lens[seq] - 1, taken
  // before any clamp (as the separate slot-mapping call takes it).  The item
  // whose keys hold that position uses the new K/V from the inputs instead of
  // re-reading the cache (no read-after-write within the launch) and stores
  // them into their slot once its loads are issued.  When the declared maxima
  // clamp the context below the position, no item attends it, and the item of
  // the last partition stores it (its slot still comes from the table, as
  // with the separate calls; past the table's end nothing is stored).
  const int new_pos = a.key_new != nullptr ? a.context_lens[seq] - 1 : -1;
  const bool fused = new_pos >= 0 && new_pos < ctx && new_pos >= tok0 && new_pos < tok1;
  const bool store = fused || (new_pos >= ctx && part == nparts - 1);
  const int new_off = new_pos % kBlockSize;                        // row inside its block
  const int new_blk = fused ? (new_pos - tok0) / kBlockSize : -1;  // partition-local block

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

  // Loads of the K and V tiles of this wave's i-th block.  The loop's loads
  // are unconditional, so its waits count only the block it consumes: past
  // the wave's last block (i >= nmine) a load repeats that block.
  //   * plain loads: the repeat hits in L2, and an unusable block id reads
  //     block 0's tile, which consume() masks;
  //   * STREAM: buffer loads with the non-temporal hint, so the stream of
  //     tiles read once does not displace what the caches hold; a repeat or
  //     an unusable block gets a zero-length buffer, which reads as zeros
  //     without touching memory (a repeated streaming load would miss L2).
  auto load = [&](int i, uint4 (&kr)[NLD], uint4 (&vr)[NLD]) -> int {
    const int raw = __builtin_amdgcn_readlane(my_entry, min(i, nmine - 1));
    const int phys = (raw >= 0 && (int64_t)raw < a.num_blocks) ? raw : -1;
    const int64_t tile = ((int64_t)max(phys, 0) * hkv + kvh) * TILE_PIECES;
    if constexpr (STREAM) {
      const int bytes = (i < nmine && phys >= 0) ? TILE_PIECES * 16 : 0;  // wave-uniform
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint4*>(kc + tile), (short)0, bytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint4*>(vc + tile), (short)0, bytes, 0x00020000);
      constexpr int kNonTemporal = 2;  // cache-policy bit nt
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        kr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rk, (lane + j * 64) * 16, 0, kNonTemporal));
        vr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rv, (lane + j * 64) * 16, 0, kNonTemporal));
      }
    } else {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        kr[j] = kc[tile + lane + j * 64];
        vr[j] = vc[tile + lane + j * 64];
      }
    }
    return phys;
  };

  // ---- one-score-per-lane softmax (16-lane rows: bf16 d=128, fp32 d=64) ----
  // After the reduce-scatter, lane c of row r holds the score(s) of index
  // k = j*G + h with j = c/4 (token r + 4j of the block) and head h; the
  // running max and sum are kept per (row, head) value, the p values are
  // broadcast back to the row for the PV products, and the accumulator is
  // rescaled only when some running max moved.
  constexpr bool kScatter = (LPT == 16);
  constexpr int V = NS >= 16 ? NS / 16 : 1;   // values per lane
  constexpr int R = NS >= 16 ? 1 : 16 / NS;   // lanes per value
  float mu[V], lu[V];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    mu[u] = kNegInf;
    lu[u] = 0.f;
  }

  auto consume = [&](int i, int phys, const uint4 (&kr)[NLD], const uint4 (&vr)[NLD]) {
    const int t_base = tok0 + (wave + nwaves * i) * kBlockSize;
    const bool tail = phys < 0 || t_base + kBlockSize > tok1;
    float s[NS];
#pragma unroll
    for (int j = 0; j < NLD; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) s[j * G + h] = dot_piece(qv[h], kr[j], IsBF16{});
    uint4 vv[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) vv[j] = vr[j];
    if (fused && wave + nwaves * i == new_blk) {
      // the new token's row comes from the inputs, not the cache
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        if (row + j * TPL == new_off) {
          vv[j] = vnew;
#pragma unroll
          for (int h = 0; h < G; ++h) s[j * G + h] = dot_piece(qv[h], knew, IsBF16{});
        }
    }
    if (tail) {
      // select, never multiply: stale slots may hold NaN
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        if (!(phys >= 0 && (t_base + row + j * TPL < tok1))) vv[j] = make_uint4(0u, 0u, 0u, 0u);
    }
    if constexpr (kScatter) {
      row_reduce_scatter<NS>(s, col);
      const int jl = col >> 2;  // this lane's token group
      const bool valid = !tail || (phys >= 0 && (t_base + row + jl * TPL < tok1));
      float su[V], mn[V];
      bool moved = false;
#pragma unroll
      for (int u = 0; u < V; ++u) {
        su[u] = valid ? s[u] * sl2 : kNegInf;
        mn[u] = fmaxf(mu[u], row_max4(su[u]));
        moved |= (mn[u] != mu[u]);
      }
      if (__any(moved)) {
        float al[V];
#pragma unroll
        for (int u = 0; u < V; ++u) {
          const float mref = (mn[u] == kNegInf) ? 0.f : mn[u];
          al[u] = fast_exp2(mu[u] - mref);
          lu[u] *= al[u];
          mu[u] = mn[u];
        }
        static_for<0, G>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          const float ah = row_bcast<(NS >= 16 ? h / V : h * R)>(al[NS >= 16 ? h % V : 0]);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= ah;
        });
      }
      float pu[V];
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const float mref = (mu[u] == kNegInf) ? 0.f : mu[u];
        pu[u] = fast_exp2(su[u] - mref);
        // bf16 values: the weights enter the V products in bf16 (below), so
        // the sum takes them rounded the same way
        if constexpr (BF16) pu[u] = round_to_bf16(pu[u]);
        lu[u] += pu[u];
      }
      float p[NS];
      static_for<0, NS>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        p[k] = row_bcast<(NS >= 16 ? k / V : k * R)>(pu[NS >= 16 ? k % V : 0]);
      });
      if constexpr (BF16) {
        // O += p V two token rows at a time: the bf16 weights of rows 2jp and
        // 2jp+1 (exact: rounded above) against the pair (v[2jp][e],
        // v[2jp+1][e]) gathered by a byte permute, one v_dot2_f32_bf16 per
        // (head, element) instead of two fp32 FMAs and the widening of v
        static_assert(NLD % 2 == 0, "token rows are paired");
#pragma unroll
        for (int jp = 0; jp < NLD / 2; ++jp) {
          bf16x2_t pp[G];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const f32x2_t f = {p[(2 * jp) * G + h], p[(2 * jp + 1) * G + h]};
            pp[h] = __builtin_convertvector(f, bf16x2_t);
          }
          const uint32_t w0[4] = {vv[2 * jp].x, vv[2 * jp].y, vv[2 * jp].z, vv[2 * jp].w};
          const uint32_t w1[4] = {vv[2 * jp + 1].x, vv[2 * jp + 1].y, vv[2 * jp + 1].z,
                                  vv[2 * jp + 1].w};
#pragma unroll
          for (int w = 0; w < EPL / 2; ++w) {
            // (row 2jp, row 2jp+1) of element 2w, and of element 2w+1
            const bf16x2_t lo = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(w1[w], w0[w], 0x05040100u));
            const bf16x2_t hi = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(w1[w], w0[w], 0x07060302u));
#pragma unroll
            for (int h = 0; h < G; ++h) {
              acc[h][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], lo, acc[h][2 * w], false);
              acc[h][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], hi, acc[h][2 * w + 1], false);
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NLD; ++j)
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            const float v = piece_elem<BF16>(vv[j], e);
#pragma unroll
            for (int h = 0; h < G; ++h) acc[h][e] = fmaf(p[j * G + h], v, acc[h][e]);
          }
      }
    } else {
      group_sum_n<LPT, NS>(s);
#pragma unroll
      for (int k = 0; k < NS; ++k) s[k] *= sl2;
      if (tail) {
#pragma unroll
        for (int j = 0; j < NLD; ++j)
          if (!(phys >= 0 && (t_base + row + j * TPL < tok1)))
#pragma unroll
            for (int h = 0; h < G; ++h) s[j * G + h] = kNegInf;
      }
      float p[NS];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mb = s[h];
#pragma unroll
        for (int j = 1; j < NLD; ++j) mb = fmaxf(mb, s[j * G + h]);
        const float mn = fmaxf(m[h], mb);
        const float mref = (mn == kNegInf) ? 0.f : mn;
        const float alpha = fast_exp2(m[h] - mref);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
          p[j * G + h] = fast_exp2(s[j * G + h] - mref);
          l[h] += p[j * G + h];
        }
        m[h] = mn;
      }
#pragma unroll
      for (int j = 0; j < NLD; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float v = piece_elem<BF16>(vv[j], e);
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h][e] = fmaf(p[j * G + h], v, acc[h][e]);
        }
    }
  };

  if (nmine > 0) {
    // a ring of NB register buffers, all filled before the first wait; the
    // block consumed from buffer b is replaced by the one NB blocks later
    uint4 kb[NB][NLD], vb[NB][NLD];
    int id[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) id[b] = load(b, kb[b], vb[b]);
    for (int i = 0; i < nmine; i += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b == 0 || i + b < nmine) consume(i + b, id[b], kb[b], vb[b]);
        id[b] = load(i + b + NB, kb[b], vb[b]);
      }
    }
  }

  if (store && wave == 0 && lane < LPT && new_pos / kBlockSize < a.max_blocks_per_seq) {
    const int raw = a.block_tables[(int64_t)tseq * a.max_blocks_per_seq + new_pos / kBlockSize];
    if (raw >= 0 && (int64_t)raw < a.num_blocks) {
      const int64_t dst = (((int64_t)raw * hkv + kvh) * kBlockSize + new_off) * LPT + lane;
      static_cast<uint4*>(a.k_cache_w)[dst] = knew;
      static_cast<uint4*>(a.v_cache_w)[dst] = vnew;
    }
  }

  if constexpr (kScatter) {
    // back to per-head running (max, sum) on every lane of the row
    float ls[V];
#pragma unroll
    for (int u = 0; u < V; ++u) ls[u] = row_sum4(lu[u]);
    static_for<0, G>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      constexpr int src = NS >= 16 ? h / V : h * R;
      m[h] = row_bcast<src>(mu[NS >= 16 ? h % V : 0]);
      l[h] = row_bcast<src>(ls[NS >= 16 ? h % V : 0]);
    });
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

  // merge the waves in LDS (the barrier first protects LDS from the previous item)
  __syncthreads();
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm.acc[wave][h][col * EPL + e] = acc[h][e];
      if (col == 0) {
        sm.ml[wave][h][0] = m[h];
        sm.ml[wave][h][1] = l[h];
      }
    }
  }
  finish_item<BF16, D, G>(a, sm, seq, qrow, kvh, part, nparts);
}

// ---------------------------------------------------------------------------
// Matrix-core item: bf16 at head_dim 128 (any g up to 16 query heads per kv head).
// ---------------------------------------------------------------------------
// The waves take the partition's blocks as above; the g query heads are the
// columns (zero queries past g) of two matrix products per 16-token block:
//   * S = K Q^T with four v_mfma_f32_16x16x32_bf16 (one per 32 dims).  A is
//     the block's 16 key rows, loaded from HBM straight into the operand
//     layout: lane l holds key row l % 16, and for product ks the 16-byte
//     piece 4 ks + l / 16 of that row; B holds the same pieces of query head
//     l % 16.  (The pairing of operand elements to dims is the same on both
//     sides, so the sum over dims is exact whatever the hardware's order.)
//     Lane l ends with the scores of tokens 4 (l / 16) + r, r = 0..3, for
//     head l % 16;
//   * O^T += V^T P^T with eight v_mfma_f32_16x16x16_bf16 (one per 16 dims).
//     B = P^T is that score accumulator itself, turned into bf16
//     exponentials in place; A = V^T comes from the transposing LDS read of
//     the block's V tile, which the wave's buffer loads put straight into
//     LDS (no register staging).  Lane l accumulates dims 16 m + 4 (l / 16) + r
//     of head l % 16.
// The softmax keeps one head per lane column: the block maximum per head takes
// two cross-row swaps, and the exponentials' reference is raised only when
// some head's block maximum lies more than 2^8 above it (so p < 256: exact in
// fp32, bf16's relative precision in the products), all heads rescaled then.
constexpr float kMfmaLazy = 8.f;  // log2 units

// LDS tiles of one block, [token][16-byte chunk] as the HBM->LDS loads
// write them (1 KiB of four consecutive token rows per wave instruction),
// with the chunk position XOR-swizzled by the token so the operand reads hit
// distinct banks: in K, chunk x of token t sits at x ^ t (the 16-byte reads
// of 16 tokens at one chunk); in V at x ^ 2 (t & 7) (the transposing 8-byte
// reads of 8 tokens at two adjacent chunks, per 32 lanes).
__device__ __forceinline__ int ktile_pos(int t, int x) { return t * 16 + (x ^ t); }
__device__ __forceinline__ int vtile_pos(int t, int x) { return t * 16 + (x ^ (2 * (t & 7))); }
constexpr int kWaveTileChunks = 592;  // per wave: K tile, V tile, the staged new row (80)

template <int G, bool VARLEN, bool STREAM>
__device__ __forceinline__ void decode_item_mfma(const DecodeArgs& a, int seq, int part, int kvh,
                                                 DecodeShared<G, 128>& sm, uint4* tiles) {
  constexpr int D = 128;
  constexpr int kRow = D * 2;                  // bytes of one token row of a tile
  constexpr int kTile = kBlockSize * kRow;     // bytes of one (block, kv head) tile
  constexpr int kAux = STREAM ? 2 : 0;         // cache policy of the tile loads (2: nt)
  constexpr float kNegInf = -INFINITY;
  static_assert(G >= 1 && G <= 16, "query heads per kv head");

  // (opaque to the compiler, so the lane's tile addresses are derived per
  // item instead of being held in registers across a persistent kernel's items)
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = a.waves;
  const int col = lane & 15;  // key row of K; head column of S, P and O
  const int grp = lane >> 4;  // piece group of K and Q; tokens 4 grp .. 4 grp + 3 of S
  const int hq = a.num_q_heads;
  const int hkv = a.num_kv_heads;
  const int pt = a.part_tokens;
  const int tok0 = a.key_start + part * pt;

  int tseq = seq;
  if constexpr (VARLEN) {
    if (a.table_rows) tseq = a.table_rows[seq];
  }
  const int32_t* table = a.block_tables + (int64_t)tseq * a.max_blocks_per_seq + tok0 / kBlockSize;
  const int row_left = a.max_blocks_per_seq - tok0 / kBlockSize;  // >= 1 for a live item
  const int my_entry = table[min(wave + nwaves * lane, row_left - 1)];
  int qrow, ctx;
  if (!decode_row<VARLEN>(a, seq, qrow, ctx)) return;
  const int nparts = parts_of(ctx - a.key_start, pt);
  if (part >= nparts) return;

  // the query pieces of head `col` (zero past g)
  uint4 qf[4];
  {
    const uint4* qb = static_cast<const uint4*>(a.q) +
                      ((int64_t)qrow * hq + kvh * G + min(col, G - 1)) * (D / 8) + grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = qb[4 * ks];
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) loaded(qf[ks]);
  loaded((uint32_t)my_entry);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    if (col >= G) qf[ks] = make_uint4(0u, 0u, 0u, 0u);

  const int tok1 = min(ctx, tok0 + pt);
  const int nblk = tok1 > tok0 ? ceil_div(tok1 - tok0, kBlockSize) : 0;
  const int nmine = nblk > wave ? ceil_div(nblk - wave, nwaves) : 0;  // <= 64

  // fused step: as in decode_item
  const int new_pos = a.key_new != nullptr ? a.context_lens[seq] - 1 : -1;
  const bool fused = new_pos >= 0 && new_pos < ctx && new_pos >= tok0 && new_pos < tok1;
  const bool store = fused || (new_pos >= ctx && part == nparts - 1);
  const int new_off = new_pos % kBlockSize;
  const int new_blk = fused ? (new_pos - tok0) / kBlockSize : -1;
  // The wave that consumes or stores the new token's row stages it in LDS
  // behind its tiles, straight from memory: V's 16 chunks at stage[0..16),
  // K's at stage[16..32) (each load writes 64 chunks, the lanes past the row
  // zeros; K's lands second).  These are the wave's oldest loads, so the
  // tile waits cover them.
  uint4* ktile = tiles;
  uint4* vtile = tiles + 256;
  uint4* stage = tiles + 512;
  const bool stager = (fused && new_blk % nwaves == wave) || (store && wave == 0);
  if (stager) {
    const int64_t row = ((int64_t)seq * hkv + kvh) * kRow;
    dma16(static_cast<const char*>(a.value_new) + row, kRow, lane * 16, stage);
    dma16(static_cast<const char*>(a.key_new) + row, kRow, lane * 16, stage + 16);
  }

  f32x4_t o[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref = kNegInf, lsum = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;  // scores in log2 units
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);

  // The wave's i-th block: its physical id (-1: unusable) and the bytes of
  // its tile that hold keys of the partition (0 past the wave's last block).
  auto block_of = [&](int i, int& phys, int64_t& tile, int& bytes) {
    const int raw = __builtin_amdgcn_readlane(my_entry, min(i, nmine - 1));
    phys = (raw >= 0 && (int64_t)raw < a.num_blocks) ? raw : -1;
    const int t_base = tok0 + (wave + nwaves * i) * kBlockSize;
    bytes = (i < nmine && phys >= 0) ? min(kBlockSize, tok1 - t_base) * kRow : 0;
    tile = ((int64_t)max(phys, 0) * hkv + kvh) * kTile;
  };
  // K and V tiles straight into LDS: load j brings token rows 4 j .. 4 j + 3,
  // lane (grp, col) the chunk landing at position col of row 4 j + grp.
  // Loads past the valid bytes write zeros without touching memory.
  auto load_tiles = [&](int64_t tile, int bytes) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * j + grp;
      dma16<kAux>(kc + tile, bytes, t * kRow + (col ^ t) * 16, ktile + 64 * j);
      dma16<kAux>(vc + tile, bytes, t * kRow + (col ^ (2 * (t & 7))) * 16, vtile + 64 * j);
    }
  };
  // the transposing reads: lane (grp, col = 4 r + q) addresses token
  // 4 grp + r at dims 16 m + 4 q .. 16 m + 4 q + 3
  const int tr_t = 4 * grp + (col >> 2);
  const int tr_q = col & 3;

  // One block per step; the next block's loads go out as soon as this
  // block's operands have been read from its LDS tiles, so the products and
  // the softmax overlap the next block's memory latency.
  if (nmine > 0) {
    int phys, bytes;
    int64_t tile;
    block_of(0, phys, tile, bytes);
    load_tiles(tile, bytes);
    for (int i = 0; i < nmine; ++i) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // block i (and the staged row) landed
      const int t_base = tok0 + (wave + nwaves * i) * kBlockSize;
      const int nvalid = phys >= 0 ? min(kBlockSize, tok1 - t_base) : 0;  // wave-uniform
      if (fused && wave + nwaves * i == new_blk && lane < 16) {
        // the new token's row comes from the inputs, not the cache: over the
        // landed tiles' row new_off (the wave's LDS accesses run in order)
        ktile[ktile_pos(new_off, lane)] = stage[16 + lane];
        vtile[vtile_pos(new_off, lane)] = stage[lane];
      }
      uint4 kf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[ks] = ktile[ktile_pos(col, 4 * ks + grp)];
      const char* vb = reinterpret_cast<const char*>(vtile);
      uint2 vf[8];
#pragma unroll
      for (int m = 0; m < 8; ++m)
        vf[m] = lds_read_tr(reinterpret_cast<const uint16_t*>(
            vb + vtile_pos(tr_t, 2 * m + (tr_q >> 1)) * 16 + (tr_q & 1) * 8));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tiles are free again
      block_of(i + 1, phys, tile, bytes);
      load_tiles(tile, bytes);
      if (nvalid <= 0) continue;  // an empty block: all its keys drop out

      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[ks]),
                                                     __builtin_bit_cast(bf16x8_t, qf[ks]), sc, 0, 0, 0);
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = (4 * grp + r < nvalid) ? sc[r] * sl2 : kNegInf;
      float bm = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
      {
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm),
                                                        false, false);
        bm = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
        const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm),
                                                        false, false);
        bm = fmaxf(__uint_as_float(z[0]), __uint_as_float(z[1]));
      }
      // a block with a valid key has a finite maximum in every column, so the
      // first one always moves the reference off -inf
      if (__any(bm > mref + kMfmaLazy)) {
        const float mn = fmaxf(mref, bm);
        const float al = fast_exp2(mref - mn);
        lsum *= al;
#pragma unroll
        for (int m = 0; m < 8; ++m) o[m] *= al;
        mref = mn;
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(y[r] - mref);
      // the weights enter the products in bf16, so the sum takes them rounded
      const uint32_t p01 = pack_f32_bf16(p[0], p[1]);
      const uint32_t p23 = pack_f32_bf16(p[2], p[3]);
      lsum += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
      const bf16x4_t pb = __builtin_bit_cast(bf16x4_t, make_uint2(p01, p23));
#pragma unroll
      for (int m = 0; m < 8; ++m)
        o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, vf[m]), pb,
                                                         o[m], 0, 0, 0);
    }
  }
  // every load has landed (the trailing zero-length ones still write their
  // LDS tiles; the staged row is read below)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (store && wave == 0 && new_pos / kBlockSize < a.max_blocks_per_seq) {
    const int raw = a.block_tables[(int64_t)tseq * a.max_blocks_per_seq + new_pos / kBlockSize];
    if (raw >= 0 && (int64_t)raw < a.num_blocks && lane < 32) {
      // lanes 0-15 the V chunks, 16-31 the K chunks
      const int64_t dst = (((int64_t)raw * hkv + kvh) * kBlockSize + new_off) * (D / 8) + col;
      uint4* cache = static_cast<uint4*>(lane < 16 ? a.v_cache_w : a.k_cache_w);
      cache[dst] = stage[lane];
    }
  }

  // sums per head over the four token groups
  {
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                    false, false);
    lsum = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                    false, false);
    lsum = __uint_as_float(z[0]) + __uint_as_float(z[1]);
  }

  __syncthreads();  // every wave is done with its tiles, which sm overlaps
  if (col < G) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.acc[wave][col][16 * m + 4 * grp + r] = o[m][r];
    if (grp == 0) {
      sm.ml[wave][col][0] = mref;
      sm.ml[wave][col][1] = lsum;
    }
  }
  finish_item<true, D, G>(a, sm, seq, qrow, kvh, part, nparts);
  __syncthreads();  // sm overlaps the waves' tiles: read before the next item loads
}

// Merge the partitions of one (sequence, q head): weights 2^(m_p - max m), the
// accumulators summed in ascending partition order.  Runs after the partition
// kernel on the same stream; the kernel boundary makes the partials visible.
// The loads go out in few dependent rounds: the first B accumulators together
// with every (max, sum) pair (thread t holds partition t's), the weights
// through LDS, then the accumulators B partitions at a time (a cascade call's
// 33 partials: two rounds with B = 32, not the ten of one pass per value in
// batches of 8).  B = 8 when there are at most 8 partials.
constexpr int kMergeLdsParts = 1024;  // partitions whose weights LDS holds

template <int B, bool BF16, int D>
__device__ __forceinline__ void merge_row(const DecodeArgs& a, int nparts, int64_t prow,
                                          int64_t out_idx, float (&wts)[kMergeLdsParts],
                                          float (&red)[2][D / 64]) {
  constexpr float kNegInf = -INFINITY;
  constexpr int kWaves = D / 64;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const float* ml = a.ws.ml + prow * 2;
  const float* pacc = a.ws.acc + prow * D + t;

  // first round (indices past the last partition are clamped, values unused)
  float av[B];
#pragma unroll
  for (int j = 0; j < B; ++j) av[j] = pacc[(int64_t)min(j, nparts - 1) * D];
  float m_own = kNegInf, l_own = 0.f;
  if (t < nparts) {
    m_own = ml[2 * t];
    l_own = ml[2 * t + 1];
  }
  float mloc = m_own;
  for (int p = t + D; p < nparts; p += D) mloc = fmaxf(mloc, ml[2 * p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
  if (lane == 0) red[0][wave] = mloc;
  __syncthreads();
  float mx = red[0][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, red[0][w]);
  const float mref = (mx == kNegInf) ? 0.f : mx;
  // each partition's weight (into LDS) and the weighted sums: a thread's
  // partitions ascending, then across lanes and waves in a fixed order
  float lloc = 0.f;
  if (t < nparts) {
    const float wt = fast_exp2(m_own - mref);
    if (t < kMergeLdsParts) wts[t] = wt;
    lloc = wt * l_own;
  }
  for (int p = t + D; p < nparts; p += D) {
    const float wt = fast_exp2(ml[2 * p] - mref);
    if (p < kMergeLdsParts) wts[p] = wt;
    lloc += wt * ml[2 * p + 1];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lloc += __shfl_xor(lloc, off);
  if (lane == 0) red[1][wave] = lloc;
  __syncthreads();
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) lsum += red[1][w];

  auto weight = [&](int q) { return q < kMergeLdsParts ? wts[q] : fast_exp2(ml[2 * q] - mref); };
  float asum = 0.f;
#pragma unroll
  for (int j = 0; j < B; ++j)
    if (j < nparts) asum += weight(j) * av[j];
  for (int p = B; p < nparts; p += B) {
#pragma unroll
    for (int j = 0; j < B; ++j) av[j] = pacc[(int64_t)min(p + j, nparts - 1) * D];
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (p + j < nparts) asum += weight(p + j) * av[j];
  }
  store_elem<BF16>(a.out, out_idx, lsum > 0.f ? asum / lsum : 0.f);
}

template <bool BF16, int D, bool VARLEN>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float wts[kMergeLdsParts];
  __shared__ float red[2][D / 64];
  // one workgroup per (sequence, q head), q head fastest (a 1-D grid: packed
  // calls taken row by row can have more rows than a grid's y extent)
  const int seq = blockIdx.x / a.num_q_heads;
  const int h = blockIdx.x - seq * a.num_q_heads;
  int qrow, ctx;
  if (!decode_row<VARLEN>(a, seq, qrow, ctx)) return;
  const int nparts = a.prefix_parts + parts_of(ctx - a.key_start, a.part_tokens);
  if (nparts <= 1) return;
  const int hq = a.num_q_heads;
  const int64_t prow = ((int64_t)seq * hq + h) * a.max_parts;
  const int64_t out_idx = ((int64_t)qrow * hq + h) * D + threadIdx.x;
  if (nparts <= 8)
    merge_row<8, BF16, D>(a, nparts, prow, out_idx, wts, red);
  else
    merge_row<32, BF16, D>(a, nparts, prow, out_idx, wts, red);
}

// Every context fits one partition: one workgroup per (sequence, kv head).
// The tiles are read as streaming data: measured on MI355X with cold caches,
// the LLaMA-2-shaped decode step took 52.6 us against 58.3 with plain loads,
// 1536 rows of 256-2048 tokens 1185 us against 1295 (6.2 TB/s), 2048 rows of
// 64 tokens 112 against 115.  The hint costs where many sequences share
// blocks that the caches would otherwise serve to each of them: 256
// sequences sharing a 256-token prompt, caches warm, ran 8% slower; through
// the list kernel, 128 sequences sharing a 4096-token prompt 25% slower
// (353 us against 283) -- a known common prefix is better served by the
// cascade call, which reads it once (100 us).  The list kernel streams too:
// the GQA batch of Pareto lengths 77-78 us against 83, the shared-prefix
// batch 1.445 ms against 1.460 (without the hint, the zero-length loads past
// a wave's last block alone gained nothing).
// One item through the vector-ALU code or the matrix-core code (MF); dyn is
// the kernel's dynamic LDS, which starts with the waves' V tiles when MF.
template <bool BF16, int D, int G, bool VARLEN, int NB, bool MF, bool STREAM>
__device__ __forceinline__ void run_item(const DecodeArgs& a, int seq, int part, int kvh,
                                         DecodeShared<G, D>& sm, uint4* dyn) {
  if constexpr (MF) {
    static_assert(BF16 && D == 128, "matrix-core decode: bf16 at head_dim 128");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    decode_item_mfma<G, VARLEN, STREAM>(a, seq, part, kvh, sm, dyn + wave * kWaveTileChunks);
  } else {
    decode_item<BF16, D, G, VARLEN, NB, STREAM>(a, seq, part, kvh, sm);
  }
}

// The item's merge area: a static LDS array for the vector item code; for the
// matrix-core code the start of the dynamic LDS, over the waves' tiles.
template <int G, int D, bool MF>
__device__ __forceinline__ DecodeShared<G, D>& item_shared(uint4* dyn) {
  if constexpr (MF) {
    return *reinterpret_cast<DecodeShared<G, D>*>(dyn);
  } else {
    __shared__ DecodeShared<G, D> sm;
    return sm;
  }
}

// dynamic LDS of a decode kernel before any plan arrays: per wave, the K and
// V tiles and the new token's staged row (80 chunks: the second staging load
// writes 64 chunks from chunk 16); the item's merge area overlaps them
template <int G, bool MF>
constexpr size_t tile_lds_bytes(int waves) {
  return MF ? std::max((size_t)waves * kWaveTileChunks * 16, sizeof(DecodeShared<G, 128>)) : 0;
}

template <bool BF16, int D, int G, bool VARLEN, int NB, bool MF>
__global__ __launch_bounds__(256, MF ? 4 : 1) void decode_direct_kernel(DecodeArgs a) {
  extern __shared__ uint4 dyn_lds[];
  // kv head fastest: the workgroups of one sequence are dispatched together,
  // so no kv head's share of the work is left to the end of the launch
  const int hkv = a.num_kv_heads;
  const int seq = blockIdx.x / hkv;
  run_item<BF16, D, G, VARLEN, NB, MF, true>(a, seq, 0, blockIdx.x - seq * hkv,
                                            item_shared<G, D, MF>(dyn_lds), dyn_lds);
}

// One workgroup per (sequence, kv head, partition); partitions past a
// sequence's context exit at once.
template <bool BF16, int D, int G, bool VARLEN, int NB, bool MF>
__global__ __launch_bounds__(256, MF ? 4 : 1) void decode_grid_kernel(DecodeArgs a) {
  extern __shared__ uint4 dyn_lds[];
  run_item<BF16, D, G, VARLEN, NB, MF, false>(a, blockIdx.x, blockIdx.z, blockIdx.y,
                                             item_shared<G, D, MF>(dyn_lds), dyn_lds);
}

// The work list without a plan launch: each workgroup derives, from the
// lengths, the same (sequence, partition) order the plan kernel writes (every
// full-length partition in sequence order, then each sequence's shorter last
// one) as two exclusive scans in LDS: ex_full[s], the full partitions before
// sequence s, and ex_part[s], the short ones.  Item i < total_full belongs to
// the last s with ex_full[s] <= i; the rest likewise in ex_part.
constexpr int kInlinePlanChunk = 8;  // sequences per thread (up to 2048 with 4 waves)

template <bool VARLEN>
__device__ __forceinline__ void inline_plan(const DecodeArgs& a, int* ex_full, int* ex_part,
                                            int& total_full, int& total) {
  __shared__ int wtot[2][kDecodeMaxWaves];
  const int n = a.num_seqs;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int nw = blockDim.x >> 6;
  const int chunk = ceil_div(n, (int)blockDim.x);  // <= kInlinePlanChunk
  const int s0 = min(n, t * chunk);
  int nf[kInlinePlanChunk], np[kInlinePlanChunk];
  int full = 0, part = 0;
#pragma unroll
  for (int j = 0; j < kInlinePlanChunk; ++j) {
    nf[j] = 0;
    np[j] = 0;
    const int s = s0 + j;
    int qrow, ctx;
    if (j < chunk && s < n && decode_row<VARLEN>(a, s, qrow, ctx)) {
      ctx = max(ctx - a.key_start, 0);
      nf[j] = ctx / a.part_tokens;
      np[j] = (ctx % a.part_tokens != 0 || ctx == 0) ? 1 : 0;
    }
    full += nf[j];
    part += np[j];
  }
  // inclusive scans over the wave, then over the waves' totals
  int fi = full, pi = part;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int fu = __shfl_up(fi, off), pu = __shfl_up(pi, off);
    if (lane >= off) {
      fi += fu;
      pi += pu;
    }
  }
  if (lane == 63) {
    wtot[0][wave] = fi;
    wtot[1][wave] = pi;
  }
  __syncthreads();
  int fbase = 0, pbase = 0;
  total_full = 0;
  int total_part = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wave) {
      fbase += wtot[0][w];
      pbase += wtot[1][w];
    }
    total_full += wtot[0][w];
    total_part += wtot[1][w];
  }
  total = total_full + total_part;
  int fx = fbase + fi - full, px = pbase + pi - part;  // exclusive, at s0
#pragma unroll
  for (int j = 0; j < kInlinePlanChunk; ++j) {
    const int s = s0 + j;
    if (j < chunk && s < n) {
      ex_full[s] = fx;
      ex_part[s] = px;
    }
    fx += nf[j];
    px += np[j];
  }
  __syncthreads();
}

// last s in [0, n) with ex[s] <= x (ex non-decreasing, ex[0] = 0 <= x): a
// 64-way search, each lane testing one candidate per round
__device__ __forceinline__ int plan_find(const int* ex, int n, int x) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int step = ceil_div(hi - lo, 64);
    const int cand = lo + lane * step;
    const bool ok = cand < hi && ex[cand] <= x;
    const unsigned long long b = __ballot(ok);  // bit 0 is set: ex[lo] <= x
    lo += (63 - __builtin_clzll(b)) * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

// Persistent workgroups walk the (sequence, partition) list for kv head blockIdx.y.
template <bool BF16, int D, int G, bool VARLEN, int NB, bool MF>
__global__ __launch_bounds__(256, MF ? 4 : 1) void decode_list_kernel(DecodeArgs a) {
  extern __shared__ uint4 dyn_lds[];  // [tiles (MF)][inline plan: ex_full[n], ex_part[n]]
  int* plan_lds = reinterpret_cast<int*>(dyn_lds + tile_lds_bytes<G, MF>(a.waves) / 16);
  int total, total_full = 0;
  if (a.inline_plan)
    inline_plan<VARLEN>(a, plan_lds, plan_lds + a.num_seqs, total_full, total);
  else
    total = *a.ws.count;
  // kv head fastest: item slot blockIdx.x / hkv, so the list's longest-first
  // order holds across kv heads in dispatch order
  const int hkv = a.num_kv_heads;
  const int slot = blockIdx.x / hkv;
  const int kvh = blockIdx.x - slot * hkv;
  const int slots = gridDim.x / hkv;
  for (int it = slot; it < total; it += slots) {
    int seq, part;
    if (a.inline_plan) {
      const int* ex_full = plan_lds;
      if (it < total_full) {
        seq = plan_find(ex_full, a.num_seqs, it);
        part = it - ex_full[seq];
      } else {
        seq = plan_find(plan_lds + a.num_seqs, a.num_seqs, it - total_full);
        part = (seq + 1 < a.num_seqs ? ex_full[seq + 1] : total_full) - ex_full[seq];
      }
      seq = __builtin_amdgcn_readfirstlane(seq);
      part = __builtin_amdgcn_readfirstlane(part);
    } else {
      const int2 w = a.ws.items[it];
      seq = w.x;
      part = w.y;
    }
    run_item<BF16, D, G, VARLEN, NB, MF, true>(a, seq, part, kvh, item_shared<G, D, MF>(dyn_lds),
                                              dyn_lds);
  }
}

// One workgroup builds the (sequence, partition) list.  Full-length
// partitions come first, then each sequence's shorter last partition, both in
// sequence order: the persistent workgroups take items round-robin, so the
// expensive items are spread one per workgroup before the short ones fill in.
template <bool VARLEN>
__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a) {
  __shared__ int scan_full[1024];
  __shared__ int scan_part[1024];
  const int n = a.num_seqs;
  const int t = threadIdx.x;
  const int pt = a.part_tokens;
  const int chunk = ceil_div(n, (int)blockDim.x);
  const int s0 = min(n, t * chunk);
  const int s1 = min(n, s0 + chunk);
  int full = 0, partial = 0;
  for (int s = s0; s < s1; ++s) {
    int qrow, ctx;
    if (!decode_row<VARLEN>(a, s, qrow, ctx)) continue;
    ctx = max(ctx - a.key_start, 0);  // keys this call attends
    full += ctx / pt;
    partial += (ctx % pt != 0 || ctx == 0) ? 1 : 0;
  }
  scan_full[t] = full;
  scan_part[t] = partial;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    const int af = t >= off ? scan_full[t - off] : 0;
    const int ap = t >= off ? scan_part[t - off] : 0;
    __syncthreads();
    scan_full[t] += af;
    scan_part[t] += ap;
    __syncthreads();
  }
  const int total_full = scan_full[blockDim.x - 1];
  int pos_full = scan_full[t] - full;
  int pos_part = total_full + scan_part[t] - partial;
  for (int s = s0; s < s1; ++s) {
    int qrow, ctx;
    if (!decode_row<VARLEN>(a, s, qrow, ctx)) continue;
    ctx = max(ctx - a.key_start, 0);
    const int nf = ctx / pt;
    for (int p = 0; p < nf; ++p) a.ws.items[pos_full++] = make_int2(s, p);
    if (ctx % pt != 0 || ctx == 0) a.ws.items[pos_part++] = make_int2(s, nf);
  }
  if (t == (int)blockDim.x - 1) *a.ws.count = total_full + scan_part[t];
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

template <bool BF16, int D, int G, bool VARLEN, int NB, bool MF>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 block(64 * a.waves);
  const size_t tiles = tile_lds_bytes<G, MF>(a.waves);
  if (a.max_parts - a.prefix_parts <= 1) {
    // one partition per context (or per private part of a cascade decode,
    // whose partials the merge then combines with the prefix's)
    hipLaunchKernelGGL((decode_direct_kernel<BF16, D, G, VARLEN, NB, MF>),
                       dim3((unsigned)a.num_seqs * a.num_kv_heads), block, tiles, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.prefix_parts == 0) return e;
    hipLaunchKernelGGL((decode_merge_kernel<BF16, D, VARLEN>),
                       dim3((unsigned)a.num_q_heads * a.num_seqs), dim3(D), 0, stream, a);
    return hipGetLastError();
  }
  hipError_t err;
  if (a.grid_mode) {
    hipLaunchKernelGGL((decode_grid_kernel<BF16, D, G, VARLEN, NB, MF>),
                       dim3(a.num_seqs, a.num_kv_heads, a.max_parts), block, tiles, stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((decode_merge_kernel<BF16, D, VARLEN>),
                       dim3((unsigned)a.num_q_heads * a.num_seqs),
                       dim3(D), 0, stream, a);
    return hipGetLastError();
  }
  size_t plan_lds = tiles;
  if (a.inline_plan) {
    plan_lds += 2 * sizeof(int) * (size_t)a.num_seqs;
  } else {
    hipLaunchKernelGGL((decode_plan_kernel<VARLEN>), dim3(1), dim3(1024), 0, stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // resident workgroups per CU of this instance, per wave count (computed once;
  // concurrent first calls compute the same value)
  static std::atomic<int> per_cu[kDecodeMaxWaves + 1];
  int resident = per_cu[a.waves].load(std::memory_order_relaxed);
  if (resident == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(&decode_list_kernel<BF16, D, G, VARLEN, NB, MF>),
            64 * a.waves, tiles) != hipSuccess ||
        nb <= 0)
      nb = 2;
    resident = nb;
    per_cu[a.waves].store(nb, std::memory_order_relaxed);
  }
  // a multiple of the resident capacity, so a finished workgroup's slot is refilled
  const int64_t want = (int64_t)a.oversub * resident * device_cus();
  const int64_t items_bound = (int64_t)a.num_seqs * a.max_parts;
  const int gx = (int)std::max<int64_t>(
      1, std::min<int64_t>(items_bound, (want + a.num_kv_heads - 1) / a.num_kv_heads));
  hipLaunchKernelGGL((decode_list_kernel<BF16, D, G, VARLEN, NB, MF>),
                     dim3((unsigned)gx * a.num_kv_heads), block, plan_lds, stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_merge_kernel<BF16, D, VARLEN>),
                       dim3((unsigned)a.num_q_heads * a.num_seqs),
                     dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16, int D, int G, bool VARLEN>
static hipError_t launch_buffers(const DecodeArgs& a, hipStream_t s) {
  if constexpr (BF16 && D == 128) {
    if (a.mfma) return launch_decode_t<BF16, D, G, VARLEN, 1, true>(a, s);
    switch (a.buffers) {
      case 1: return launch_decode_t<BF16, D, G, VARLEN, 1, false>(a, s);
      case 3: return launch_decode_t<BF16, D, G, VARLEN, 3, false>(a, s);
      case 4: return launch_decode_t<BF16, D, G, VARLEN, 4, false>(a, s);
      default: return launch_decode_t<BF16, D, G, VARLEN, 2, false>(a, s);
    }
  } else {
    return launch_decode_t<BF16, D, G, VARLEN, 2, false>(a, s);
  }
}

template <bool BF16, int D, int G>
static hipError_t launch_mode(const DecodeArgs& a, hipStream_t s) {
  return a.varlen ? launch_buffers<BF16, D, G, true>(a, s) : launch_buffers<BF16, D, G, false>(a, s);
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

static int env_int(const char* name, int fallback) {
  const char* v = getenv(name);
  if (!v || !*v) return fallback;
  char* end = nullptr;
  const long x = strtol(v, &end, 10);
  return (end && *end == 0) ? (int)x : fallback;
}

void decode_config(int num_seqs, int num_kv_heads, int max_context_len, int* waves,
                   int* part_tokens, int* buffers, int* grid_mode, int* oversub) {
  // Measured on MI355X (cold caches): 4 waves, 2 buffers and 512-token
  // partitions are best up to a few thousand tokens; for very long contexts
  // 1024-token partitions halve the partial traffic and the item count.  When
  // (sequence, kv head) pairs alone fill the chip twice over (>= 4096 of them)
  // and no context is longer than one workgroup covers in a single item, a
  // split only adds partial traffic and a merge launch: one partition per
  // context (mixed decode/prefill steps of ~750 decode rows at <= 2048 tokens
  // ran 10% faster that way).
  int w = 4, pt = max_context_len >= 8192 ? 1024 : 512, nb = 0;  // nb 0: chosen at launch
  const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
  // Many short contexts: an item of a few blocks spreads them over fewer
  // waves, which saves the cross-wave merge, and there are items enough to
  // fill the chip (2048 sequences of 64 tokens, g=4: 116 us with one wave per
  // item against 181 us with four; 1024 of 100 tokens: 98 against 115).
  if (max_context_len <= 256 && pairs >= 8192) w = 1;
  else if (max_context_len <= 512 && pairs >= 4096) w = 2;
  const int whole = ceil_div(max(max_context_len, 1), kBlockSize) * kBlockSize;
  if (pairs >= 4096 && whole <= kBlockSize * kMaxEntriesPerWave * w) pt = max(pt, whole);
  // Contexts of at most 1024 tokens: one partition each from 1024 pairs on
  // (the single-partition kernel's streaming loads and no merge).  Measured:
  // 256 sequences x 8 kv heads of U[64, 1024] tokens 111 us against 137 split
  // at 512; 128 of them 58 against 63; Pareto lengths clipped at 1024, 54
  // against 57.  Not for longer contexts, where a few long ones in a skewed
  // batch become the tail (Pareto clipped at 2048, 1024 pairs: 63 against 39).
  else if (pairs >= 1024 && whole <= 1024) pt = max(pt, whole);
  // tuning overrides; only values that keep every access in bounds are taken
  const int ew = env_int("PA_DECODE_WAVES", 0);
  if (ew == 1 || ew == 2 || ew == 4) w = ew;
  const int ept = env_int("PA_DECODE_PARTITION", 0);
  if (ept >= kMinPartitionTokens && ept % kBlockSize == 0) pt = ept;
  if (pt > kBlockSize * kMaxEntriesPerWave * w) pt = kBlockSize * kMaxEntriesPerWave * w;
  const int enb = env_int("PA_DECODE_BUFFERS", 0);
  if (enb >= 1 && enb <= 4) nb = enb;
  *waves = w;
  *part_tokens = pt;
  *buffers = nb;
  *grid_mode = env_int("PA_DECODE_GRID", 0) == 1;
  const int eo = env_int("PA_DECODE_OVERSUB", 0);
  *oversub = (eo >= 1 && eo <= 8) ? eo : 4;
}

bool decode_inline_plan(int num_seqs, int waves) {
  // every thread of the workgroup scans at most kInlinePlanChunk sequences
  return num_seqs <= kInlinePlanChunk * 64 * waves && env_int("PA_DECODE_INLINE_PLAN", 1) != 0;
}

hipError_t launch_decode(const DecodeArgs& args, hipStream_t stream) {
  if (args.num_seqs == 0) return hipSuccess;
  DecodeArgs a = args;
  // bf16 at head_dim 128: the matrix cores take the score and value products
  // (PA_DECODE_MFMA=0: the vector code).  Measured against the vector code on
  // one box: the LLaMA-2-shaped step (g = 1) 49.6 us against 50.8, the GQA
  // batch (g = 4) 68.5 against 75.5, the same lengths at g = 2 55.9 against
  // 60.1, long and short g = 1 batches 0.5-1.7% faster.
  a.mfma = a.dtype == PA_BF16 && a.head_dim == 128 && env_int("PA_DECODE_MFMA", 1) != 0;
  // Split contexts on the matrix-core code: one wave per item (no cross-wave
  // merge, items balance across the chip on their own).  Measured against
  // four: the GQA Pareto batch 63.5 us against 68.3, the 4096-token common
  // prompt 240 against 284, the long shared-prefix batch 1.391 ms against
  // 1.426.  A wave holds 64 table entries, so partitions up to 1024 tokens.
  if (a.mfma && a.max_parts - a.prefix_parts > 1 &&
      a.part_tokens <= kBlockSize * kMaxEntriesPerWave && env_int("PA_DECODE_WAVES", 0) == 0)
    a.waves = 1;
  // Contexts of at most 512 tokens in one partition each, from 2048 (sequence,
  // kv head) pairs, on the matrix-core code: two waves per item (each wave
  // still streams several blocks, and the cross-wave merge halves).  Measured
  // against four in six alternating runs: the LLaMA-2-shaped step 48.86-48.98
  // us against 49.18-49.27.  Longer contexts keep four (the mixed step's
  // decode rows of up to 2048 tokens: 0.671 ms with two against 0.659).
  if (a.mfma && a.max_parts - a.prefix_parts <= 1 && a.waves == 4 && a.max_context_len <= 512 &&
      (int64_t)a.num_seqs * a.num_kv_heads >= 2048 && env_int("PA_DECODE_WAVES", 0) == 0)
    a.waves = 2;
  a.inline_plan = decode_inline_plan(a.num_seqs, a.waves) ? 1 : 0;
  // K/V register buffers per wave of the vector item code (bf16 at head_dim
  // 128 with PA_DECODE_MFMA=0), unless set: two on the single-partition
  // kernel; one on the split kernels, whose item code then fits 128 VGPRs (4
  // waves per SIMD instead of 3): the Pareto GQA batch 82 us against 83.6,
  // the 4096-token common prompt 253 against 263, the long shared-prefix
  // batch within 0.5%.
  if (a.buffers == 0) a.buffers = a.max_parts - a.prefix_parts <= 1 ? 2 : 1;
  if (a.mfma) a.buffers = 1;  // the matrix-core item code overlaps one block ahead itself
  return a.dtype == PA_BF16 ? launch_dim<true>(a, stream) : launch_dim<false>(a, stream);
}

}  // namespace pa
