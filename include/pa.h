/*
 * pa.h -- C ABI of the paged-attention library for AMD Instinct MI355X (gfx950).
 *
 * Attention over a KV cache that is split into fixed-size physical blocks of
 * 16 tokens, drawn from one pool shared by every sequence and addressed through
 * a per-sequence block table.
 *
 * Sources, cited by page title and section:
 *   "vLLM：颠覆大模型推理的高效API服务引擎深度解析" (below: [KW])
 *       §1.2  fixed-size blocks; a block table per request mapping logical blocks
 *             to physical ones.
 *       §1.3  one pre-allocated pool shared by all requests; the new token's
 *             K/V are stored into a physical block; attention gathers the
 *             scattered blocks through the block table into a logically
 *             contiguous cache; blocks may be shared read-only by several
 *             block tables.
 *       §2.2  the worker runs a fused kernel that reads the KV cache straight
 *             from the scattered physical blocks.
 *   "vLLM изнутри: как устроен движок для быстрого инференса LLM" (below: [VI])
 *       allocate_slots paragraph: 16 tokens per block by default, ceil(n/16)
 *             blocks for n tokens.
 *       forward-pass paragraph: the model runner builds the slot mapping and
 *             attention metadata; all sequences of a step are packed into one
 *             super-sequence whose masks and positions keep each sequence on
 *             its own tokens.
 *       the paragraph on the three stages of a step: prefill is compute-bound,
 *             decode is memory-bandwidth-bound.
 *
 * Conventions (every call):
 *   - All array pointers are device pointers into caller-owned memory (e.g.
 *     PyTorch tensors).  The library allocates nothing and keeps no state; it
 *     is reentrant.  Work is enqueued on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream) and the calls return without waiting.
 *   - Arrays are dense row-major with the shapes given below.
 *   - KV cache layout, K and V alike:
 *         [num_blocks][num_kv_heads][block_size][head_dim]
 *     so one (block, kv head) tile of 16 tokens is one contiguous run of
 *     16 * head_dim elements.  The slot of a token is
 *         physical_block * block_size + offset_in_block.
 *   - Element types: PA_F32 (float) or PA_BF16 (bfloat16, 2 bytes).  Queries,
 *     keys, values, caches and outputs of one call share the element type.
 *     Accumulation is always fp32; outputs are rounded to nearest-even.
 *   - Supported shapes: block_size == 16; head_dim 64 or 128;
 *     num_q_heads == g * num_kv_heads with g in {1, 2, 4, 8}; q head h reads
 *     kv head h / g (contiguous groups).
 *   - Return value: PA_OK, or a non-zero pa_status for a fault the host can
 *     see (null pointer, unsupported shape or type, bad count, workspace too
 *     small, launch failure).  Host-side checks happen before anything is
 *     enqueued: a call that returns an error has launched nothing.  No
 *     exception or abort crosses this ABI.
 *   - Device-resident integer inputs are not validated on the host (that would
 *     need a device-to-host copy).  Kernels keep every access in bounds
 *     regardless: a block id outside [0, num_blocks) is treated as an empty
 *     block (its tokens take no part), a context length above the stated
 *     maxima is clamped to them, and a slot outside the pool is not written.
 *     Such inputs still give meaningless results for the affected rows.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_VERSION 100 /* 1.0.0 */
#define PA_BLOCK_SIZE 16

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_BF16 = 1
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  PA_ERR_UNSUPPORTED = 2,         /* dtype, head_dim, block_size or head ratio */
  PA_ERR_INVALID_ARGUMENT = 3,    /* negative or inconsistent count, non-finite scale */
  PA_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes below the size query */
  PA_ERR_HIP = 5,                 /* the HIP runtime refused a launch */
  PA_ERR_NO_FREE_BLOCKS = 6,      /* block manager: the free queue is too short */
  PA_ERR_HOST_MEMORY = 7,         /* block manager: a host allocation failed */
  PA_ERR_SCRATCH_TOO_SMALL = 8    /* pa_decode_noalloc: shapes beyond its fixed scratch */
} pa_status;

/* Library version as PA_VERSION. */
int32_t pa_version(void);

/* Static, NUL-terminated description of a status code. */
const char* pa_status_string(int32_t status);

/*
 * pa_build_slot_mapping -- cache slot of every new token of a packed step
 * ([VI] forward-pass paragraph: the runner builds the slot mapping; [KW] §1.2:
 * the block table maps logical blocks to physical ones).
 *
 *   slot_mapping     out  int64 [num_tokens]
 *   cu_seqlens       in   int32 [num_seqs + 1], cu_seqlens[0] = 0,
 *                         cu_seqlens[num_seqs] = num_tokens; sequence i owns
 *                         packed tokens cu_seqlens[i] .. cu_seqlens[i+1]-1
 *   context_offsets  in   int32 [num_seqs]: tokens of sequence i already in
 *                         the cache; its j-th new token is at position
 *                         context_offsets[i] + j
 *   block_tables     in   int32 [num_seqs][max_blocks_per_seq]
 *
 * slot = block_tables[i][pos / block_size] * block_size + pos % block_size.
 * A position whose logical block is past max_blocks_per_seq gets slot -1
 * (stored nowhere by pa_write_kv).  Token indices that inconsistent
 * cu_seqlens place outside [0, num_tokens) are not written.
 */
int32_t pa_build_slot_mapping(int64_t* slot_mapping, const int32_t* cu_seqlens,
                              const int32_t* context_offsets, const int32_t* block_tables,
                              int32_t num_seqs, int64_t num_tokens,
                              int32_t max_blocks_per_seq, int32_t block_size, void* stream);

/*
 * pa_write_kv -- store new tokens' K and V into their cache slots ([KW] §1.3:
 * the new token's K/V vectors are stored into the allocated physical block).
 *
 *   key, value       in   [num_tokens][num_kv_heads][head_dim]
 *   k_cache, v_cache in/out  [num_blocks][num_kv_heads][block_size][head_dim]
 *   slot_mapping     in   int64 [num_tokens]; slot < 0 marks padding (skipped)
 *
 * A bit-exact copy.  Slots at or beyond num_blocks * block_size are skipped.
 * Two tokens with the same slot: which one is stored is unspecified.
 */
int32_t pa_write_kv(const void* key, const void* value, void* k_cache, void* v_cache,
                    const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                    void* stream);

/*
 * Bytes of device workspace pa_decode needs for these shapes (0 when the
 * longest context fits one split-K partition).  Depends on shapes only.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t dtype);

/*
 * pa_decode -- one query token per sequence attends to all of its cached
 * tokens, read straight from the paged cache ([KW] §1.3 gather through the
 * block table, §2.2 fused kernel; [VI]: decode is bound by memory bandwidth).
 *
 *   out              out  [num_seqs][num_q_heads][head_dim]
 *   q                in   [num_seqs][num_q_heads][head_dim]
 *   k_cache, v_cache in   cache layout above
 *   block_tables     in   int32 [num_seqs][max_blocks_per_seq]; only the first
 *                         ceil(context_lens[i] / block_size) entries are read
 *   context_lens     in   int32 [num_seqs]: tokens in the cache for sequence i,
 *                         including this step's new token (write it first)
 *   max_context_len       host copy of max(context_lens) (sizes the grid)
 *   scale                 softmax scale, usually 1/sqrt(head_dim); any finite
 *                         value (0 weighs every key alike, a negative one favours
 *                         the smallest scores); NaN or an infinity is refused
 *                         with PA_ERR_INVALID_ARGUMENT (every attention call)
 *   workspace             device scratch of >= pa_decode_workspace_size(...)
 *                         bytes (may be NULL when that size is 0)
 *
 * out[i][h] = sum_t softmax_t(scale * <q[i][h], K_i[t][h/g]>) V_i[t][h/g]
 * over t < context_lens[i]; a sequence with context 0 gets a zero row.  The
 * result depends only on the logical token order: the same for any physical
 * placement of the blocks and for blocks shared between sequences.
 */
int32_t pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
                  int64_t num_blocks, float scale, int32_t dtype, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  It calls no allocator.
 *
 *   arguments        as pa_decode, minus workspace and workspace_bytes
 *
 * Same kernels, launch choice and result as pa_decode (bit-identical).  The
 * split-K partials and work list live in a fixed device buffer of
 * PA_NOALLOC_SCRATCH_BYTES (128 MiB) that the library holds on every GPU it
 * runs on until the process ends; the first call on a device looks up that
 * device's copy.  A call whose partials need more (num_seqs * num_q_heads *
 * partitions * (head_dim + 2) * 4 bytes plus 8 bytes per work item, when some
 * context spans several partitions; e.g. 128 sequences x 32 q heads with
 * contexts up to 32768 tokens, 32 partitions of 1024, take 68 MB) returns
 * PA_ERR_SCRATCH_TOO_SMALL and launches nothing.  Nothing in the buffer needs
 * to start at zero: every value a call reads it has written earlier in the
 * same call.  All calls on one GPU share the buffer, which keeps the last
 * call's contents: calls that overlap in time on one GPU (several streams or
 * threads) race and give wrong results, so serialise them.  Errors otherwise
 * as pa_decode (PA_ERR_HIP also when the device's buffer cannot be found).
 */
#define PA_NOALLOC_SCRATCH_BYTES (128u << 20)

int32_t pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t max_context_len, int64_t num_blocks, float scale, int32_t dtype,
                          void* stream);

/*
 * pa_decode_step -- one decode step in a single launch: store each sequence's
 * new token and attend ([KW] §1.3: store the new token's K/V into its block,
 * then gather through the block table; the same result as pa_build_slot_mapping
 * + pa_write_kv + pa_decode, fused so that the step pays one launch).
 *
 *   key, value       in   [num_seqs][num_kv_heads][head_dim]: the new token of
 *                         sequence i, at position context_lens[i] - 1
 *   k_cache, v_cache in/out  the new token is stored into slot
 *                         block_tables[i][(ctx-1)/16] * 16 + (ctx-1) % 16
 *   other arguments  as pa_decode (context_lens includes the new token;
 *                         workspace size from pa_decode_workspace_size)
 *
 * The new token's K/V take part in the attention from the inputs, so the
 * result does not depend on when the store becomes visible.  Its position is
 * context_lens[i] - 1 as given, before any clamp to max_context_len or the
 * table's size: it is stored into that position's slot whenever the
 * position's block lies inside the table row and names a block of the pool
 * (what pa_build_slot_mapping + pa_write_kv store), and it takes part in the
 * attention only when the clamped context still includes it.  So an
 * understated max_context_len never redirects the store onto an older token.
 */
int32_t pa_decode_step(void* out, const void* q, const void* key, const void* value,
                       void* k_cache, void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                       float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Bytes of device workspace pa_cascade_decode needs for these shapes (never
 * less than pa_decode_workspace_size of the same shapes).  Depends on shapes
 * only.
 */
size_t pa_cascade_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t num_common_prefix_blocks, int32_t dtype);

/*
 * pa_cascade_decode -- pa_decode for sequences whose block tables begin with
 * the same physical blocks: a common prompt prefix whose blocks every table
 * references read-only ([KW] §1.3: blocks shared by several block tables;
 * "vLLMつかったら、ベクトル検索サーバーが高速化して安定性も向上した", the walk
 * through Scheduler.schedule(): a step's scheduler output carries the number
 * of blocks common to all of its requests).
 *
 *   num_common_prefix_blocks  P, in [0, max_blocks_per_seq]: the first P
 *                         entries of every block-table row name the same
 *                         blocks (precondition; only row 0's are read for
 *                         them).  A sequence whose context ends inside the
 *                         prefix attends only its first context_lens[i] keys.
 *   workspace             device scratch of >= pa_cascade_workspace_size(...)
 *                         bytes
 *   other arguments  as pa_decode
 *
 * The same attention as pa_decode (up to rounding order and the bf16 rounding
 * of the prefix's softmax weights).  For bf16 at head_dim 128 the prefix is
 * attended once per kv head for all sequences on the matrix cores, its rows
 * being the g query heads of each sequence, and the rest of every context by
 * the decode kernels; the partial results are combined by their
 * max-rescaled sums.  Other types and head sizes, and P = 0, run pa_decode.
 */
int32_t pa_cascade_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t max_context_len, int64_t num_blocks,
                          int32_t num_common_prefix_blocks, float scale, int32_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace pa_varlen_prefill needs for these shapes.
 */
size_t pa_varlen_workspace_size(int32_t num_seqs, int32_t total_q_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                                int32_t dtype);

/*
 * pa_varlen_prefill -- attention over one packed super-sequence of prefill
 * chunks and decode rows ([VI] forward-pass paragraph: sequences packed into
 * one super-sequence with per-sequence masks and positions; the V1 scheduler
 * mixes prefill and decode requests in one step).
 *
 *   out              out  [total_q_tokens][num_q_heads][head_dim]
 *   q                in   [total_q_tokens][num_q_heads][head_dim]
 *   cu_seqlens       in   int32 [num_seqs + 1]: sequence i owns query rows
 *                         cu_seqlens[i] .. cu_seqlens[i+1]-1
 *   context_offsets  in   int32 [num_seqs]: tokens of sequence i cached before
 *                         this step; its j-th row sits at position
 *                         context_offsets[i] + j
 *   block_tables     in   int32 [num_seqs][max_blocks_per_seq]
 *   max_q_len, max_context_len  host copies of max(q_len_i) and
 *                         max(context_offsets[i] + q_len_i)
 *
 * The K/V of every row (positions up to context_offsets[i] + q_len_i - 1) must
 * already be in the cache (pa_write_kv first).  Row j of sequence i attends
 * keys 0 .. context_offsets[i] + j of its own sequence (causal, its own key
 * included).  For PA_BF16 at head_dim 128, rows of single-token sequences
 * take the decode kernels and longer chunks the matrix-core prefill kernel;
 * for PA_F32, or head_dim 64, every row takes the decode kernels on its own
 * (same result, without the matrix-core reuse of each K/V tile across a
 * chunk's rows).
 */
int32_t pa_varlen_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* cu_seqlens, const int32_t* context_offsets,
                          const int32_t* block_tables, int32_t num_seqs, int32_t total_q_tokens,
                          int32_t max_q_len, int32_t max_context_len, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                          int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_varlen_prefill_ex -- pa_varlen_prefill with the host's count of the
 * step's single-token rows ([VI] forward-pass paragraph: the runner builds
 * the step's attention metadata on the host, where it knows how many of the
 * packed sequences are decode rows).
 *
 *   num_decode_rows  host count of sequences with exactly one query row, or
 *                    any negative value for "unknown" (then the call is
 *                    pa_varlen_prefill).  With 0 the call launches no decode
 *                    kernels (a prefill-only step saves their launches); a
 *                    positive count runs them as pa_varlen_prefill does.
 *
 * A count of 0 while some sequence has exactly one query row leaves that
 * row of `out` unwritten on the matrix-core path (PA_BF16, head_dim 128;
 * nothing is read or written out of bounds); the other types and head dims
 * take every row through the decode kernels and ignore the count.
 * Arguments, workspace (pa_varlen_workspace_size) and errors otherwise as
 * pa_varlen_prefill; with a true count the output is bit-identical to it.
 */
int32_t pa_varlen_prefill_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* cu_seqlens, const int32_t* context_offsets,
                             const int32_t* block_tables, int32_t num_seqs,
                             int32_t total_q_tokens, int32_t max_q_len, int32_t max_context_len,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                             float scale, int32_t dtype, int32_t num_decode_rows,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_swap_blocks -- copy whole blocks between two block pools of one layout
 * ([KW] §2.2: the block manager moves inactive blocks out to host memory
 * when device memory runs short and back in when they are needed; the same
 * call copies blocks inside one pool).
 *
 *   dst, src         pools of dst_num_blocks / src_num_blocks blocks of
 *                    block_bytes each (for one K or V cache:
 *                    num_kv_heads * 16 * head_dim * element bytes).  Each is
 *                    device memory or pinned host memory (hipHostMalloc,
 *                    torch pin_memory), which the kernel reads or writes
 *                    over the host link.
 *   block_pairs      int64 [num_pairs][2]: (source block, destination block);
 *                    device or pinned host memory
 *   block_bytes      a positive multiple of 16
 *
 * dst[pair.dst] = src[pair.src], bit for bit.  A pair with an id outside its
 * pool is skipped.  Two pairs must not write the same destination block, and
 * within one pool no pair may read a block another pair writes (the order of
 * the copies is unspecified).
 * Errors: NULL pointers, num_pairs < 0, block_bytes, a pointer the runtime
 * knows as neither device nor pinned host memory (PA_ERR_INVALID_ARGUMENT;
 * nothing is launched).
 */
int32_t pa_swap_blocks(void* dst, const void* src, const int64_t* block_pairs, int64_t num_pairs,
                       int64_t block_bytes, int64_t dst_num_blocks, int64_t src_num_blocks,
                       void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* PA_H_ */
