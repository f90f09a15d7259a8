/*
 * pa_blocks.h -- host-side block manager for the paged KV cache (C ABI).
 *
 * The bookkeeping that runs just before the attention path: a pool of
 * physical blocks, a free-block queue, a block table per sequence, reference
 * counts for blocks shared read-only by several sequences, and the builder of
 * a step's attention metadata (block tables, packing offsets, slot mapping).
 *
 * Sources, cited by page title and section:
 *   "vLLM изнутри: как устроен движок для быстрого инференса LLM" ([VI])
 *       engine-core paragraph: the KV-cache manager keeps a queue of free
 *             blocks (free_block_queue) from which requests get blocks;
 *       allocate_slots paragraph: it counts the new blocks a request needs
 *             (16 tokens per block, ceil(17/16) = 2), checks that the pool has
 *             that many free, and otherwise the request is not scheduled this
 *             step (or a running one is preempted -- a scheduler decision,
 *             left to the caller here);
 *       forward-pass paragraph: the runner builds the slot mapping and the
 *             attention metadata of the packed step.
 *   "vLLM：颠覆大模型推理的高效API服务引擎深度解析" ([KW])
 *       §1.2  a block table per request: logical block -> physical block and
 *             the number of tokens stored in each logical block (16 / 8 / 0);
 *       §1.3  one pre-allocated pool shared by all requests; blocks of a
 *             common prefix referenced read-only by several block tables;
 *       §2.1  the blocks of a finished request return to the free pool at
 *             once.
 *
 * Conventions:
 *   - Everything here runs on the host; every pointer is a host pointer.  A
 *     manager is a plain C++ object behind an opaque handle: not thread-safe
 *     (one owner, e.g. the scheduler thread).
 *   - Block ids are 0 .. num_blocks-1, the row index of the device caches
 *     (include/pa.h: [num_blocks][num_kv_heads][16][head_dim]).
 *   - The free queue starts as 0, 1, ..., num_blocks-1; allocation takes from
 *     its front, freed blocks join its back.
 *   - Sequence ids are caller-chosen int64 values.
 *   - Return value: PA_OK or a pa_status (include/pa.h).  A call that fails
 *     changes nothing.  The free queue is sized to the pool at creation;
 *     pa_bm_create, pa_bm_allocate_slots (a new sequence or a longer block
 *     list) and pa_bm_share_prefix allocate host memory and return
 *     PA_ERR_HOST_MEMORY if that fails.  No C++ exception leaves a call.
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/*
 * pa_bm_create -- a manager over num_blocks physical blocks of block_size
 * tokens (block_size must be 16).  *out receives the handle; release it with
 * pa_bm_destroy.  Errors: NULL out, num_blocks < 1 or > 2^31-1, block_size.
 */
int32_t pa_bm_create(int64_t num_blocks, int32_t block_size, pa_block_manager** out);

/* pa_bm_destroy -- release a manager (NULL is ignored). */
void pa_bm_destroy(pa_block_manager* bm);

/* Blocks currently in the free queue (-1 for a NULL handle). */
int64_t pa_bm_num_free_blocks(const pa_block_manager* bm);

/*
 * pa_bm_allocate_slots -- make room for num_new_tokens more tokens of
 * sequence seq_id ([VI] allocate_slots), creating the sequence if it is new.
 *
 * The sequence must afterwards own ceil((tokens + num_new_tokens +
 * num_lookahead_tokens) / 16) blocks, where tokens is its current count; the
 * missing ones come from the front of the free queue.  num_lookahead_tokens
 * reserves room for tokens written later without counting them (e.g.
 * candidate tokens); it does not change the token count.  On success the
 * token count grows by num_new_tokens.
 *
 * Errors: PA_ERR_NO_FREE_BLOCKS when the queue holds fewer blocks than needed
 * (nothing is taken: the caller may skip or preempt, then retry);
 * PA_ERR_INVALID_ARGUMENT for negative counts or a count past 2^31-1 tokens.
 */
int32_t pa_bm_allocate_slots(pa_block_manager* bm, int64_t seq_id, int32_t num_new_tokens,
                             int32_t num_lookahead_tokens);

/*
 * pa_bm_allocate_batch -- pa_bm_allocate_slots for seq_ids[i] with
 * num_new_tokens[i], i = 0 .. num_seqs-1 in order (one scheduling step in one
 * call), stopping at the first sequence the free queue cannot serve.
 * *num_served receives how many were served; those before it are allocated
 * exactly as by pa_bm_allocate_slots, nothing is taken for the rest.
 *
 * Returns PA_OK when all were served, PA_ERR_NO_FREE_BLOCKS when the queue ran
 * short at sequence *num_served (the caller may preempt and retry from
 * there), PA_ERR_INVALID_ARGUMENT for an invalid count (at *num_served, the
 * earlier ones served), PA_ERR_NULL_POINTER for NULL arrays.
 */
int32_t pa_bm_allocate_batch(pa_block_manager* bm, const int64_t* seq_ids,
                             const int32_t* num_new_tokens, int32_t num_seqs,
                             int32_t num_lookahead_tokens, int32_t* num_served);

/*
 * pa_bm_share_prefix -- start sequence dst_seq (which must not exist) on the
 * first num_tokens tokens of src_seq by reference ([KW] §1.3 read-only
 * sharing of a common prefix).  Only whole blocks are shared: dst_seq gets
 * src's first floor(num_tokens / 16) blocks (each reference count + 1) and a
 * token count of 16 * that; a partial last block is not shared (its tokens
 * are recomputed into a block of dst's own).
 *
 * Errors: unknown src_seq, existing dst_seq, src == dst, num_tokens < 0 or
 * past src's token count (PA_ERR_INVALID_ARGUMENT).
 */
int32_t pa_bm_share_prefix(pa_block_manager* bm, int64_t src_seq, int64_t dst_seq,
                           int32_t num_tokens);

/*
 * pa_bm_free_sequence -- forget seq_id: each of its blocks loses one
 * reference, and a block nobody references any more joins the back of the
 * free queue at once ([KW] §2.1), in table order.
 * Errors: unknown seq_id (PA_ERR_INVALID_ARGUMENT).
 */
int32_t pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);

/*
 * pa_bm_sequence_info -- token and block counts of seq_id (either output
 * pointer may be NULL).  Errors: unknown seq_id.
 */
int32_t pa_bm_sequence_info(const pa_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                            int32_t* num_blocks);

/* Reference count of a block (0 = free; -1 for an id outside the pool). */
int32_t pa_bm_block_refcount(const pa_block_manager* bm, int64_t block_id);

/*
 * pa_bm_block_table -- copy seq_id's block table into out[0 .. capacity-1];
 * entries past its block count are set to -1.  Errors: unknown seq_id, NULL
 * out, capacity below the block count (PA_ERR_INVALID_ARGUMENT).
 */
int32_t pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out,
                          int32_t capacity);

/*
 * pa_bm_build_step -- host-side attention metadata of one packed step
 * ([VI] forward-pass paragraph) for sequences seq_ids[0 .. num_seqs-1],
 * whose newest q_lens[i] tokens (already counted by pa_bm_allocate_slots)
 * are the step's new tokens:
 *
 *   block_tables     out  int32 [num_seqs][max_blocks_per_seq], rows padded
 *                         with -1
 *   cu_seqlens       out  int32 [num_seqs + 1], running sum of q_lens
 *   context_offsets  out  int32 [num_seqs]: tokens before the step
 *   context_lens     out  int32 [num_seqs]: tokens after the step
 *   slot_mapping     out  int64 [cu_seqlens[num_seqs]]: the slot of each new
 *                         token, block * 16 + offset (include/pa.h)
 *
 * (the same arrays pa_build_slot_mapping, pa_write_kv, pa_decode and
 * pa_varlen_prefill take, once copied to the device).
 *
 * Errors: NULL pointers, num_seqs < 0, an unknown sequence, q_lens[i] < 0 or
 * above its token count, a block table longer than max_blocks_per_seq, or
 * more new tokens than slot_capacity (PA_ERR_INVALID_ARGUMENT).
 */
int32_t pa_bm_build_step(const pa_block_manager* bm, const int64_t* seq_ids, const int32_t* q_lens,
                         int32_t num_seqs, int32_t max_blocks_per_seq, int32_t* block_tables,
                         int32_t* cu_seqlens, int32_t* context_offsets, int32_t* context_lens,
                         int64_t* slot_mapping, int64_t slot_capacity);

#ifdef __cplusplus
}
#endif

#endif  /* PA_BLOCKS_H_ */
