// pa_blocks.cpp -- host-side block manager of the paged KV cache.
//
// "vLLM изнутри: как устроен движок для быстрого инференса LLM": the KV-cache
// manager hands out blocks from a queue of free ones (engine-core paragraph);
// allocate_slots counts ceil(tokens / 16) blocks and refuses when the pool is
// short (allocate_slots paragraph); the runner builds the slot mapping and
// the attention metadata of the packed step (forward-pass paragraph).
// "vLLM：颠覆大模型推理的高效API服务引擎深度解析" §1.2 (block table: logical ->
// physical block, tokens per block), §1.3 (one shared pool, read-only sharing
// of common blocks), §2.1 (a finished request's blocks return at once).
//
// Plain C++17 on the host: a FIFO of free block ids, a reference count per
// block, and per sequence its block list and token count.  The FIFO is a ring
// sized to the pool when the manager is made, so taking and returning blocks
// never allocates; the calls that do allocate (a new sequence, a longer block
// list) do so before they change anything, and no C++ exception leaves the
// library: a failed host allocation returns PA_ERR_HOST_MEMORY with the
// manager as it was.

#include <cstdint>
#include <limits>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa_blocks.h"

struct pa_block_manager {
  struct Sequence {
    std::vector<int32_t> blocks;  // logical block i -> physical block
    int64_t tokens = 0;           // tokens stored (the last block may be partial)
  };
  int32_t block_size = PA_BLOCK_SIZE;
  // free-block FIFO: ring[(head + i) % capacity] for i < free_count
  std::vector<int32_t> ring;
  int64_t head = 0, free_count = 0;
  std::vector<int32_t> refcount;  // per physical block; 0 = in the free queue
  std::unordered_map<int64_t, Sequence> seqs;

  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }
  int64_t capacity() const { return static_cast<int64_t>(ring.size()); }
  int32_t pop_free() {
    const int32_t b = ring[static_cast<size_t>(head)];
    head = head + 1 == capacity() ? 0 : head + 1;
    --free_count;
    return b;
  }
  // a block whose count reached 0 (at most num_blocks are ever queued)
  void push_free(int32_t b) {
    int64_t tail = head + free_count;
    if (tail >= capacity()) tail -= capacity();
    ring[static_cast<size_t>(tail)] = b;
    ++free_count;
  }
};

namespace {

constexpr int64_t kMaxTokens = std::numeric_limits<int32_t>::max();

const pa_block_manager::Sequence* find(const pa_block_manager* bm, int64_t seq_id) {
  const auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? nullptr : &it->second;
}

}  // namespace

extern "C" {

int32_t pa_bm_create(int64_t num_blocks, int32_t block_size, pa_block_manager** out) {
  if (!out) return PA_ERR_NULL_POINTER;
  *out = nullptr;
  if (block_size != PA_BLOCK_SIZE) return PA_ERR_UNSUPPORTED;
  if (num_blocks < 1 || num_blocks > std::numeric_limits<int32_t>::max())
    return PA_ERR_INVALID_ARGUMENT;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return PA_ERR_HOST_MEMORY;
  try {
    bm->refcount.assign(static_cast<size_t>(num_blocks), 0);
    bm->ring.resize(static_cast<size_t>(num_blocks));
  } catch (...) {
    delete bm;
    return PA_ERR_HOST_MEMORY;
  }
  bm->block_size = block_size;
  for (int64_t b = 0; b < num_blocks; ++b) bm->ring[static_cast<size_t>(b)] = static_cast<int32_t>(b);
  bm->free_count = num_blocks;
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int64_t pa_bm_num_free_blocks(const pa_block_manager* bm) {
  return bm ? bm->free_count : -1;
}

int32_t pa_bm_allocate_slots(pa_block_manager* bm, int64_t seq_id, int32_t num_new_tokens,
                             int32_t num_lookahead_tokens) {
  if (!bm) return PA_ERR_NULL_POINTER;
  if (num_new_tokens < 0 || num_lookahead_tokens < 0) return PA_ERR_INVALID_ARGUMENT;
  const auto* existing = find(bm, seq_id);
  const int64_t tokens = existing ? existing->tokens : 0;
  const int64_t have = existing ? static_cast<int64_t>(existing->blocks.size()) : 0;
  const int64_t after = tokens + num_new_tokens;
  if (after + num_lookahead_tokens > kMaxTokens) return PA_ERR_INVALID_ARGUMENT;
  const int64_t need = bm->blocks_for(after + num_lookahead_tokens) - have;
  if (need > bm->free_count) return PA_ERR_NO_FREE_BLOCKS;
  pa_block_manager::Sequence* s = nullptr;
  try {
    s = &bm->seqs[seq_id];  // creates a new sequence
    if (need > 0) s->blocks.reserve(static_cast<size_t>(have + need));
  } catch (...) {
    if (!existing) bm->seqs.erase(seq_id);
    return PA_ERR_HOST_MEMORY;
  }
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = bm->pop_free();
    bm->refcount[b] = 1;
    s->blocks.push_back(b);  // within the reserved capacity
  }
  s->tokens = after;
  return PA_OK;
}

int32_t pa_bm_allocate_batch(pa_block_manager* bm, const int64_t* seq_ids,
                             const int32_t* num_new_tokens, int32_t num_seqs,
                             int32_t num_lookahead_tokens, int32_t* num_served) {
  if (!bm || !num_served) return PA_ERR_NULL_POINTER;
  *num_served = 0;
  if (num_seqs < 0) return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs > 0 && (!seq_ids || !num_new_tokens)) return PA_ERR_NULL_POINTER;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t st = pa_bm_allocate_slots(bm, seq_ids[i], num_new_tokens[i], num_lookahead_tokens);
    if (st != PA_OK) return st;
    *num_served = i + 1;
  }
  return PA_OK;
}

int32_t pa_bm_share_prefix(pa_block_manager* bm, int64_t src_seq, int64_t dst_seq,
                           int32_t num_tokens) {
  if (!bm) return PA_ERR_NULL_POINTER;
  const auto* src = find(bm, src_seq);
  if (!src || src_seq == dst_seq || find(bm, dst_seq) || num_tokens < 0 ||
      num_tokens > src->tokens)
    return PA_ERR_INVALID_ARGUMENT;
  const int64_t full = num_tokens / bm->block_size;  // whole blocks only
  pa_block_manager::Sequence* d = nullptr;
  try {
    std::vector<int32_t> shared(src->blocks.begin(), src->blocks.begin() + full);
    d = &bm->seqs[dst_seq];
    d->blocks = std::move(shared);
  } catch (...) {
    bm->seqs.erase(dst_seq);
    return PA_ERR_HOST_MEMORY;
  }
  for (const int32_t b : d->blocks) ++bm->refcount[b];
  d->tokens = full * bm->block_size;
  return PA_OK;
}

int32_t pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL_POINTER;
  const auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARGUMENT;
  for (const int32_t b : it->second.blocks)
    if (--bm->refcount[b] == 0) bm->push_free(b);
  bm->seqs.erase(it);
  return PA_OK;
}

int32_t pa_bm_sequence_info(const pa_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                            int32_t* num_blocks) {
  if (!bm) return PA_ERR_NULL_POINTER;
  const auto* s = find(bm, seq_id);
  if (!s) return PA_ERR_INVALID_ARGUMENT;
  if (num_tokens) *num_tokens = static_cast<int32_t>(s->tokens);
  if (num_blocks) *num_blocks = static_cast<int32_t>(s->blocks.size());
  return PA_OK;
}

int32_t pa_bm_block_refcount(const pa_block_manager* bm, int64_t block_id) {
  if (!bm || block_id < 0 || block_id >= static_cast<int64_t>(bm->refcount.size())) return -1;
  return bm->refcount[static_cast<size_t>(block_id)];
}

int32_t pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out,
                          int32_t capacity) {
  if (!bm || !out) return PA_ERR_NULL_POINTER;
  const auto* s = find(bm, seq_id);
  if (!s || capacity < static_cast<int64_t>(s->blocks.size())) return PA_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < capacity; ++i)
    out[i] = i < static_cast<int32_t>(s->blocks.size()) ? s->blocks[i] : -1;
  return PA_OK;
}

int32_t pa_bm_build_step(const pa_block_manager* bm, const int64_t* seq_ids, const int32_t* q_lens,
                         int32_t num_seqs, int32_t max_blocks_per_seq, int32_t* block_tables,
                         int32_t* cu_seqlens, int32_t* context_offsets, int32_t* context_lens,
                         int64_t* slot_mapping, int64_t slot_capacity) {
  if (!bm || !cu_seqlens) return PA_ERR_NULL_POINTER;
  if (num_seqs < 0 || max_blocks_per_seq < 1) return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs > 0 && (!seq_ids || !q_lens || !block_tables || !context_offsets ||
                       !context_lens || !slot_mapping))
    return PA_ERR_NULL_POINTER;
  // validate everything first: a failing call writes nothing
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto* s = find(bm, seq_ids[i]);
    if (!s || q_lens[i] < 0 || q_lens[i] > s->tokens ||
        static_cast<int64_t>(s->blocks.size()) > max_blocks_per_seq)
      return PA_ERR_INVALID_ARGUMENT;
    total += q_lens[i];
  }
  if (total > slot_capacity || total > kMaxTokens) return PA_ERR_INVALID_ARGUMENT;
  cu_seqlens[0] = 0;
  int64_t t = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto* s = find(bm, seq_ids[i]);
    int32_t* row = block_tables + static_cast<int64_t>(i) * max_blocks_per_seq;
    const int32_t nb = static_cast<int32_t>(s->blocks.size());
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < nb ? s->blocks[j] : -1;
    const int64_t before = s->tokens - q_lens[i];
    context_offsets[i] = static_cast<int32_t>(before);
    context_lens[i] = static_cast<int32_t>(s->tokens);
    for (int64_t p = before; p < s->tokens; ++p)
      slot_mapping[t++] = static_cast<int64_t>(s->blocks[p / bm->block_size]) * bm->block_size +
                          p % bm->block_size;
    cu_seqlens[i + 1] = static_cast<int32_t>(t);
  }
  return PA_OK;
}

}  // extern "C"
