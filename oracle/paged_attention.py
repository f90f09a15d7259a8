"""CPU oracle for paged attention.  TEST INFRASTRUCTURE -- not the library.

A plain, slow, obviously correct numpy implementation in float64 of what the
paged-attention hot path computes.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it.  It imports nothing from the
library (``paged_kv_cache_token_amd``) and the library never imports it; the
two share no code, headers, tables or helpers.

Sources, cited by page title and section:

  [VI]  "vLLM изнутри: как устроен движок для быстрого инференса LLM" --
        the allocate_slots paragraph (each KV block holds 16 tokens by default;
        17 new tokens need ceil(17/16) = 2 blocks) and the forward-pass
        paragraph (the model runner builds a slot mapping and attention
        metadata; all sequences are packed into one super-sequence whose masks
        and positions keep each sequence on its own tokens).
  [ZN]  "vLLMつかったら、ベクトル検索サーバーが高速化して安定性も向上した" --
        the walk through Scheduler.schedule() (its output carries the number
        of blocks common to every scheduled request).
  [KW]  "vLLM：颠覆大模型推理的高效API服务引擎深度解析" --
        §1.2 (fixed-size blocks; a per-request block table mapping logical to
        physical blocks with a fill count per block; the 16 / 8 / 0 example),
        §1.3 (one pre-allocated pool shared by all requests; new-token K/V are
        stored into a physical block; attention gathers the scattered blocks
        through the block table into a logically contiguous KV cache and then
        computes; physical blocks may be referenced read-only by several block
        tables).

The pages name attention but never print it.  The oracle takes the textbook
scaled dot-product form softmax(scale * q K^T) V, with grouped-query heads
mapped in contiguous groups (q head h reads kv head h // (Hq / Hkv)).

Conventions shared with the library by specification only (not by code):
  * cache layout [num_blocks, num_kv_heads, block_size, head_dim];
  * slot = physical_block * block_size + offset_in_block;
  * context_lens[i] counts the cached tokens including this step's new one.

Inputs are numpy arrays.  bf16 data is passed as its raw uint16 bit patterns
(numpy has no bf16); fp32 as float32.  Every function widens to float64
exactly before any arithmetic.

Every function here is pinned by tests that do not reuse its code (worked
values from the pages, closed forms, brute force on tiny inputs, a library
attention routine, invariants).
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16  # [VI] allocate_slots paragraph; [KW] §1.2 example block size


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def widen(a: np.ndarray) -> np.ndarray:
    """Exact conversion to float64: bf16 bit patterns (uint16) or fp32/fp64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported element type {a.dtype}")


# --------------------------------------------------------------------------
# block bookkeeping  ([VI] allocate_slots; [KW] §1.2)
# --------------------------------------------------------------------------

def blocks_needed(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Physical blocks that hold num_tokens tokens: ceil(num_tokens / block_size).

    [VI] allocate_slots paragraph: a prefill of 17 new tokens needs 2 blocks.
    """
    n = int(num_tokens)
    if n < 0:
        raise ValueError("negative token count")
    full, rest = divmod(n, block_size)
    return full + (1 if rest else 0)


def slot_mapping(block_tables: np.ndarray, cu_seqlens: np.ndarray,
                 context_offsets: np.ndarray, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Cache slot of every new token of a packed step.

    Sequence i brings tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 of the packed
    list; its j-th new token sits at logical position context_offsets[i] + j,
    i.e. in logical block position // block_size at offset position % block_size;
    the block table turns the logical block into a physical one ([KW] §1.2),
    and the slot is physical_block * block_size + offset.
    """
    bt = np.asarray(block_tables)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    c = np.asarray(context_offsets, dtype=np.int64)
    n = len(c)
    lens = cu[1:] - cu[:-1]
    seq = np.repeat(np.arange(n), lens)                    # owning sequence of each token
    j = np.arange(int(cu[-1])) - cu[:-1][seq]              # index inside its sequence
    pos = c[seq] + j                                       # logical position
    logical_block = pos // block_size
    offset = pos % block_size
    physical = bt[seq, logical_block].astype(np.int64)
    return physical * block_size + offset


def write_kv(k_cache: np.ndarray, v_cache: np.ndarray, key: np.ndarray,
             value: np.ndarray, slots: np.ndarray, block_size: int = BLOCK_SIZE) -> None:
    """Store each new token's K and V into its slot, in place ([KW] §1.3: the
    new token's KV vectors are stored into the allocated physical block).

    key / value are [num_tokens, Hkv, d]; the caches [num_blocks, Hkv,
    block_size, d] of the same element type.  A negative slot marks a padding
    token that is not stored.  This is a bit copy: no arithmetic touches the
    values.
    """
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    blk = slots[keep] // block_size
    off = slots[keep] % block_size
    k_cache[blk, :, off, :] = key[keep]
    v_cache[blk, :, off, :] = value[keep]


def swap_blocks(dst: np.ndarray, src: np.ndarray, block_pairs: np.ndarray) -> None:
    """Copy whole blocks between two pools of one layout, in place: for each
    (source block, destination block) pair, the destination block becomes a
    bit copy of the source block ([KW] §2.2: inactive blocks are moved out to
    host memory and back in when needed).  A pair naming a block outside its
    pool is skipped.  Pairs are taken one at a time, in order.
    """
    for s_blk, d_blk in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= s_blk < src.shape[0] and 0 <= d_blk < dst.shape[0]:
            dst[d_blk] = src[s_blk]


def gather(cache: np.ndarray, table_row: np.ndarray, length: int,
           block_size: int = BLOCK_SIZE) -> np.ndarray:
    """One sequence's logically contiguous cache [length, Hkv, d] ([KW] §1.3:
    the blocks scattered over the pool are gathered through the block table).

    Only the first ceil(length / block_size) table entries are live, and only
    the first ``length`` tokens of them; the rest (an allocated-but-empty tail
    block as in [KW] §1.2's example, stale slots) is never read.
    """
    nb = blocks_needed(length, block_size)
    if nb == 0:
        return np.zeros((0, cache.shape[1], cache.shape[3]), dtype=cache.dtype)
    tiles = [cache[int(b)] for b in table_row[:nb]]        # each [Hkv, block_size, d]
    seq = np.concatenate(tiles, axis=1)                     # [Hkv, nb*block_size, d]
    return np.ascontiguousarray(seq[:, :length, :].transpose(1, 0, 2))


# --------------------------------------------------------------------------
# attention over a contiguous K/V (textbook scaled dot-product attention)
# --------------------------------------------------------------------------

def attend(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray,
           scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for each query row and q head, in float64.

    q_rows [R, Hq, d]; k, v [Lk, Hkv, d] (already float64); row r sees keys
    0 .. visible[r]-1.  q head h reads kv head h // (Hq / Hkv).  A row that
    sees no key gets zeros.
    """
    r_count, hq, d = q_rows.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((r_count, hq, d), dtype=np.float64)
    for r in range(r_count):
        n = int(visible[r])
        if n == 0:
            continue
        for h in range(hq):
            kvh = h // group
            scores = scale * (k[:n, kvh, :] @ q_rows[r, h, :])   # [n]
            m = scores.max()
            p = np.exp(scores - m)
            out[r, h, :] = (p @ v[:n, kvh, :]) / p.sum()
    return out


# --------------------------------------------------------------------------
# the two attention calls
# --------------------------------------------------------------------------

def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
           seqs=None, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Decode: sequence i's single query row attends all context_lens[i] cached
    tokens (the new token's K/V already stored).  Returns float64
    [len(seqs), Hq, d] for the requested sequences (default: all)."""
    qf = widen(q)
    if seqs is None:
        seqs = range(qf.shape[0])
    seqs = list(seqs)
    out = np.zeros((len(seqs), qf.shape[1], qf.shape[2]), dtype=np.float64)
    for o, i in enumerate(seqs):
        n = int(context_lens[i])
        k = widen(gather(k_cache, block_tables[i], n, block_size))
        v = widen(gather(v_cache, block_tables[i], n, block_size))
        out[o] = attend(qf[i:i + 1], k, v, np.array([n]), scale)[0]
    return out


def cascade_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                   block_tables: np.ndarray, context_lens: np.ndarray,
                   num_common_prefix_blocks: int, scale: float, seqs=None,
                   block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Decode of sequences that share their first ``num_common_prefix_blocks``
    physical blocks (the scheduler's count of blocks common to every request,
    [ZN] Scheduler.schedule(); blocks referenced read-only by several block
    tables, [KW] §1.3).

    Attending the common prefix once for all sequences and each private rest
    on its own, then combining the two by their max-rescaled sums, is the same
    attention: the result is ``decode`` of the same inputs.  What the split
    adds is a precondition, checked here: every row's live entries inside the
    prefix (the first min(P, ceil(len/16)) of them) name the same blocks as
    row 0's, since the shared pass reads the prefix from row 0 alone.
    """
    p = int(num_common_prefix_blocks)
    if p < 0 or p > block_tables.shape[1]:
        raise ValueError("num_common_prefix_blocks outside the table")
    for i in range(len(context_lens)):
        live = min(p, blocks_needed(int(context_lens[i]), block_size))
        if not np.array_equal(block_tables[i, :live], block_tables[0, :live]):
            raise ValueError(f"row {i} does not share the first {live} prefix blocks of row 0")
    return decode(q, k_cache, v_cache, block_tables, context_lens, scale, seqs, block_size)


def varlen_prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                   cu_seqlens: np.ndarray, context_offsets: np.ndarray,
                   block_tables: np.ndarray, scale: float, seqs=None,
                   block_size: int = BLOCK_SIZE) -> dict:
    """Packed super-sequence attention ([VI] forward-pass paragraph): sequence
    i owns query rows cu_seqlens[i] .. cu_seqlens[i+1]-1; its j-th row sits at
    position context_offsets[i] + j and sees exactly its own sequence's keys
    0 .. context_offsets[i] + j (causal, own key included).  Returns
    {i: float64 [q_len_i, Hq, d]} for the requested sequences (default: all).
    """
    qf = widen(q)
    n_seq = len(context_offsets)
    if seqs is None:
        seqs = range(n_seq)
    res = {}
    for i in seqs:
        lo, hi = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        c = int(context_offsets[i])
        length = c + (hi - lo)
        k = widen(gather(k_cache, block_tables[i], length, block_size))
        v = widen(gather(v_cache, block_tables[i], length, block_size))
        visible = c + np.arange(hi - lo) + 1
        res[i] = attend(qf[lo:hi], k, v, visible, scale)
    return res
