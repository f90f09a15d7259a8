"""Seeded synthetic inputs for the paged-attention hot path.

This module only draws random numbers and lays them out in the shapes the
library's calls take: per-sequence lengths, physical block placements (block
tables), and query / key / value values.  It holds none of the method's
arithmetic -- no slot computation, no gather, no softmax -- so that the HIP
path and the CPU oracle can both consume its output without sharing any of the
code that is being checked.

The one piece of integer bookkeeping it does is allocation sizing: a sequence
that must hold n tokens is handed ``-(-n // block_size)`` physical blocks from
the pool, as a block manager would.  Which slot a token lands in is decided by
each side on its own (the library's slot-mapping call, the oracle's own
function).

Workloads follow the synthetic configurations the pages' serving scenario is
shaped like ("vLLM：颠覆大模型推理的高效API服务引擎深度解析", §三: LLaMA-2-7B,
128-token prompts and up to 256 generated tokens, power-law lengths):

  tiny_decode          4 seqs, lens {1,16,17,100}, 4/4 heads, d=64, fp32
  llama2_decode        64 seqs, lens U[128,384], 32/32 heads, d=128, bf16
  gqa_decode           256 seqs, Pareto(1.2) lens in [64,4096], 32/8 heads, bf16
  mixed_step           4096-token super-sequence: 8 prefill chunks + decode rows
  shared_prefix_decode 128 seqs sharing 64 prefix blocks + private suffixes

Every integer "uniform in [a, b]" is inclusive.  Values are N(0,1) drawn in
fp32 by a seeded torch generator on the requested device, then rounded to
nearest-even into bf16 where the workload is bf16; consumers see only the
rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Iterator, Optional

import numpy as np
import torch

BLOCK_SIZE = 16
FILL_CHUNK_TOKENS = 1 << 16  # history values are drawn in chunks of this many tokens

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _alloc_count(n_tokens: int, block_size: int) -> int:
    """Blocks a block manager hands out for n_tokens (allocation sizing only)."""
    return -(-int(n_tokens) // block_size)


@dataclass
class PagedBatch:
    """One attention call's inputs plus the history that fills the cache first.

    Step semantics: sequence i has ``q_len_i = cu_seqlens[i+1] - cu_seqlens[i]``
    new tokens at positions ``context_offsets[i] .. context_offsets[i]+q_len_i-1``;
    those new tokens' K/V are written (``new_kv``) and then attended to together
    with the ``context_offsets[i]`` tokens already in the cache (``history``).
    A decode batch has q_len_i = 1 for all i.

    History is described as fill segments: segment s writes ``fill_cu[s+1] -
    fill_cu[s]`` tokens into sequence ``fill_seq[s]`` starting at position
    ``fill_start[s]``, taking its values from rows ``fill_src[s] ...`` of the
    history value stream (a shared prefix is one segment written through one of
    the sharing sequences' tables; an unshared copy of it is one segment per
    sequence that reads the same value rows).
    """

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    block_tables: np.ndarray          # int32 [n, max_blocks_per_seq]
    cu_seqlens: np.ndarray            # int32 [n+1]
    context_offsets: np.ndarray       # int32 [n]
    fill_seq: np.ndarray              # int32 [S]
    fill_start: np.ndarray            # int32 [S]
    fill_cu: np.ndarray               # int32 [S+1]
    seed: int
    fill_src: Optional[np.ndarray] = None   # int32 [S]: first value row of segment s
    num_values: Optional[int] = None        # rows in the history value stream
    layer: int = 0
    block_size: int = BLOCK_SIZE
    kind: str = "decode"              # "decode" or "varlen"
    notes: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.fill_src is None:
            self.fill_src = self.fill_cu[:-1].astype(np.int32).copy()
        if self.num_values is None:
            self.num_values = int(self.fill_cu[-1])

    # ---- derived integer metadata (plain bookkeeping on the inputs) ----
    @property
    def num_seqs(self) -> int:
        return int(self.context_offsets.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens).astype(np.int32)

    @property
    def context_lens(self) -> np.ndarray:
        """Tokens each sequence attends to in this step (history + new)."""
        return (self.context_offsets + self.q_lens).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def total_fill(self) -> int:
        return int(self.fill_cu[-1])

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_layer(self, layer: int) -> "PagedBatch":
        """Same metadata (as every layer of a model shares its block tables),
        values drawn from another stream: one more layer's cache."""
        return replace(self, layer=layer)

    # ---- values ----
    def _gen(self, device, stream: int) -> torch.Generator:
        g = torch.Generator(device=device)
        g.manual_seed(self.seed * 1_000_003 + self.layer * 7919 + stream)
        return g

    def _draw(self, shape, device, stream) -> torch.Tensor:
        x = torch.randn(shape, generator=self._gen(device, stream), device=device,
                        dtype=torch.float32)
        return x.to(self.torch_dtype)

    def queries(self, device="cpu") -> torch.Tensor:
        """q [total_q, Hq, d]."""
        return self._draw((self.total_q, self.num_q_heads, self.head_dim), device, 1)

    def new_kv(self, device="cpu"):
        """K and V of the step's new tokens, [total_q, Hkv, d] each."""
        shape = (self.total_q, self.num_kv_heads, self.head_dim)
        return self._draw(shape, device, 2), self._draw(shape, device, 3)

    def history_values(self, device="cpu"):
        """The history value stream: K and V [num_values, Hkv, d], drawn in
        fixed chunks of FILL_CHUNK_TOKENS rows (chunk c from its own stream)."""
        shape_tail = (self.num_kv_heads, self.head_dim)
        ks, vs = [], []
        for ci, t0 in enumerate(range(0, self.num_values, FILL_CHUNK_TOKENS)):
            n = min(self.num_values, t0 + FILL_CHUNK_TOKENS) - t0
            ks.append(self._draw((n,) + shape_tail, device, 100 + 2 * ci))
            vs.append(self._draw((n,) + shape_tail, device, 101 + 2 * ci))
        if not ks:
            empty = torch.empty((0,) + shape_tail, dtype=self.torch_dtype, device=device)
            return empty, empty.clone()
        return torch.cat(ks), torch.cat(vs)

    def fill_rows(self) -> np.ndarray:
        """int64 [total_fill]: value-stream row of each packed fill token."""
        parts = [np.arange(s, s + (e - b), dtype=np.int64)
                 for s, b, e in zip(self.fill_src, self.fill_cu[:-1], self.fill_cu[1:])]
        return np.concatenate(parts) if parts else np.zeros(0, np.int64)

    def fill_is_identity(self) -> bool:
        return bool(np.array_equal(self.fill_src, self.fill_cu[:-1])
                    and self.num_values == self.total_fill)

    def canary_pools(self, device="cpu"):
        """k_cache, v_cache [num_blocks, Hkv, block_size, d] filled with NaN."""
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        k = torch.full(shape, float("nan"), dtype=self.torch_dtype, device=device)
        v = torch.full(shape, float("nan"), dtype=self.torch_dtype, device=device)
        return k, v

    def fill_tables(self) -> np.ndarray:
        """Block-table rows of the fill segments (row s = table of fill_seq[s])."""
        return np.ascontiguousarray(self.block_tables[self.fill_seq])

    # ---- sizes for reporting ----
    def unique_kv_blocks(self) -> int:
        """Distinct (physical block) ids the step's attention reads."""
        ids = set()
        for i, ctx in enumerate(self.context_lens):
            ids.update(self.block_tables[i, : _alloc_count(ctx, self.block_size)].tolist())
        return len(ids)


# --------------------------------------------------------------------------
# placement helpers
# --------------------------------------------------------------------------

def _place(rng: np.random.Generator, need: list[int], pool: int, maxb: int,
           shared: Optional[np.ndarray] = None) -> np.ndarray:
    """Hand each sequence need[i] distinct random blocks from a pool.

    Entries past a sequence's need are padded with other in-range block ids
    (an allocated-but-unused tail, as in the pages' block-table example), so a
    reader that strays past the live entries reads canary data, never out of
    bounds.  With ``shared`` (ids already taken), every sequence's table starts
    with those ids.
    """
    taken = 0 if shared is None else len(shared)
    perm = rng.permutation(pool).astype(np.int32)
    if shared is not None:
        perm = np.concatenate([shared, perm[~np.isin(perm, shared)]])
    total = taken + sum(need)
    assert total <= pool, (total, pool)
    spare = perm[total:] if total < pool else perm[:1]
    bt = np.empty((len(need), maxb), dtype=np.int32)
    cur = taken
    for i, nb in enumerate(need):
        row = list(perm[:taken]) + list(perm[cur:cur + nb])
        cur += nb
        pad = maxb - len(row)
        if pad:
            row += list(rng.choice(spare, size=pad, replace=True))
        bt[i] = np.asarray(row, dtype=np.int32)
    return bt


def _segments_plain(context_offsets: np.ndarray):
    """One history segment per sequence covering positions [0, c_i)."""
    n = len(context_offsets)
    seq = np.arange(n, dtype=np.int32)
    start = np.zeros(n, dtype=np.int32)
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(context_offsets)
    keep = context_offsets > 0
    seq, start = seq[keep], start[keep]
    cu = np.concatenate([[0], np.cumsum(context_offsets[keep])]).astype(np.int32)
    return seq, start, cu


def decode_batch(name: str, seed: int, ctx_lens, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, dtype: str, pool: Optional[int] = None,
                 pool_factor: float = 1.1, maxb: Optional[int] = None,
                 perm_rng_seed: Optional[int] = None) -> PagedBatch:
    """A decode step: each sequence appends one token and attends to ctx_len keys."""
    rng = np.random.default_rng(seed if perm_rng_seed is None else perm_rng_seed)
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    assert (ctx >= 1).all(), "a decode row attends at least its own new token"
    need = [_alloc_count(c, BLOCK_SIZE) for c in ctx]
    if pool is None:
        pool = max(1, int(np.ceil(sum(need) * pool_factor)))
    if maxb is None:
        maxb = max(1, max(need) if len(need) else 1)
    bt = _place(rng, need, pool, maxb)
    n = len(ctx)
    cu = np.arange(n + 1, dtype=np.int32)
    c_off = (ctx - 1).astype(np.int32)
    fseq, fstart, fcu = _segments_plain(c_off)
    return PagedBatch(name=name, dtype=dtype, num_q_heads=num_q_heads,
                      num_kv_heads=num_kv_heads, head_dim=head_dim, num_blocks=pool,
                      block_tables=bt, cu_seqlens=cu, context_offsets=c_off,
                      fill_seq=fseq, fill_start=fstart, fill_cu=fcu, seed=seed,
                      kind="decode", notes={"ctx_lens": ctx})


def varlen_batch(name: str, seed: int, q_lens, ctx_offsets, num_q_heads: int,
                 num_kv_heads: int, head_dim: int, dtype: str,
                 pool_factor: float = 1.1) -> PagedBatch:
    """A packed super-sequence: sequence i brings q_lens[i] new tokens after
    ctx_offsets[i] cached ones."""
    rng = np.random.default_rng(seed)
    ql = np.asarray(q_lens, dtype=np.int32)
    c_off = np.asarray(ctx_offsets, dtype=np.int32)
    need = [_alloc_count(c + l, BLOCK_SIZE) for c, l in zip(c_off, ql)]
    pool = max(1, int(np.ceil(sum(need) * pool_factor)))
    maxb = max(1, max(need) if len(need) else 1)
    bt = _place(rng, need, pool, maxb)
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    fseq, fstart, fcu = _segments_plain(c_off)
    return PagedBatch(name=name, dtype=dtype, num_q_heads=num_q_heads,
                      num_kv_heads=num_kv_heads, head_dim=head_dim, num_blocks=pool,
                      block_tables=bt, cu_seqlens=cu, context_offsets=c_off,
                      fill_seq=fseq, fill_start=fstart, fill_cu=fcu, seed=seed,
                      kind="varlen")


# --------------------------------------------------------------------------
# the five configurations
# --------------------------------------------------------------------------

def tiny_decode(seed: int = 1) -> PagedBatch:
    """4 sequences, lens {1,16,17,100}, 4 q = 4 kv heads, d=64, fp32; a pool of 64
    blocks whose order is a seeded permutation (sequences take consecutive
    slices of it)."""
    return decode_batch("tiny_decode_fp32", seed, [1, 16, 17, 100], 4, 4, 64, "f32",
                        pool=64, maxb=7)


def llama2_decode(seed: int = 2) -> PagedBatch:
    """LLaMA-2-7B-shaped decode: 64 seqs, ctx U[128,384], 32/32 heads, d=128,
    bf16, blocks drawn at random from a 4096-block pool."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(128, 384 + 1, size=64)
    return decode_batch("llama2_7b_decode_bf16", seed, ctx, 32, 32, 128, "bf16",
                        pool=4096, perm_rng_seed=seed + 10_000)


def gqa_decode(seed: int = 3) -> PagedBatch:
    """GQA decode: 256 seqs, 32 q / 8 kv heads, d=128, bf16, context lengths
    Pareto-I (alpha 1.2, x_m = 64) clipped to [64, 4096], pool = need x 1.1."""
    rng = np.random.default_rng(seed)
    ctx = np.clip(np.floor(64.0 * (1.0 + rng.pareto(1.2, size=256))), 64, 4096).astype(np.int64)
    return decode_batch("gqa_decode_bf16", seed, ctx, 32, 8, 128, "bf16",
                        pool_factor=1.1, perm_rng_seed=seed + 10_000)


def mixed_step(seed: int = 4, budget: int = 4096, n_prefill: int = 8) -> PagedBatch:
    """One super-sequence of ``budget`` tokens: single-token decode rows (context
    U[256,2048]) first, as a scheduler serves running requests before waiting
    ones, then ``n_prefill`` prefill chunks (length U[128,512], each after
    U[0,1024] cached tokens).  32 q / 8 kv heads, d=128, bf16."""
    rng = np.random.default_rng(seed)
    chunk_len = rng.integers(128, 512 + 1, size=n_prefill)
    chunk_ctx = rng.integers(0, 1024 + 1, size=n_prefill)
    n_dec = budget - int(chunk_len.sum())
    dec_ctx = rng.integers(256, 2048 + 1, size=n_dec)
    q_lens = np.concatenate([np.ones(n_dec, np.int32), chunk_len]).astype(np.int32)
    c_off = np.concatenate([dec_ctx - 1, chunk_ctx]).astype(np.int32)
    b = varlen_batch("mixed_step_bf16", seed, q_lens, c_off, 32, 8, 128, "bf16")
    b.notes.update({"n_decode_rows": n_dec, "n_prefill": n_prefill})
    return b


def prefill_only(seed: int = 4, n_prefill: int = 8) -> PagedBatch:
    """The prefill chunks of ``mixed_step`` alone (same draws), for a clean
    matrix-core measurement of the prefill part."""
    rng = np.random.default_rng(seed)
    chunk_len = rng.integers(128, 512 + 1, size=n_prefill)
    chunk_ctx = rng.integers(0, 1024 + 1, size=n_prefill)
    return varlen_batch("prefill_chunks_bf16", seed, chunk_len, chunk_ctx, 32, 8, 128, "bf16")


def prefill_long(seed: int = 7, n: int = 4, chunk: int = 2048, cached: int = 2048) -> PagedBatch:
    """Long prefill chunks: n sequences each bring `chunk` new tokens after
    `cached` cached ones (32 q / 8 kv heads, d=128, bf16) -- items of up to 64
    key tiles, where start-up and the longest-first tail weigh little."""
    return varlen_batch("prefill_long_bf16", seed, [chunk] * n, [cached] * n, 32, 8, 128, "bf16")


def shared_prefix_decode(seed: int = 5, n: int = 128, prefix_blocks: int = 64,
                         suffix_range=(16, 31744), unshared: bool = False,
                         num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                         dtype: str = "bf16") -> PagedBatch:
    """n decode sequences whose tables all start with the same prefix_blocks
    physical blocks (a 1024-token shared prompt), then private suffixes of
    U[16, 31744] tokens; 32 q / 8 kv heads, d=128, bf16 (the defaults).

    With ``unshared=True`` the same token values are laid out with a private
    copy of the prefix per sequence (the comparison case: outputs must match).
    """
    rng = np.random.default_rng(seed)
    suffix = rng.integers(suffix_range[0], suffix_range[1] + 1, size=n)
    prefix_tokens = prefix_blocks * BLOCK_SIZE
    ctx = (prefix_tokens + suffix).astype(np.int32)
    priv_need = [_alloc_count(s, BLOCK_SIZE) for s in suffix]
    maxb = prefix_blocks + max(priv_need)
    prng = np.random.default_rng(seed + 10_000)
    if not unshared:
        pool = int(np.ceil((prefix_blocks + sum(priv_need)) * 1.1))
        shared = prng.permutation(pool)[:prefix_blocks].astype(np.int32)
        bt = _place(prng, priv_need, pool, maxb, shared=shared)
    else:
        need = [prefix_blocks + p for p in priv_need]
        pool = int(np.ceil(sum(need) * 1.1))
        bt = _place(prng, need, pool, maxb)
    c_off = (ctx - 1).astype(np.int32)
    cu = np.arange(n + 1, dtype=np.int32)
    # history: the shared prompt once (through sequence 0's table), then each
    # sequence's private tokens before its new one.  The value stream is the
    # same in both layouts: rows 0..prefix_tokens-1 hold the prompt, then the
    # private tokens of sequence 0, 1, ...; the unshared layout writes the
    # prompt rows into every sequence's own copy.
    priv_len = (c_off - prefix_tokens).astype(np.int64)
    priv_src = prefix_tokens + np.concatenate([[0], np.cumsum(priv_len)[:-1]])
    num_values = int(prefix_tokens + priv_len.sum())
    if not unshared:
        fseq = np.concatenate([[0], np.arange(n)]).astype(np.int32)
        fstart = np.concatenate([[0], np.full(n, prefix_tokens)]).astype(np.int32)
        flen = np.concatenate([[prefix_tokens], priv_len])
        fsrc = np.concatenate([[0], priv_src]).astype(np.int32)
    else:
        fseq = np.repeat(np.arange(n), 2).astype(np.int32)
        fstart = np.tile([0, prefix_tokens], n).astype(np.int32)
        flen = np.stack([np.full(n, prefix_tokens), priv_len], axis=1).reshape(-1)
        fsrc = np.stack([np.zeros(n, np.int64), priv_src], axis=1).reshape(-1).astype(np.int32)
    fcu = np.concatenate([[0], np.cumsum(flen)]).astype(np.int32)
    shape = "" if (num_q_heads, num_kv_heads, head_dim) == (32, 8, 128) else \
        f"_{num_q_heads}_{num_kv_heads}_{head_dim}"
    b = PagedBatch(name=f"shared_prefix_decode_{dtype}{shape}" + ("_unshared" if unshared else ""),
                   dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                   head_dim=head_dim,
                   num_blocks=pool, block_tables=bt, cu_seqlens=cu, context_offsets=c_off,
                   fill_seq=fseq, fill_start=fstart, fill_cu=fcu, seed=seed, kind="decode",
                   fill_src=fsrc, num_values=num_values,
                   notes={"prefix_tokens": prefix_tokens, "unshared": unshared})
    return b


def long_prefix_decode(seed: int = 6, n: int = 128) -> PagedBatch:
    """A long common prompt and short private parts: n = 128 decode sequences
    whose tables start with the same 256 blocks (4096 tokens), then private
    suffixes of U[16, 1024] tokens; 32 q / 8 kv heads, d=128, bf16.  The case
    a common-prefix split is for: the prefix is ~85% of every context."""
    b = shared_prefix_decode(seed=seed, n=n, prefix_blocks=256, suffix_range=(16, 1024))
    b.name = "long_prefix_decode_bf16"
    return b


CONFIGS = {
    "tiny_decode": tiny_decode,
    "llama2_decode": llama2_decode,
    "gqa_decode": gqa_decode,
    "mixed_step": mixed_step,
    "shared_prefix_decode": shared_prefix_decode,
}
