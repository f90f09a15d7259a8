"""Device-side setup of a seeded workload through the library's own calls.

Given a ``workloads.PagedBatch``, allocate NaN-filled K/V pools on the GPU,
write the history tokens into them with ``build_slot_mapping`` + ``write_kv``,
and run the step: slot mapping and write of the step's new tokens, then
``decode`` (decode batches) or ``varlen_prefill`` (packed batches).

Used by the GPU tests, the smoke check and the benchmark.  It calls only the
library binding and torch allocation; no oracle code.
"""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_token_amd as pa
from workloads import PagedBatch


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceBatch:
    def __init__(self, batch: PagedBatch, device="cuda", fill: bool = True,
                 hint_rows: bool = True):
        self.b = batch
        self.device = torch.device(device)
        self.hint_rows = hint_rows
        self.num_decode_rows = int((batch.q_lens == 1).sum()) if batch.num_seqs else 0
        self.block_tables = _dev(batch.block_tables, device)
        self.cu_seqlens = _dev(batch.cu_seqlens, device)
        self.context_offsets = _dev(batch.context_offsets, device)
        self.context_lens = _dev(batch.context_lens, device)
        self.q = batch.queries(device)
        self.k_new, self.v_new = batch.new_kv(device)
        self.k_cache, self.v_cache = batch.canary_pools(device)
        self.out = torch.empty_like(self.q)
        self.slots = torch.empty(batch.total_q, dtype=torch.int64, device=device)
        if batch.kind == "decode":
            size = pa.decode_workspace_size(batch.num_seqs, batch.num_q_heads, batch.head_dim,
                                            batch.max_context_len, batch.torch_dtype)
        else:
            size = pa.varlen_workspace_size(batch.num_seqs, batch.total_q, batch.num_q_heads,
                                            batch.num_kv_heads, batch.head_dim,
                                            batch.max_context_len, batch.torch_dtype)
        self.workspace = torch.empty(max(size, 1), dtype=torch.uint8, device=device)
        if fill:
            self.fill_history()

    def fill_history(self) -> None:
        """Write every history token into the pools (pa slot mapping + write)."""
        b = self.b
        if b.total_fill == 0:
            return
        k, v = b.history_values(self.device)
        if not b.fill_is_identity():
            rows = _dev(b.fill_rows(), self.device)
            k, v = k.index_select(0, rows), v.index_select(0, rows)
        ftab = _dev(b.fill_tables(), self.device)
        fcu = _dev(b.fill_cu, self.device)
        fstart = _dev(b.fill_start, self.device)
        slots = pa.build_slot_mapping(fcu, fstart, ftab, b.total_fill)
        pa.write_kv(k, v, self.k_cache, self.v_cache, slots)
        del k, v, slots

    def write_new(self) -> None:
        b = self.b
        pa.build_slot_mapping(self.cu_seqlens, self.context_offsets, self.block_tables, b.total_q,
                              out=self.slots)
        pa.write_kv(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slots)

    def attend(self, out: torch.Tensor | None = None) -> torch.Tensor:
        b = self.b
        out = self.out if out is None else out
        if b.kind == "decode":
            return pa.decode(self.q, self.k_cache, self.v_cache, self.block_tables,
                             self.context_lens, b.max_context_len, b.scale, out=out,
                             workspace=self.workspace)
        # the host knows how many sequences are single-token rows (a step's
        # metadata is built there): a prefill-only step launches no decode kernels
        return pa.varlen_prefill(self.q, self.k_cache, self.v_cache, self.cu_seqlens,
                                 self.context_offsets, self.block_tables, b.max_q_len,
                                 b.max_context_len, b.scale, out=out, workspace=self.workspace,
                                 num_decode_rows=self.num_decode_rows if self.hint_rows else None)

    def step(self) -> torch.Tensor:
        """One pass of the hot path: slots + write of the new tokens, attention
        (three calls)."""
        self.write_new()
        return self.attend()

    def cascade(self, out: torch.Tensor | None = None,
                prefix_blocks: int | None = None) -> torch.Tensor:
        """Decode attention through pa_cascade_decode, the common prefix being
        the batch's shared prompt (or ``prefix_blocks`` blocks)."""
        b = self.b
        assert b.kind == "decode"
        if prefix_blocks is None:
            prefix_blocks = b.notes["prefix_tokens"] // b.block_size
        size = pa.cascade_workspace_size(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                         b.max_context_len, prefix_blocks, b.torch_dtype)
        if getattr(self, "cascade_ws", None) is None or self.cascade_ws.numel() < size:
            self.cascade_ws = torch.empty(max(size, 1), dtype=torch.uint8, device=self.device)
        out = self.out if out is None else out
        return pa.cascade_decode(self.q, self.k_cache, self.v_cache, self.block_tables,
                                 self.context_lens, b.max_context_len, prefix_blocks, b.scale,
                                 out=out, workspace=self.cascade_ws)

    def fused_step(self, out: torch.Tensor | None = None) -> torch.Tensor:
        """The same decode step in one launch (pa_decode_step)."""
        b = self.b
        assert b.kind == "decode"
        out = self.out if out is None else out
        return pa.decode_step(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache,
                              self.block_tables, self.context_lens, b.max_context_len, b.scale,
                              out=out, workspace=self.workspace)
