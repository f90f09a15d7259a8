"""The oracle's view of a seeded workload: host K/V pools built with the
oracle's own slot mapping and write from the generator's values (drawn on the
given device, copied to the host), and the oracle's expected outputs.  Nothing
here reads a result of the HIP path."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle
from conftest import host_bits
from workloads import PagedBatch

NAN_BITS = {"bf16": np.uint16(0x7FC0)}


@dataclass
class HostState:
    k_cache: np.ndarray
    v_cache: np.ndarray
    q: np.ndarray
    new_slots: np.ndarray
    fill_slots: np.ndarray


def _pool(batch: PagedBatch) -> np.ndarray:
    shape = (batch.num_blocks, batch.num_kv_heads, batch.block_size, batch.head_dim)
    if batch.dtype == "bf16":
        return np.full(shape, NAN_BITS["bf16"], np.uint16)
    return np.full(shape, np.nan, np.float32)


def host_state(batch: PagedBatch, device="cuda") -> HostState:
    kc, vc = _pool(batch), _pool(batch)
    fill_slots = np.zeros(0, np.int64)
    if batch.total_fill:
        k, v = batch.history_values(device)
        rows = batch.fill_rows()
        k, v = host_bits(k)[rows], host_bits(v)[rows]
        fill_slots = oracle.slot_mapping(batch.fill_tables(), batch.fill_cu, batch.fill_start)
        oracle.write_kv(kc, vc, k, v, fill_slots)
        del k, v
    kn, vn = batch.new_kv(device)
    new_slots = oracle.slot_mapping(batch.block_tables, batch.cu_seqlens, batch.context_offsets)
    oracle.write_kv(kc, vc, host_bits(kn), host_bits(vn), new_slots)
    return HostState(kc, vc, host_bits(batch.queries(device)), new_slots, fill_slots)


def expected(batch: PagedBatch, hs: HostState, seqs=None):
    """Decode: float64 [len(seqs), Hq, d].  Varlen: {seq: float64 [q_len, Hq, d]}."""
    if batch.kind == "decode":
        return oracle.decode(hs.q, hs.k_cache, hs.v_cache, batch.block_tables,
                             batch.context_lens, batch.scale, seqs=seqs)
    return oracle.varlen_prefill(hs.q, hs.k_cache, hs.v_cache, batch.cu_seqlens,
                                 batch.context_offsets, batch.block_tables, batch.scale, seqs=seqs)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    """Bitwise equality (NaN patterns included)."""
    if a.dtype == np.float32:
        a = a.view(np.uint32)
    if b.dtype == np.float32:
        b = b.view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)
