"""The seeded generators produce the configured shapes, deterministically."""
import numpy as np
import torch

import workloads as W


def test_tiny_decode_shape():
    b = W.tiny_decode()
    assert b.context_lens.tolist() == [1, 16, 17, 100]
    assert (b.num_q_heads, b.num_kv_heads, b.head_dim, b.dtype) == (4, 4, 64, "f32")
    assert b.num_blocks == 64 and b.max_blocks_per_seq == 7
    live = [b.block_tables[0, :1], b.block_tables[1, :1], b.block_tables[2, :2], b.block_tables[3, :7]]
    ids = np.concatenate(live)
    assert len(set(ids.tolist())) == 11 and ids.min() >= 0 and ids.max() < 64
    assert (b.block_tables >= 0).all() and (b.block_tables < 64).all()


def test_configs_ranges():
    b = W.llama2_decode()
    assert b.num_seqs == 64 and b.context_lens.min() >= 128 and b.context_lens.max() <= 384
    assert b.num_blocks == 4096
    b = W.gqa_decode()
    assert b.num_seqs == 256 and b.context_lens.min() >= 64 and b.context_lens.max() <= 4096
    b = W.mixed_step()
    assert b.total_q == 4096 and (b.q_lens[:-8] == 1).all() and (b.q_lens[-8:] >= 128).all()
    b = W.shared_prefix_decode()
    assert b.num_seqs == 128 and (b.block_tables[:, :64] == b.block_tables[0, :64]).all()
    assert b.context_lens.min() >= 1040 and b.context_lens.max() <= 32768


def test_tables_in_range_and_disjoint():
    for f in (W.llama2_decode, W.gqa_decode, W.mixed_step):
        b = f()
        assert (b.block_tables >= 0).all() and (b.block_tables < b.num_blocks).all()
        live = [b.block_tables[i, : -(-int(n) // 16)] for i, n in enumerate(b.context_lens)]
        ids = np.concatenate(live)
        assert len(np.unique(ids)) == len(ids)


def test_values_deterministic_and_rounded():
    b = W.tiny_decode()
    q1, q2 = b.queries(), b.queries()
    assert torch.equal(q1, q2) and q1.dtype == torch.float32
    k, v = b.history_values()
    assert k.shape == (b.num_values, 4, 64) and not torch.equal(k, v)
    b2 = W.decode_batch("t", 3, [5, 9], 2, 1, 64, "bf16")
    assert b2.queries().dtype == torch.bfloat16
    assert not torch.equal(b2.with_layer(1).queries(), b2.queries())


def test_unshared_prefix_same_values():
    a = W.shared_prefix_decode(n=4, suffix_range=(16, 100))
    u = W.shared_prefix_decode(n=4, suffix_range=(16, 100), unshared=True)
    assert a.num_values == u.num_values
    assert np.array_equal(a.context_lens, u.context_lens)
    rows_u = u.fill_rows()
    assert rows_u.max() < a.num_values and len(rows_u) == a.total_fill + 3 * 1024
