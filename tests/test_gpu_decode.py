"""GPU parity of slot mapping, KV write and paged decode against the oracle.

Bars: slot mapping and cache contents bit-exact (NaN canaries in every slot
nobody wrote must survive); attention max-abs error <= 1e-5 for fp32 and
<= 2e-2 for bf16 (fp32 accumulation) against the float64 oracle; placement,
sharing and repeat runs bit-identical on the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from conftest import host_bits
from oracle_side import bits_equal, expected, host_state

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _device_batch(batch):
    from device_batch import DeviceBatch
    return DeviceBatch(batch)


def _max_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all()
    return float(np.abs(g - want).max()) if want.size else 0.0


def _check_decode(batch, seqs=None, check_pools=True):
    say(batch.name, "n", batch.num_seqs, "maxctx", batch.max_context_len, batch.dtype,
        "d", batch.head_dim, "g", batch.num_q_heads // batch.num_kv_heads)
    db = _device_batch(batch)
    out = db.step()
    torch.cuda.synchronize()
    hs = host_state(batch)
    assert np.array_equal(db.slots.cpu().numpy(), hs.new_slots), "slot mapping differs"
    if check_pools:
        assert bits_equal(host_bits(db.k_cache), hs.k_cache), "k_cache differs"
        assert bits_equal(host_bits(db.v_cache), hs.v_cache), "v_cache differs"
    want = expected(batch, hs, seqs)
    got = out if seqs is None else out[torch.as_tensor(list(seqs), device=out.device)]
    err = _max_err(got, want)
    say("max abs err", err)
    assert err <= TOL[batch.dtype], err
    return db, out


def test_tiny_decode_fp32(gpu):
    _check_decode(W.tiny_decode())


@pytest.mark.parametrize("dtype,d,hq,hkv", [
    ("f32", 64, 4, 4), ("f32", 128, 8, 2), ("bf16", 128, 8, 8), ("bf16", 128, 16, 4),
    ("bf16", 64, 8, 4), ("bf16", 128, 16, 2), ("bf16", 128, 32, 4), ("f32", 64, 16, 2),
])
def test_decode_ragged_multi_partition(gpu, dtype, d, hq, hkv):
    # exact fill, one over, partial blocks, partition edges (512) and several partitions
    lens = [1, 2, 15, 16, 17, 100, 511, 512, 513, 1024, 1100, 2049]
    batch = W.decode_batch(f"ragged_{dtype}_{d}_{hq}_{hkv}", 7, lens, hq, hkv, d, dtype,
                           pool_factor=1.3)
    _check_decode(batch)


def test_decode_zero_context(gpu):
    """A sequence with context 0 gets a zero row; the others are unaffected."""
    batch = W.decode_batch("zero_ctx", 8, [1, 5, 1, 600], 8, 2, 128, "bf16", pool_factor=1.5)
    db = _device_batch(batch)
    base = db.step().clone()
    db.context_lens[0] = 0
    db.context_lens[2] = 0
    db.out.fill_(7.0)
    out = db.attend()
    torch.cuda.synchronize()
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert torch.equal(out[1], base[1]) and torch.equal(out[3], base[3])


def test_decode_garbage_tail_entries_and_bad_ids(gpu):
    """Table entries past ceil(ctx/16) are never read: poisoning them (even with
    out-of-range ids) changes nothing."""
    batch = W.decode_batch("tail", 9, [5, 16, 33, 700], 8, 2, 128, "bf16", pool_factor=1.5)
    db = _device_batch(batch)
    base = db.step().clone()
    bt = db.block_tables.clone()
    for i, n in enumerate(batch.context_lens):
        live = -(-int(n) // 16)
        bt[i, live:] = -7 if i % 2 else 10 ** 6
    db.block_tables.copy_(bt)
    again = db.attend().clone()
    torch.cuda.synchronize()
    assert torch.equal(base, again)


def test_decode_placement_invariance(gpu):
    lens = [3, 40, 333, 900, 1500]
    a = W.decode_batch("place_a", 10, lens, 16, 4, 128, "bf16", pool_factor=2.0, perm_rng_seed=1)
    b = W.decode_batch("place_b", 10, lens, 16, 4, 128, "bf16", pool_factor=2.0, perm_rng_seed=2)
    assert not np.array_equal(a.block_tables, b.block_tables)
    oa = _device_batch(a).step().clone()
    ob = _device_batch(b).step().clone()
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)


def test_decode_deterministic(gpu):
    batch = W.decode_batch("repeat", 11, [700, 1300, 64, 2000], 32, 8, 128, "bf16")
    db = _device_batch(batch)
    o1 = db.step().clone()
    o2 = db.attend().clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_shared_prefix_small_equals_unshared(gpu):
    kw = dict(n=6, suffix_range=(16, 1500))
    shared = W.shared_prefix_decode(**kw)
    unshared = W.shared_prefix_decode(unshared=True, **kw)
    db_s, out_s = _check_decode(shared)
    out_u = _device_batch(unshared).step()
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_u)


def test_varlen_decode_rows_equal_decode(gpu):
    """All-single-token rows through the packed call take the decode kernels:
    identical output to pa_decode."""
    import paged_kv_cache_token_amd as pa
    lens = [1, 17, 600, 1200, 64]
    batch = W.decode_batch("rows", 12, lens, 32, 8, 128, "bf16", pool_factor=1.2)
    db = _device_batch(batch)
    dec = db.step().clone()
    vl = pa.varlen_prefill(db.q, db.k_cache, db.v_cache, db.cu_seqlens, db.context_offsets,
                           db.block_tables, 1, batch.max_context_len, batch.scale)
    torch.cuda.synchronize()
    assert torch.equal(dec, vl)


# ---- the full-size configurations --------------------------------------------

def test_llama2_decode_full(gpu):
    _check_decode(W.llama2_decode())


def test_gqa_decode_full(gpu):
    """GQA decode (256 sequences, Pareto lengths up to 4096): every row
    against the oracle, pools bit-exact."""
    _check_decode(W.gqa_decode())


def test_many_pairs_single_partition(gpu):
    """>= 4096 (sequence, kv head) pairs with contexts past one 512-token
    partition: the launch keeps each context in one partition.  Every row
    against the oracle."""
    rng = np.random.default_rng(28)
    lens = rng.integers(16, 1500, size=520)
    batch = W.decode_batch("many_pairs", 28, lens, 32, 8, 128, "bf16")
    _check_decode(batch, check_pools=False)


def test_shared_prefix_full_and_unshared(gpu):
    """Shared-prefix decode (128 sequences whose tables share 64 blocks,
    contexts up to 32768): every row against the oracle, and bit-identical
    to the same tokens laid out with a private copy of the prefix each."""
    shared = W.shared_prefix_decode()
    _, out_s = _check_decode(shared, check_pools=False)
    out_s = out_s.clone()
    torch.cuda.empty_cache()
    out_u = _device_batch(W.shared_prefix_decode(unshared=True)).step()
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_u)


# ---- the fused decode step ----------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ragged_f32_128", "ragged_bf16_g4", "llama2", "gqa"])
def test_fused_step_equals_separate_calls(gpu, name):
    """pa_decode_step (one launch) = slot mapping + pa_write_kv + pa_decode:
    bit-identical output and bit-identical pools afterwards."""
    lens = [1, 2, 15, 16, 17, 100, 511, 512, 513, 1100, 2049]
    batch = {
        "tiny": W.tiny_decode,
        "ragged_f32_128": lambda: W.decode_batch("r1", 31, lens, 8, 2, 128, "f32", pool_factor=1.3),
        "ragged_bf16_g4": lambda: W.decode_batch("r2", 32, lens, 32, 8, 128, "bf16", pool_factor=1.3),
        "llama2": W.llama2_decode,
        "gqa": W.gqa_decode,
    }[name]()
    say("fused vs separate", batch.name)
    a, b = _device_batch(batch), _device_batch(batch)
    oa = a.step().clone()
    ob = b.fused_step().clone()
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    assert bits_equal(host_bits(a.k_cache), host_bits(b.k_cache))
    assert bits_equal(host_bits(a.v_cache), host_bits(b.v_cache))


@pytest.mark.parametrize("max_ctx", [600, 1000])
def test_fused_step_understated_max_context(gpu, max_ctx):
    """With max_context_len below some contexts, the fused step still stores
    each new token at position context_lens[i] - 1 (never over an older
    token), and attends what pa_decode attends under the same clamp: pools
    and output bit-identical to slot mapping + pa_write_kv + pa_decode."""
    lens = [1, 17, 300, 599, 600, 601, 700, 1100, 1500]
    batch = W.decode_batch("fused_clamp", 34, lens, 16, 4, 128, "bf16", pool_factor=1.3)
    say("fused step, max_context_len", max_ctx, "of", batch.max_context_len)
    import paged_kv_cache_token_amd as pa
    a, b = _device_batch(batch), _device_batch(batch)
    a.write_new()
    oa = pa.decode(a.q, a.k_cache, a.v_cache, a.block_tables, a.context_lens, max_ctx,
                   batch.scale).clone()
    ob = pa.decode_step(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_tables,
                        b.context_lens, max_ctx, batch.scale).clone()
    torch.cuda.synchronize()
    hs = host_state(batch)
    assert bits_equal(host_bits(a.k_cache), hs.k_cache)
    assert bits_equal(host_bits(b.k_cache), hs.k_cache), "fused store went to another slot"
    assert bits_equal(host_bits(b.v_cache), hs.v_cache), "fused store went to another slot"
    assert torch.equal(oa, ob)


def test_fused_step_against_oracle(gpu):
    batch = W.decode_batch("fused_oracle", 33, [1, 16, 17, 700, 1500], 16, 4, 128, "bf16",
                           pool_factor=1.3)
    db = _device_batch(batch)
    out = db.fused_step()
    torch.cuda.synchronize()
    hs = host_state(batch)
    assert bits_equal(host_bits(db.k_cache), hs.k_cache)
    assert bits_equal(host_bits(db.v_cache), hs.v_cache)
    err = _max_err(out, expected(batch, hs))
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("bad_id", [-3, 10 ** 6])
def test_decode_out_of_pool_block_takes_no_part(gpu, bad_id):
    """A live table entry outside [0, num_blocks) is an empty block: its 16
    tokens drop out of the softmax.  Expected: the oracle's attention over
    the sequence's other tokens."""
    import oracle
    lens = [40, 700, 1500]
    batch = W.decode_batch("bad_block_dec", 27, lens, 32, 8, 128, "bf16")
    db = _device_batch(batch)
    db.step()
    hs = host_state(batch)
    drop = {0: 1, 1: 20, 2: 50}   # logical block dropped per sequence
    bt = db.block_tables.clone()
    for i, j in drop.items():
        bt[i, j] = bad_id
    db.block_tables.copy_(bt)
    got = db.attend().clone()
    torch.cuda.synchronize()
    want = np.zeros((len(lens), batch.num_q_heads, batch.head_dim))
    for i, j in drop.items():
        n = int(batch.context_lens[i])
        keep = np.r_[0:16 * j, 16 * (j + 1):n]
        k = oracle.widen(oracle.gather(hs.k_cache, batch.block_tables[i], n))[keep]
        v = oracle.widen(oracle.gather(hs.v_cache, batch.block_tables[i], n))[keep]
        want[i] = oracle.attend(oracle.widen(hs.q[i:i + 1]), k, v, np.array([n - 16]),
                                batch.scale)[0]
    err = _max_err(got, want)
    say("max abs err", err)
    assert err <= TOL["bf16"], err


# ---- work list derived in every workgroup vs the plan kernel ------------------

@pytest.mark.parametrize("name", ["gqa", "ragged_g8", "varlen_mixed", "varlen_rows_f32"])
def test_inline_plan_equals_plan_kernel(gpu, monkeypatch, name):
    """The list kernel's own work list (the default) and the plan kernel's
    list name the same (sequence, partition) items: bit-identical outputs."""
    lens = [1, 2, 15, 16, 17, 100, 511, 512, 513, 1024, 1100, 2049, 0]
    batch = {
        "gqa": W.gqa_decode,
        "ragged_g8": lambda: W.decode_batch("il_g8", 33, lens[:-1], 16, 2, 128, "bf16",
                                            pool_factor=1.3),
        "varlen_mixed": lambda: W.varlen_batch("il_vm", 34, [1, 1, 300, 1, 64, 1],
                                               [700, 1500, 200, 20, 900, 2500], 32, 8, 128,
                                               "bf16"),
        "varlen_rows_f32": lambda: W.varlen_batch("il_vf", 35, [1, 40, 1, 3],
                                                  [600, 100, 1300, 517], 8, 2, 64, "f32"),
    }[name]()
    say("inline plan vs plan kernel", batch.name)
    db = _device_batch(batch)
    db.write_new()
    monkeypatch.setenv("PA_DECODE_INLINE_PLAN", "0")
    a = db.attend().clone()
    monkeypatch.setenv("PA_DECODE_INLINE_PLAN", "1")
    b = db.attend().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    if name in ("ragged_g8", "varlen_mixed"):
        hs = host_state(batch)
        want = expected(batch, hs)
        if batch.kind == "decode":
            err = _max_err(b, want)
        else:
            cu = batch.cu_seqlens
            err = max(_max_err(b[int(cu[i]):int(cu[i + 1])], want[i]) for i in want)
        say("max abs err", err)
        assert err <= TOL[batch.dtype], err


# ---- launch-shape variants ----------------------------------------------------

@pytest.mark.parametrize("env", [
    {"PA_DECODE_WAVES": "1"}, {"PA_DECODE_WAVES": "2"}, {"PA_DECODE_WAVES": "4"},
    {"PA_DECODE_BUFFERS": "1"}, {"PA_DECODE_BUFFERS": "3"}, {"PA_DECODE_BUFFERS": "4"},
    {"PA_DECODE_PARTITION": "256"}, {"PA_DECODE_PARTITION": "1024"},
    {"PA_DECODE_GRID": "1"}, {"PA_DECODE_OVERSUB": "1"},
    {"PA_DECODE_WAVES": "1", "PA_DECODE_PARTITION": "1024"},
    {"PA_DECODE_MFMA": "0"}, {"PA_DECODE_MFMA": "0", "PA_DECODE_BUFFERS": "1"},
    {"PA_DECODE_MFMA": "0", "PA_DECODE_GRID": "1"},
], ids=lambda e: ",".join(f"{k[10:].lower()}={v}" for k, v in e.items()))
def test_decode_launch_variants(gpu, monkeypatch, env):
    """Every launch shape the library can pick (waves per workgroup, register
    buffers, partition length, grid or list, matrix-core or vector item code)
    gives oracle parity."""
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    lens = [1, 2, 15, 16, 17, 100, 511, 512, 513, 1024, 1100, 2049]
    for dtype, d, hq, hkv in (("bf16", 128, 32, 8), ("f32", 64, 8, 8)):
        batch = W.decode_batch(f"variant_{dtype}", 36, lens, hq, hkv, d, dtype, pool_factor=1.3)
        _check_decode(batch, check_pools=False)


@pytest.mark.parametrize("n,max_len", [(1100, 256), (600, 500)])
def test_decode_many_short_contexts(gpu, n, max_len):
    """Batches of many short contexts run one or two waves per item (no
    cross-wave merge for one): every row against the oracle."""
    rng = np.random.default_rng(37 + n)
    lens = rng.integers(1, max_len + 1, size=n)
    lens[0] = max_len
    batch = W.decode_batch(f"short_{n}", 37, lens, 32, 8, 128, "bf16", pool_factor=1.2)
    _check_decode(batch, check_pools=False)


@pytest.mark.parametrize("dtype,d,hq,hkv,n", [("bf16", 128, 32, 8, 160), ("f32", 64, 8, 8, 130)])
def test_decode_one_partition_up_to_1024(gpu, dtype, d, hq, hkv, n):
    """At least 1024 (sequence, kv head) pairs with contexts of at most 1024
    tokens run one partition per context on the streaming kernel (a context
    of 1024 tokens in one item, no merge): every row against the oracle."""
    rng = np.random.default_rng(39 + n)
    lens = rng.integers(1, 1025, size=n)
    lens[:6] = [1024, 1023, 513, 512, 511, 1]
    batch = W.decode_batch(f"one_part_{dtype}_{n}", 39, lens, hq, hkv, d, dtype, pool_factor=1.2)
    _check_decode(batch, check_pools=False)


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 32, 8), ("f32", 128, 8, 8)])
def test_decode_very_long_context(gpu, dtype, d, hq, hkv):
    """A 65536-token context next to short ones: 1024-token partitions (64 of
    them, more than one batch of the merge's loads) and the fused step's
    store at the far end of the table; every row against the oracle."""
    lens = [65536, 1, 700, 65535 - 16 * 7]
    batch = W.decode_batch(f"very_long_{dtype}", 40, lens, hq, hkv, d, dtype, pool_factor=1.05)
    _check_decode(batch, check_pools=False)


def test_decode_list_beyond_inline_plan(gpu):
    """More sequences than a workgroup derives its work list for (2048), with
    a context long enough to need partitions: the plan-kernel path."""
    rng = np.random.default_rng(38)
    lens = rng.integers(1, 65, size=2100)
    lens[7] = 5000
    batch = W.decode_batch("list_2100", 38, lens, 32, 8, 128, "bf16", pool_factor=1.2)
    _check_decode(batch, check_pools=False)


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8), (16, 4), (8, 8), (16, 8)])
def test_decode_matrix_core_and_vector_items(gpu, monkeypatch, hq, hkv):
    """bf16 at head_dim 128 runs the matrix-core item code (g = 1 to 8 here);
    the vector item code (PA_DECODE_MFMA=0) computes the same attention.  Both against the oracle, on ragged contexts with block,
    partition and single-partition edges, and the fused step's new token at
    every offset of its block."""
    lens = [1, 2, 3, 15, 16, 17, 31, 100, 255, 511, 512, 513, 1024, 1100, 2049, 4100]
    batch = W.decode_batch(f"items_{hq}_{hkv}", 41, lens, hq, hkv, 128, "bf16", pool_factor=1.3)
    for mf in ("1", "0"):
        monkeypatch.setenv("PA_DECODE_MFMA", mf)
        say("PA_DECODE_MFMA", mf)
        _check_decode(batch)
