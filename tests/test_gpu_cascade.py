"""GPU parity of pa_cascade_decode (decode of sequences that share their first
blocks: the prefix on the matrix cores once per kv head, the private rest on
the decode kernels, partials combined) against the oracle.

Bars: max-abs error <= 2e-2 for bf16 and <= 1e-5 for fp32 against the float64
oracle.  The row tiles of the prefix pass hold 256/g sequences and its key
tiles 64 keys, so the cases take sequence counts and prefix lengths that
leave ragged row and key tiles, several key splits, contexts that end inside
the prefix, and partition edges of the private part.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle_side import host_state

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


def _check(batch, prefix_blocks=None, ctx=None, seqs=None):
    """Store the step's new tokens, run the cascade call (optionally with
    shortened contexts) and compare with the oracle."""
    p = batch.notes["prefix_tokens"] // 16 if prefix_blocks is None else prefix_blocks
    say(batch.name, "n", batch.num_seqs, "prefix blocks", p, "maxctx", batch.max_context_len,
        "g", batch.num_q_heads // batch.num_kv_heads)
    db = _device_batch(batch)
    db.write_new()
    lens = batch.context_lens.copy()
    if ctx is not None:
        for i, c in ctx.items():
            lens[i] = c
        db.context_lens.copy_(torch.from_numpy(lens))
    out = db.cascade(prefix_blocks=p).clone()
    torch.cuda.synchronize()
    hs = host_state(batch)
    want = oracle.cascade_decode(hs.q, hs.k_cache, hs.v_cache, batch.block_tables, lens, p,
                                 batch.scale, seqs=seqs)
    got = out if seqs is None else out[torch.as_tensor(list(seqs), device=out.device)]
    err = _max_err(got, want)
    say("max abs err", err)
    assert err <= TOL[batch.dtype], err
    return db, out


@pytest.mark.parametrize("n,hq,hkv,prefix_blocks,suffix", [
    (70, 32, 8, 5, (1, 700)),      # g=4: 64 sequences per row tile (one full, one of 6);
                                   # 80 prefix keys (a full key tile and one of 16)
    (300, 8, 8, 9, (1, 300)),      # g=1: 256 per row tile
    (40, 16, 2, 33, (1, 1200)),    # g=8: 32 per row tile; 528 prefix keys, several splits
    (130, 16, 8, 16, (16, 2100)),  # g=2: 128 per row tile; partition edges in the rest
])
def test_cascade_shapes(gpu, n, hq, hkv, prefix_blocks, suffix):
    batch = W.shared_prefix_decode(seed=40 + n, n=n, prefix_blocks=prefix_blocks,
                                   suffix_range=suffix, num_q_heads=hq, num_kv_heads=hkv)
    _check(batch)


def test_cascade_contexts_inside_prefix(gpu):
    """Sequences whose context ends inside the prefix (row 0's among them)
    attend only their first context_lens[i] keys; at the prefix's end exactly,
    the private part is empty."""
    batch = W.shared_prefix_decode(seed=51, n=20, prefix_blocks=12, suffix_range=(1, 400))
    p = 12 * 16
    _check(batch, ctx={0: 3, 1: 1, 2: 16, 3: 17, 4: p - 1, 5: p, 6: p + 1, 7: 64, 8: 65})


@pytest.mark.parametrize("split_tiles", ["1", "3", "1000"])
def test_cascade_key_splits(gpu, monkeypatch, split_tiles):
    """Any split of the prefix into key ranges gives the same attention: one
    tile per item, ragged splits, and the whole prefix in one item."""
    monkeypatch.setenv("PA_CASCADE_SPLIT_TILES", split_tiles)
    batch = W.shared_prefix_decode(seed=52, n=90, prefix_blocks=22, suffix_range=(1, 900))
    _check(batch)


def test_cascade_part_of_the_prefix(gpu):
    """Declaring fewer common blocks than the sequences share is valid: the
    rest of the shared blocks are read through each table by the decode
    kernels."""
    batch = W.shared_prefix_decode(seed=53, n=33, prefix_blocks=10, suffix_range=(1, 500))
    _check(batch, prefix_blocks=7)


@pytest.mark.parametrize("dtype,d,hq,hkv", [("f32", 128, 8, 2), ("f32", 64, 8, 8),
                                            ("bf16", 64, 16, 4)])
def test_cascade_other_types_run_decode(gpu, dtype, d, hq, hkv):
    """fp32 and head_dim 64 run the decode kernels over whole contexts: the
    same output as pa_decode, bit for bit, and oracle parity."""
    batch = W.shared_prefix_decode(seed=54, n=12, prefix_blocks=6, suffix_range=(1, 700),
                                   num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype)
    db, out = _check(batch)
    dec = db.attend().clone()
    torch.cuda.synchronize()
    assert torch.equal(out, dec)


def test_cascade_zero_prefix_is_decode(gpu):
    batch = W.shared_prefix_decode(seed=55, n=24, prefix_blocks=8, suffix_range=(1, 900))
    db, out = _check(batch, prefix_blocks=0)
    dec = db.attend().clone()
    torch.cuda.synchronize()
    assert torch.equal(out, dec)


def test_cascade_repeat_is_deterministic(gpu):
    batch = W.shared_prefix_decode(seed=56, n=70, prefix_blocks=20, suffix_range=(1, 1500))
    db, out = _check(batch)
    again = db.cascade().clone()
    torch.cuda.synchronize()
    assert torch.equal(out, again)


def test_cascade_out_of_pool_prefix_block(gpu):
    """A prefix entry outside the pool is an empty block for every sequence:
    its 16 keys drop out of every softmax, as in pa_decode."""
    batch = W.shared_prefix_decode(seed=57, n=10, prefix_blocks=8, suffix_range=(1, 300))
    db = _device_batch(batch)
    db.write_new()
    hs = host_state(batch)
    bt = db.block_tables.clone()
    bt[:, 3] = batch.num_blocks + 7
    db.block_tables.copy_(bt)
    got = db.cascade().clone()
    torch.cuda.synchronize()
    want = np.zeros((batch.num_seqs, batch.num_q_heads, batch.head_dim))
    for i in range(batch.num_seqs):
        n = int(batch.context_lens[i])
        keep = np.r_[0:48, 64:n]
        k = oracle.widen(oracle.gather(hs.k_cache, batch.block_tables[i], n))[keep]
        v = oracle.widen(oracle.gather(hs.v_cache, batch.block_tables[i], n))[keep]
        want[i] = oracle.attend(oracle.widen(hs.q[i:i + 1]), k, v, np.array([n - 16]),
                                batch.scale)[0]
    err = _max_err(got, want)
    say("max abs err", err)
    assert err <= TOL["bf16"], err


def test_cascade_full_shared_prefix(gpu):
    """The full shared-prefix configuration (128 sequences, 64 shared blocks,
    contexts up to 32768) in the benchmark's launch shape: every row against
    the oracle and against pa_decode."""
    batch = W.shared_prefix_decode()
    db, out = _check(batch)
    dec = db.attend().clone()
    torch.cuda.synchronize()
    err = float((out.float() - dec.float()).abs().max())
    say("cascade vs decode max abs diff", err)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("direct", ["0", "1"])
def test_cascade_private_parts_split_or_whole(gpu, monkeypatch, direct):
    """>= 1024 (sequence, kv head) pairs whose private parts fit one item:
    one partition per private part (the default) or 512-token partitions
    (PA_CASCADE_DIRECT=0), both against the oracle."""
    monkeypatch.setenv("PA_CASCADE_DIRECT", direct)
    batch = W.shared_prefix_decode(seed=60, n=132, prefix_blocks=24, suffix_range=(1, 1800))
    p = 24 * 16
    seqs = sorted(set(list(range(6)) + [66, 131]))
    _check(batch, ctx={0: 7, 1: p, 2: p + 1}, seqs=seqs)


@pytest.mark.parametrize("scale", [0.0, -0.0883883476])
def test_cascade_any_finite_scale(gpu, scale):
    """The common-prefix pass runs on the matrix cores, which fold a positive
    scale into their exponentials: a zero or negative scale still gives the
    oracle's attention with that scale (prefix partials merged with the
    decode kernels' private parts)."""
    import paged_kv_cache_token_amd as pa
    batch = W.shared_prefix_decode(seed=61, n=70, prefix_blocks=9, suffix_range=(1, 900))
    say(batch.name, "scale", scale)
    db = _device_batch(batch)
    db.write_new()
    p = batch.notes["prefix_tokens"] // 16
    out = pa.cascade_decode(db.q, db.k_cache, db.v_cache, db.block_tables, db.context_lens,
                            batch.max_context_len, p, scale)
    torch.cuda.synchronize()
    hs = host_state(batch)
    want = oracle.cascade_decode(hs.q, hs.k_cache, hs.v_cache, batch.block_tables,
                                 batch.context_lens, p, scale)
    err = _max_err(out, want)
    say("max abs err", err)
    assert err <= TOL["bf16"], err
