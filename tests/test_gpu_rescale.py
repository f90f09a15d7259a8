"""GPU parity under steep score ramps: the matrix-core kernels keep the
exponentials' reference lazily (raised only when a block's or tile's maximum
climbs more than 2^8 above it), so a context whose scores rise by more than
that from one 16-token block to the next forces a rescale on every block,
and one whose scores fall never rescales after its first block.

Inputs: the generated batch's caches and queries as the oracle writes them
(host side), with K of token t moved by beta * t along a fixed unit
direction u and every query by alpha * u, so each head's scores grow (or
shrink) by about alpha * beta per token; rounded to bf16 on the host and
uploaded over the device pools, so both sides read the same bits.  Bar: the
bf16 2e-2 max-abs error against the float64 oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle_side import host_state

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch on the CPU)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _ramp(batch, hs, alpha: float, beta: float, seed: int):
    """Host caches and queries with the score ramp (every written slot of
    every sequence: token t of its table row moves by beta * t along u)."""
    rng = np.random.default_rng(seed)
    d = batch.head_dim
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    k = oracle.widen(hs.k_cache).astype(np.float32)
    bs = batch.block_size
    if batch.kind == "decode":
        lens = np.asarray(batch.context_lens)
    else:
        lens = np.asarray(batch.context_offsets) + np.diff(np.asarray(batch.cu_seqlens))
    for i, n in enumerate(lens):
        for t in range(int(n)):
            blk = int(batch.block_tables[i][t // bs])
            k[blk, :, t % bs, :] += (beta * t) * u
    # the queries' own component along u is taken out first, so every head's
    # slope is alpha * beta (not alpha * beta + beta * (q . u), whose sign varies)
    q = oracle.widen(hs.q)
    q = (q - (q @ u)[..., None] * u + alpha * u).astype(np.float32)
    return _bf16_bits(k), _bf16_bits(q)


def _check_steep(batch, k_bits, q_bits, i: int, n: int, rising: bool):
    """Host check that the ramp does what the tests rely on, for every q head
    of sequence i (context n): in log2 units, the score maximum of at least 90%
    of its 16-token blocks lies more than 8 above the previous block's (a
    factor of 2^8: a rescale on nearly every block), or, falling, no block's
    maximum comes within 8 of the first block's (no rescale after it)."""
    bs = batch.block_size
    kv = oracle.widen(k_bits)
    g = batch.num_q_heads // batch.num_kv_heads
    rows = [int(batch.block_tables[i][t // bs]) for t in range(n)]
    for h in range(batch.num_q_heads):
        qv = oracle.widen(q_bits)[i, h]
        s = np.array([kv[rows[t], h // g, t % bs] @ qv for t in range(n)])
        s *= batch.scale * np.log2(np.e)
        bm = np.array([s[b:b + bs].max() for b in range(0, n, bs)])
        if rising:
            frac = float(np.mean(np.diff(bm) > 8.0))
            assert frac >= 0.9, (h, frac)
        else:
            assert np.all(bm[1:] < bm[0] - 8.0), (h, bm[1:].max() - bm[0])


def _upload(db, k_bits: np.ndarray, q_bits: np.ndarray):
    db.k_cache.copy_(torch.from_numpy(k_bits.view(np.int16)).view(db.k_cache.dtype))
    db.q.copy_(torch.from_numpy(q_bits.view(np.int16)).view(db.q.dtype))
    torch.cuda.synchronize()


@pytest.mark.parametrize("mfma", ["1", "0"])
@pytest.mark.parametrize("beta", [1.5, -1.5])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8)])
def test_decode_score_ramp(gpu, monkeypatch, mfma, beta, hq, hkv):
    """Decode with rising scores (a rescale on every block, all weight on the
    last token) and falling ones (all weight on the first), matrix-core and
    vector item code, split and single-partition contexts."""
    from device_batch import DeviceBatch
    monkeypatch.setenv("PA_DECODE_MFMA", mfma)
    lens = [1, 3, 17, 100, 513, 1100, 2049]
    batch = W.decode_batch(f"ramp_{hq}_{hkv}", 71, lens, hq, hkv, 128, "bf16", pool_factor=1.2)
    say(batch.name, "beta", beta, "PA_DECODE_MFMA", mfma)
    db = DeviceBatch(batch)
    db.write_new()
    hs = host_state(batch)
    k_bits, q_bits = _ramp(batch, hs, 4.0, beta, 5)
    _check_steep(batch, k_bits, q_bits, len(lens) - 1, lens[-1], beta > 0)
    _upload(db, k_bits, q_bits)
    got = db.attend().clone()
    torch.cuda.synchronize()
    want = oracle.decode(q_bits, k_bits, hs.v_cache, batch.block_tables, batch.context_lens,
                         batch.scale)
    err = float(np.abs(got.float().cpu().numpy().astype(np.float64) - want).max())
    say("max abs err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("beta", [1.5, -1.5])
def test_prefill_score_ramp(gpu, beta):
    """Packed chunks (the matrix-core prefill) and decode rows with rising
    and falling scores: every row of every chunk against the oracle."""
    from device_batch import DeviceBatch
    batch = W.varlen_batch("ramp_packed", 72, [1, 200, 77, 1, 300], [400, 130, 0, 1500, 700],
                           32, 8, 128, "bf16")
    say(batch.name, "beta", beta)
    db = DeviceBatch(batch)
    db.write_new()
    hs = host_state(batch)
    k_bits, q_bits = _ramp(batch, hs, 4.0, beta, 6)
    _upload(db, k_bits, q_bits)
    got = db.attend().clone()
    torch.cuda.synchronize()
    want = oracle.varlen_prefill(q_bits, k_bits, hs.v_cache, batch.cu_seqlens,
                                 batch.context_offsets, batch.block_tables, batch.scale)
    g = got.float().cpu().numpy().astype(np.float64)
    cu = batch.cu_seqlens
    err = max(float(np.abs(g[int(cu[i]):int(cu[i + 1])] - w).max()) for i, w in want.items())
    say("max abs err", err)
    assert err <= TOL, err
