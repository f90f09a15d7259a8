"""Seeded random sweep: many small shapes drawn at once (element type, head
dim, head ratio, sequence count, context lengths with partition and block
edges mixed in, chunk lengths, pool slack, common-prefix length) through the
decode, packed and cascade calls, each checked against the oracle: pools bit
for bit, outputs within max-abs 1e-5 (fp32) / 2e-2 (bf16)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from conftest import host_bits
from oracle_side import bits_equal, expected, host_state

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
# cases per call kind; PA_TEST_SWEEP_CASES=N draws N of each (same generator,
# the first cases unchanged) for a longer run
N_CASES = int(os.environ.get("PA_TEST_SWEEP_CASES", "0")) or None
# lengths that sit on the edges the kernels care about: one block, a tile of
# 64 keys, a 512-token partition, a 1024-token partition
EDGES = [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025]


def _heads(rng):
    g = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 3, 4]))
    return g * hkv, hkv


def _length(rng, hi):
    if rng.random() < 0.4:
        return int(rng.choice([e for e in EDGES if e <= hi]))
    return int(rng.integers(1, hi + 1))


def _decode_case(i):
    rng = np.random.default_rng(7000 + i)
    dtype = str(rng.choice(["f32", "bf16"]))
    d = int(rng.choice([64, 128]))
    hq, hkv = _heads(rng)
    n = int(rng.integers(1, 25))
    lens = [_length(rng, 2100) for _ in range(n)]
    pf = float(rng.uniform(1.0, 2.0))
    return W.decode_batch(f"sweep_decode_{i}", 7000 + i, lens, hq, hkv, d, dtype, pool_factor=pf)


def _varlen_case(i):
    rng = np.random.default_rng(8000 + i)
    # mostly the matrix-core path (bf16, d = 128); the rest take the row path
    dtype, d = ("bf16", 128) if rng.random() < 0.7 else (str(rng.choice(["f32", "bf16"])), 64)
    hq, hkv = _heads(rng)
    n = int(rng.integers(1, 9))
    q_lens = [1 if rng.random() < 0.35 else _length(rng, 300) for _ in range(n)]
    ctx = [0 if rng.random() < 0.2 else _length(rng, 1200) for _ in range(n)]
    pf = float(rng.uniform(1.0, 2.0))
    return W.varlen_batch(f"sweep_varlen_{i}", 8000 + i, q_lens, ctx, hq, hkv, d, dtype,
                          pool_factor=pf)


def _cascade_case(i):
    rng = np.random.default_rng(9000 + i)
    dtype, d = ("bf16", 128) if rng.random() < 0.75 else ("f32", 64)
    hq, hkv = _heads(rng)
    n = int(rng.integers(1, 71))
    pb = int(rng.integers(1, 41))
    lo = int(rng.integers(1, 40))
    return W.shared_prefix_decode(seed=9000 + i, n=n, prefix_blocks=pb,
                                  suffix_range=(lo, lo + int(rng.integers(0, 700))),
                                  num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _describe(b):
    return (b.name, b.dtype, "d", b.head_dim, "hq/hkv", b.num_q_heads, b.num_kv_heads,
            "n", b.num_seqs, "maxctx", b.max_context_len)


def _max_err(got, want):
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all()
    return float(np.abs(g - want).max()) if want.size else 0.0


@pytest.mark.parametrize("i", range(N_CASES or 24))
def test_sweep_decode(gpu, i):
    from device_batch import DeviceBatch
    b = _decode_case(i)
    say(*_describe(b))
    db = DeviceBatch(b)
    out = db.step()
    torch.cuda.synchronize()
    hs = host_state(b)
    assert bits_equal(host_bits(db.k_cache), hs.k_cache)
    assert bits_equal(host_bits(db.v_cache), hs.v_cache)
    err = _max_err(out, expected(b, hs))
    say("max abs err", err)
    assert err <= TOL[b.dtype], err


@pytest.mark.parametrize("i", range(N_CASES or 24))
def test_sweep_varlen(gpu, i):
    from device_batch import DeviceBatch
    b = _varlen_case(i)
    say(*_describe(b), "q_lens", (b.cu_seqlens[1:] - b.cu_seqlens[:-1]).tolist())
    db = DeviceBatch(b)
    out = db.step()
    torch.cuda.synchronize()
    hs = host_state(b)
    assert bits_equal(host_bits(db.k_cache), hs.k_cache)
    want = expected(b, hs)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = max((float(np.abs(got[int(b.cu_seqlens[s]):int(b.cu_seqlens[s + 1])] - w).max())
               for s, w in want.items() if w.size), default=0.0)
    say("max abs err", err)
    assert err <= TOL[b.dtype], err


@pytest.mark.parametrize("i", range(N_CASES or 16))
def test_sweep_cascade(gpu, i):
    from device_batch import DeviceBatch
    b = _cascade_case(i)
    p = b.notes["prefix_tokens"] // 16
    say(*_describe(b), "prefix blocks", p)
    db = DeviceBatch(b)
    db.write_new()
    out = db.cascade(prefix_blocks=p).clone()
    torch.cuda.synchronize()
    hs = host_state(b)
    want = oracle.cascade_decode(hs.q, hs.k_cache, hs.v_cache, b.block_tables, b.context_lens, p,
                                 b.scale)
    err = _max_err(out, want)
    say("max abs err", err)
    assert err <= TOL[b.dtype], err
