"""Slot mapping and KV store on inconsistent or out-of-range device metadata:
the kernels keep every access inside the buffers the call names, and what they
do write is what the oracle computes (bit-exact)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from conftest import host_bits

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def test_slot_mapping_stops_at_num_tokens(gpu):
    """cu_seqlens that run past num_tokens: the first num_tokens slots are the
    oracle's and the guard entries behind them are left as they were."""
    pa = gpu
    say("slot mapping, cu_seqlens past num_tokens")
    dev = torch.device("cuda")
    rng = np.random.default_rng(61)
    lens = np.array([5, 40, 1, 300, 17], np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ctx = rng.integers(0, 200, size=len(lens)).astype(np.int32)
    maxb = int(-(-(ctx + lens).max() // 16))
    bt = rng.permutation(len(lens) * maxb).reshape(len(lens), maxb).astype(np.int32)
    n_tok = int(cu[-1]) - 123               # the last sequence overruns by 123 tokens
    guard = 256
    out = torch.full((n_tok + guard,), -7, dtype=torch.int64, device=dev)
    pa.build_slot_mapping(torch.from_numpy(cu).to(dev), torch.from_numpy(ctx).to(dev),
                          torch.from_numpy(bt).to(dev), n_tok, out=out[:n_tok])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.slot_mapping(bt, cu, ctx)
    assert np.array_equal(got[:n_tok], want[:n_tok])
    assert (got[n_tok:] == -7).all()


def test_slot_mapping_past_table_and_store_skips(gpu):
    """Positions past the table get slot -1; pa_write_kv stores nothing for a
    negative slot or one past the pool, and every other row bit for bit."""
    pa = gpu
    say("slot -1 past the table, store skips bad slots")
    dev = torch.device("cuda")
    hkv, d, nblk = 2, 64, 6
    cu = np.array([0, 20, 50], np.int32)
    ctx = np.array([0, 10], np.int32)
    bt = np.array([[3, 1], [0, 5]], np.int32)   # sequence 1's tokens 22.. run past its table
    slots = pa.build_slot_mapping(torch.from_numpy(cu).to(dev), torch.from_numpy(ctx).to(dev),
                                  torch.from_numpy(bt).to(dev), 50)
    torch.cuda.synchronize()
    s = slots.cpu().numpy()
    assert (s[20 + 22:] == -1).all() and (s[:20 + 22] >= 0).all()
    assert np.array_equal(s[:42], oracle.slot_mapping(bt, cu[:2], ctx[:1]).tolist()
                          + oracle.slot_mapping(bt[1:], np.array([0, 22]), ctx[1:]).tolist())
    s_bad = s.copy()
    s_bad[3] = nblk * 16          # first slot past the pool
    s_bad[4] = 10 ** 9
    g = torch.Generator(device="cpu").manual_seed(62)
    k = torch.randn(50, hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(50, hkv, d, generator=g).to(torch.bfloat16)
    kc = torch.full((nblk, hkv, 16, d), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full_like(kc, float("nan"))
    pa.write_kv(k.to(dev), v.to(dev), kc, vc, torch.from_numpy(s_bad).to(dev))
    torch.cuda.synchronize()
    kw = np.full((nblk, hkv, 16, d), 0x7FC0, np.uint16)
    vw = kw.copy()
    keep = (s_bad >= 0) & (s_bad < nblk * 16)
    oracle.write_kv(kw, vw, host_bits(k)[keep], host_bits(v)[keep], s_bad[keep])
    assert np.array_equal(host_bits(kc), kw)
    assert np.array_equal(host_bits(vc), vw)
