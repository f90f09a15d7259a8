"""GPU parity of pa_varlen_prefill (packed super-sequence: prefill chunks and
decode rows) against the oracle, max-abs error <= 2e-2 (bf16 inputs, fp32
accumulation), plus packing invariance and agreement with pa_decode."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle_side import expected, host_state

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _device_batch(batch):
    from device_batch import DeviceBatch
    return DeviceBatch(batch)


def _check(batch, seqs=None):
    say(batch.name, "n", batch.num_seqs, "total_q", batch.total_q, "max_q", batch.max_q_len,
        "maxctx", batch.max_context_len, "g", batch.num_q_heads // batch.num_kv_heads)
    db = _device_batch(batch)
    out = db.step()
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    hs = host_state(batch)
    assert np.array_equal(db.slots.cpu().numpy(), hs.new_slots)
    want = expected(batch, hs, seqs)
    err = 0.0
    for i, rows in want.items():
        lo, hi = int(batch.cu_seqlens[i]), int(batch.cu_seqlens[i + 1])
        err = max(err, float(np.abs(got[lo:hi] - rows).max()) if rows.size else 0.0)
    say("max abs err", err)
    assert err <= TOL, err
    return db, out


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (16, 4), (32, 4), (16, 8)])
def test_prefill_chunks_with_context(gpu, hq, hkv):
    # ragged chunk lengths (q tiles and 64-key tiles with tails), prior context
    # off and on block / tile edges, a two-token chunk
    q_lens = [100, 70, 2, 129, 33, 64]
    ctx = [0, 37, 5, 200, 64, 1000]
    _check(W.varlen_batch(f"chunks_{hq}_{hkv}", 21, q_lens, ctx, hq, hkv, 128, "bf16"))


def test_mixed_rows_small(gpu):
    # decode rows (q_len 1) interleaved with chunks in one super-sequence
    q_lens = [1, 45, 1, 1, 300, 1, 17]
    ctx = [700, 0, 1, 2047, 300, 15, 16]
    _check(W.varlen_batch("mixed_small", 22, q_lens, ctx, 32, 8, 128, "bf16"))


def test_packing_invariance(gpu):
    """Each sequence's rows are the same whether it is packed with others or
    alone: bit for bit for the prefill chunks (one item per query tile,
    whatever else is packed); a decode row's split over partitions and waves
    follows the call's shape (its longest context, whether any context is
    split), so packed and alone it agrees within the bf16 bar."""
    import paged_kv_cache_token_amd as pa
    q_lens = [1, 96, 1, 40]
    ctx = [500, 33, 1200, 0]
    batch = W.varlen_batch("packed", 23, q_lens, ctx, 32, 8, 128, "bf16")
    db = _device_batch(batch)
    packed = db.step().clone()
    for i in range(batch.num_seqs):
        lo, hi = int(batch.cu_seqlens[i]), int(batch.cu_seqlens[i + 1])
        cu = torch.tensor([0, hi - lo], dtype=torch.int32, device="cuda")
        co = db.context_offsets[i:i + 1].contiguous()
        bt = db.block_tables[i:i + 1].contiguous()
        solo = pa.varlen_prefill(db.q[lo:hi].contiguous(), db.k_cache, db.v_cache, cu, co, bt,
                                 hi - lo, int(batch.context_lens[i]), batch.scale)
        torch.cuda.synchronize()
        if hi - lo > 1:
            assert torch.equal(solo, packed[lo:hi]), i
        else:
            err = float((solo.float() - packed[lo:hi].float()).abs().max())
            assert err <= TOL, (i, err)


def test_prefill_rows_match_decode(gpu):
    """Row j of a chunk after c cached tokens attends what a decode step with
    context c + j + 1 attends (two kernels: equal within the tolerance)."""
    import paged_kv_cache_token_amd as pa
    batch = W.varlen_batch("rows_vs_decode", 24, [77], [150], 32, 8, 128, "bf16")
    db = _device_batch(batch)
    pre = db.step().clone()
    L = 77
    bt = db.block_tables.expand(L, -1).contiguous()
    lens = torch.arange(151, 151 + L, dtype=torch.int32, device="cuda")
    dec = pa.decode(db.q, db.k_cache, db.v_cache, bt, lens, 150 + L, batch.scale)
    torch.cuda.synchronize()
    assert float((dec.float() - pre.float()).abs().max()) <= TOL


def test_prefill_deterministic(gpu):
    batch = W.varlen_batch("repeat", 25, [200, 1, 90], [300, 40, 0], 32, 8, 128, "bf16")
    db = _device_batch(batch)
    a = db.step().clone()
    b = db.attend().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_prefill_only_config(gpu):
    _check(W.prefill_only())


def test_prefill_long_one_sequence(gpu):
    """The long-chunk workload (4 x 2048 new tokens after 2048 cached, the
    benchmark's launch): one whole sequence against the oracle."""
    _check(W.prefill_long(), seqs=[2])


def test_mixed_step_full(gpu):
    """The mixed step (4096 packed rows: ~750 decode rows and 8 prefill
    chunks): every row of every sequence against the oracle."""
    _check(W.mixed_step())


@pytest.mark.parametrize("bad_id", [-3, 10 ** 6])
def test_out_of_pool_block_takes_no_part(gpu, bad_id):
    """A live table entry outside [0, num_blocks) is an empty block: its 16
    tokens drop out of every row's softmax (the documented contract for
    invalid ids).  Expected: the oracle's attention over the sequence's other
    tokens, each row seeing 16 fewer keys."""
    import oracle
    q_lens, ctx = [90, 1], [70, 300]
    batch = W.varlen_batch("bad_block", 26, q_lens, ctx, 32, 8, 128, "bf16")
    db = _device_batch(batch)
    db.step()
    hs = host_state(batch)
    drop = {0: 2, 1: 7}  # logical block dropped per sequence (inside the context)
    bt = db.block_tables.clone()
    for i, j in drop.items():
        bt[i, j] = bad_id
    db.block_tables.copy_(bt)
    got = db.attend().float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    err = 0.0
    for i, j in drop.items():
        n = int(batch.context_lens[i])
        keep = np.r_[0:16 * j, 16 * (j + 1):n]
        k = oracle.widen(oracle.gather(hs.k_cache, batch.block_tables[i], n))[keep]
        v = oracle.widen(oracle.gather(hs.v_cache, batch.block_tables[i], n))[keep]
        lo, hi = int(batch.cu_seqlens[i]), int(batch.cu_seqlens[i + 1])
        visible = int(batch.context_offsets[i]) + np.arange(1, hi - lo + 1) - 16
        want = oracle.attend(oracle.widen(hs.q[lo:hi]), k, v, visible, batch.scale)
        err = max(err, float(np.abs(got[lo:hi] - want).max()))
    say("max abs err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 64, 32, 8), ("f32", 128, 8, 8),
                                            ("f32", 64, 16, 4)])
def test_varlen_rows_path(gpu, dtype, d, hq, hkv):
    """fp32 and head_dim 64: every packed row through the decode kernels on its
    own (causal context per row), decode rows and chunks mixed."""
    q_lens = [1, 70, 1, 33, 2, 1]
    ctx = [300, 0, 17, 150, 900, 1]
    batch = W.varlen_batch(f"rows_{dtype}_{d}_{hq}_{hkv}", 29, q_lens, ctx, hq, hkv, d, dtype)
    tol = 1e-5 if dtype == "f32" else TOL
    say(batch.name, "tol", tol)
    db = _device_batch(batch)
    out = db.step()
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    hs = host_state(batch)
    want = expected(batch, hs)
    err = 0.0
    for i, rows in want.items():
        lo, hi = int(batch.cu_seqlens[i]), int(batch.cu_seqlens[i + 1])
        err = max(err, float(np.abs(got[lo:hi] - rows).max()))
    say("max abs err", err)
    assert err <= tol, err


@pytest.mark.parametrize("grid,hq,hkv", [("1", 32, 8), ("3", 32, 8), ("17", 32, 8),
                                         ("2", 8, 8), ("5", 16, 2)])
def test_prefill_many_items_per_workgroup(gpu, monkeypatch, grid, hq, hkv):
    """Persistent workgroups run several items each, the next item's record,
    first two key tiles and queries loaded during the current one (items of
    1, 2, 3 and more key tiles back to back): same output, bit for bit, as
    one item per workgroup, and parity with the oracle."""
    q_lens = [100, 70, 2, 129, 33, 64, 1, 250]
    ctx = [0, 37, 5, 200, 64, 1000, 300, 17]
    batch = W.varlen_batch(f"many_items_{grid}_{hq}_{hkv}", 23, q_lens, ctx, hq, hkv, 128,
                           "bf16")
    db, out = _check(batch)
    ref = out.clone()
    monkeypatch.setenv("PA_PREFILL_GRID", grid)
    got = db.attend().clone()
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


@pytest.mark.parametrize("inline", ["0", "1"])
def test_packed_call_beyond_plan_lds(gpu, monkeypatch, inline):
    """A packed call of more sequences than the prefill plan kernel holds in
    LDS (2048): mostly decode rows, a few chunks; that kernel's loop path
    (PA_PREFILL_INLINE_PLAN=0), and the list built in every workgroup."""
    monkeypatch.setenv("PA_PREFILL_INLINE_PLAN", inline)
    rng = np.random.default_rng(24)
    n = 2100
    q_lens = np.ones(n, dtype=np.int64)
    chunk_at = [5, 900, 2099]
    for i, L in zip(chunk_at, (70, 130, 33)):
        q_lens[i] = L
    ctx = rng.integers(0, 200, size=n)
    batch = W.varlen_batch("plan_2100", 24, q_lens, ctx, 32, 8, 128, "bf16")
    seqs = sorted(set(chunk_at + [0, 1, 2000] + rng.choice(n, size=20, replace=False).tolist()))
    _check(batch, seqs=seqs)


def _plan_case(kind):
    """Packed calls at the edges of the in-workgroup work list: many (sequence,
    query tile) pairs (4000 two-row sequences, each wave of the ranking over
    500 pairs), the largest sequence count it takes (4096) and one more (the
    plan kernel's), one kv head per item on a one-row-per-head model, and a
    grid of 3 workgroups holding about 120 items each."""
    rng = np.random.default_rng(26)
    if kind == "pairs_4000":
        n = 4000
        return W.varlen_batch(kind, 26, np.full(n, 2), rng.integers(0, 300, size=n), 32, 8, 128,
                              "bf16"), None
    if kind in ("seqs_4096", "seqs_4097"):
        n = int(kind.split("_")[1])
        q_lens = np.ones(n, dtype=np.int64)
        at = rng.choice(n, size=40, replace=False)
        q_lens[at] = rng.integers(2, 200, size=40)
        q_lens[n - 1] = 77  # the last sequence's end row is read too
        return W.varlen_batch(kind, 27, q_lens, rng.integers(0, 400, size=n), 32, 8, 128,
                              "bf16"), None
    if kind == "mha":
        return W.varlen_batch(kind, 28, [300, 1, 257, 2, 700, 64], [0, 50, 300, 4, 1, 999],
                              32, 32, 128, "bf16"), None
    return W.varlen_batch(kind, 29, [100, 70, 2, 129, 33, 64, 1, 250, 400, 31],
                          [0, 37, 5, 200, 64, 1000, 300, 17, 2, 90], 32, 8, 128, "bf16"), "3"


@pytest.mark.parametrize("kind", ["pairs_4000", "seqs_4096", "seqs_4097", "mha", "grid_3"])
def test_inline_plan_matches_plan_kernel(gpu, monkeypatch, kind):
    """Every workgroup builds the longest-first work list itself (no plan
    launch) when the call fits its bounds; PA_PREFILL_INLINE_PLAN=0 makes the
    one-workgroup plan kernel build it instead.  Each item's arithmetic does
    not depend on where it runs, so both give the same output bit for bit --
    every row written (outputs start as NaN) -- and sampled sequences match
    the oracle."""
    batch, grid = _plan_case(kind)
    if grid:
        monkeypatch.setenv("PA_PREFILL_GRID", grid)
    rng = np.random.default_rng(30)
    n = batch.num_seqs
    multi = [i for i in range(n) if batch.cu_seqlens[i + 1] - batch.cu_seqlens[i] >= 2]
    seqs = sorted(set([0, n - 1] + rng.choice(multi, size=min(len(multi), 24),
                                                replace=False).tolist()))
    db, out = _check(batch, seqs=seqs)
    outs = []
    for inline in ("1", "0"):
        monkeypatch.setenv("PA_PREFILL_INLINE_PLAN", inline)
        o = torch.full_like(out, float("nan"))
        db.attend(out=o)
        torch.cuda.synchronize()
        say(kind, "PA_PREFILL_INLINE_PLAN", inline, "all finite", bool(torch.isfinite(o).all()))
        outs.append(o)
    assert torch.isfinite(outs[0]).all() and torch.isfinite(outs[1]).all()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0], out)


def test_packed_call_more_rows_than_grid_y(gpu):
    """70000 single-token rows, one of them with a context long enough to be
    split: the merge runs over more (row, head) pairs than a grid's y extent
    holds (its grid is 1-D)."""
    rng = np.random.default_rng(25)
    n = 70000
    ctx = rng.integers(0, 4, size=n)
    ctx[123] = 5000
    batch = W.varlen_batch("rows_70000", 25, np.ones(n, dtype=np.int64), ctx, 8, 1, 128, "bf16")
    seqs = sorted(set([0, 123, n - 1] + rng.choice(n, size=30, replace=False).tolist()))
    _check(batch, seqs=seqs)


@pytest.mark.parametrize("name", ["prefill_only", "mixed", "mixed_f32_rows"])
def test_decode_row_count_hint(gpu, name):
    """pa_varlen_prefill_ex with the host's count of single-token rows gives
    pa_varlen_prefill's output bit for bit (0 for a prefill-only step, where
    it launches no decode kernels; the fp32 row path ignores the count)."""
    from device_batch import DeviceBatch
    if name == "prefill_only":
        batch = W.varlen_batch("hint_chunks", 61, [70, 300, 2, 129], [0, 900, 5, 40], 32, 8, 128,
                               "bf16")
    elif name == "mixed":
        batch = W.varlen_batch("hint_mixed", 62, [1, 70, 1, 1, 200], [800, 30, 2000, 0, 0], 32,
                               8, 128, "bf16")
    else:
        batch = W.varlen_batch("hint_f32", 64, [1, 33, 1, 9], [300, 20, 700, 0], 8, 2, 64, "f32")
    a = DeviceBatch(batch, hint_rows=False)
    want = a.step().clone()
    b = DeviceBatch(batch, hint_rows=True)
    say(name, "decode rows", b.num_decode_rows)
    got = b.step().clone()
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    # "unknown" (negative) and a positive count that overstates the rows run
    # the decode kernels as pa_varlen_prefill does: the same output
    for count in (-1, b.num_decode_rows + 3):
        b.num_decode_rows = count
        again = b.attend().clone()
        torch.cuda.synchronize()
        assert torch.equal(again, want), count


def test_zero_row_count_skips_decode_rows(gpu):
    """A count of 0 with single-token rows present: those rows of out are
    left as they were, every chunk row is pa_varlen_prefill's."""
    import paged_kv_cache_token_amd as pa
    from device_batch import DeviceBatch
    batch = W.varlen_batch("hint_zero", 63, [1, 90, 1, 40], [300, 10, 700, 0], 32, 8, 128, "bf16")
    db = DeviceBatch(batch, hint_rows=False)
    want = db.step().clone()
    out = torch.full_like(want, 7.0)
    pa.varlen_prefill(db.q, db.k_cache, db.v_cache, db.cu_seqlens, db.context_offsets,
                      db.block_tables, batch.max_q_len, batch.max_context_len, batch.scale,
                      out=out, workspace=db.workspace, num_decode_rows=0)
    torch.cuda.synchronize()
    ql = torch.as_tensor(batch.q_lens).long()
    rows = (ql == 1).repeat_interleave(ql)
    rows = rows.to(out.device)
    assert (out[rows] == 7.0).all()
    assert torch.equal(out[~rows], want[~rows])



@pytest.mark.parametrize("scale", [0.0, -0.0883883476, -1.0])
def test_varlen_any_finite_scale(gpu, scale):
    """The matrix-core path takes any finite scale, as the decode kernels do:
    0 weighs every visible key alike, a negative scale favours the smallest
    scores.  Chunks (matrix cores) and a decode row against the oracle run
    with the same scale."""
    import oracle
    import paged_kv_cache_token_amd as pa
    batch = W.varlen_batch("any_scale", 27, [90, 1, 33, 200], [70, 300, 0, 64], 32, 8, 128,
                           "bf16")
    say(batch.name, "scale", scale)
    db = _device_batch(batch)
    db.write_new()
    out = pa.varlen_prefill(db.q, db.k_cache, db.v_cache, db.cu_seqlens, db.context_offsets,
                            db.block_tables, batch.max_q_len, batch.max_context_len, scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    hs = host_state(batch)
    want = oracle.varlen_prefill(hs.q, hs.k_cache, hs.v_cache, batch.cu_seqlens,
                                 batch.context_offsets, batch.block_tables, scale)
    err = max(float(np.abs(got[int(batch.cu_seqlens[i]):int(batch.cu_seqlens[i + 1])] - w).max())
              for i, w in want.items())
    say("max abs err", err)
    assert err <= TOL, err
