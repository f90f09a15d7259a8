"""pa_decode_noalloc: pa_decode with its split-K partials in the library's
fixed per-GPU scratch instead of a caller workspace (for callers that cannot
allocate).  Called through the C ABI (the binding marshals pointers only) and
compared with pa_decode on the same inputs, bit for bit, and with the oracle
at the bf16 bar, on two calls in a row, the second smaller: the scratch keeps
the first call's contents, which the second must not read; and captured in a
HIP graph, replayed."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle_side import expected, host_state

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _one(batch):
    import paged_kv_cache_token_amd as pa
    from device_batch import DeviceBatch
    say("noalloc vs pa_decode", batch.name, "n", batch.num_seqs, "maxctx", batch.max_context_len)
    db = DeviceBatch(batch)
    db.write_new()
    want_gpu = db.attend().clone()
    out = torch.full_like(db.q, float("nan"))
    got = pa.decode_noalloc(db.q, db.k_cache, db.v_cache, db.block_tables, db.context_lens,
                            batch.max_context_len, batch.scale, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got, want_gpu), "pa_decode_noalloc differs from pa_decode"
    hs = host_state(batch)
    g = got.float().cpu().numpy().astype(np.float64)
    err = float(np.abs(g - expected(batch, hs)).max())
    say("max abs err", err)
    assert err <= TOL[batch.dtype], err


def test_noalloc_two_calls_second_smaller(gpu):
    # contexts past one partition: the partials and the work list use the scratch
    lens_a = [1, 17, 511, 513, 1100, 2049, 3000, 4096, 700, 64] * 3
    a = W.decode_batch("noalloc_a", 71, lens_a, 32, 8, 128, "bf16", pool_factor=1.2)
    b = W.decode_batch("noalloc_b", 72, [1500, 3, 900, 2100], 16, 4, 128, "bf16",
                       pool_factor=1.2)
    _one(a)
    _one(b)


def test_noalloc_fp32_and_single_partition(gpu):
    # fp32 d=64 with a split, then a batch that fits one partition (no scratch)
    _one(W.decode_batch("noalloc_f32", 73, [1, 16, 17, 700, 1500], 8, 8, 64, "f32",
                        pool_factor=1.3))
    _one(W.llama2_decode())


def test_noalloc_in_a_graph(gpu):
    """The callers it is for: a captured pa_decode_noalloc (work list, split
    items and merge on the library's scratch) replayed four times with eager
    work between, every replay equal to the eager call bit for bit and to
    the oracle within the bar."""
    import paged_kv_cache_token_amd as pa
    from device_batch import DeviceBatch
    batch = W.decode_batch("noalloc_graph", 74, [1, 17, 513, 1100, 2049, 4096, 300] * 4, 32, 8,
                           128, "bf16", pool_factor=1.2)
    say("noalloc graph", batch.name)
    db = DeviceBatch(batch)
    db.write_new()
    out = torch.empty_like(db.q)

    def run():
        pa.decode_noalloc(db.q, db.k_cache, db.v_cache, db.block_tables, db.context_lens,
                          batch.max_context_len, batch.scale, out=out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    hs = host_state(batch)
    want = expected(batch, hs)
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
        err = float(np.abs(out.float().cpu().numpy().astype(np.float64) - want).max())
        say("replay", r, "max abs err", err)
        assert err <= TOL[batch.dtype], err
        torch.randn(1 << 20, device="cuda").sum().item()


def test_noalloc_refuses_beyond_scratch(gpu):
    """Shapes whose partials exceed the fixed scratch are refused on the
    host, before anything is enqueued (status PA_ERR_SCRATCH_TOO_SMALL)."""
    import paged_kv_cache_token_amd as pa
    fake = 0x1000
    # 4096 sequences x 64 q heads of 65536 tokens: 64 partitions of 1024
    st = pa.lib.pa_decode_noalloc(fake, fake, fake, fake, fake, fake, 4096, 64, 8, 128, 16,
                                  4096, 65536, 1 << 20, 0.1, pa.PA_BF16, None)
    assert st == 8
