"""HIP-graph capture of the hot path: a decode step (pa_decode_step), a
packed prefill call (slot mapping + write + pa_varlen_prefill) and a cascade
decode are captured once and replayed several times, with eager work and synchronisation between
replays; every replay must equal the eager result bit for bit (the library
allocates nothing, synchronises nothing and records no memset, so a captured
call is the same launches)."""
import sys

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _bits(t: torch.Tensor) -> torch.Tensor:
    """integer view, so NaN canaries compare by bit pattern"""
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def _replays(make_batch, run, n_replays=4):
    from device_batch import DeviceBatch
    batch = make_batch()
    say(batch.name, "graph replays", n_replays)
    db = DeviceBatch(batch)
    k0, v0 = db.k_cache.clone(), db.v_cache.clone()
    eager = run(db).clone()
    torch.cuda.synchronize()
    k_eager, v_eager = db.k_cache.clone(), db.v_cache.clone()

    db.k_cache.copy_(k0)
    db.v_cache.copy_(v0)
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(db, out)  # warm-up on the capture stream (first-call host setup)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(db, out)
    for r in range(n_replays):
        db.k_cache.copy_(k0)
        db.v_cache.copy_(v0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(eager)), f"replay {r}: output differs from the eager call"
        assert torch.equal(_bits(db.k_cache), _bits(k_eager)) and \
            torch.equal(_bits(db.v_cache), _bits(v_eager)), f"replay {r}: cache differs from the eager call"
        # unrelated eager work between replays
        torch.randn(1 << 20, device="cuda").sum().item()


def test_graph_decode_step(gpu):
    def run(db, out=None):
        return db.fused_step(out)
    _replays(W.llama2_decode, run)


def test_graph_gqa_decode_multi_partition(gpu):
    # plan + list + merge launches (multi-partition contexts) in one graph
    def run(db, out=None):
        return db.fused_step(out)
    _replays(W.gqa_decode, run)


def test_graph_mixed_step(gpu):
    def run(db, out=None):
        db.write_new()
        return db.attend(out)
    _replays(W.mixed_step, run)


def test_graph_cascade_decode(gpu):
    # the common-prefix pass, the decode kernels over the private parts and
    # the merge, captured together
    def run(db, out=None):
        db.write_new()
        return db.cascade(out)
    _replays(lambda: W.shared_prefix_decode(seed=58, n=70, prefix_blocks=20,
                                            suffix_range=(1, 1500)), run)


def test_graph_cascade_single_partition_rest(gpu):
    # >= 1024 (sequence, kv head) pairs with short private parts: the prefix
    # pass, the single-partition kernel writing one partial per pair, and the
    # merge, captured together
    def run(db, out=None):
        db.write_new()
        return db.cascade(out)
    _replays(lambda: W.shared_prefix_decode(seed=59, n=130, prefix_blocks=20,
                                            suffix_range=(1, 1500)), run)


def test_graph_prefill_only_step(gpu):
    # a packed step with no single-token rows, the row count passed: slot
    # mapping, store, the prefill plan and the prefill kernel only
    def run(db, out=None):
        db.write_new()
        return db.attend(out)
    _replays(W.prefill_only, run)
