"""HIP-graph capture of the hot path: a decode step (pa_decode_step), a
packed prefill call (slot mapping + write + pa_varlen_prefill) and a cascade
decode are captured once and replayed several times, with eager work and synchronisation between
replays; every replay must equal the eager result bit for bit (the library
allocates nothing, synchronises nothing and records no memset, so a captured
call is the same launches) and the oracle within the bars (max-abs 1e-5 for
fp32, 2e-2 for bf16), with the caches the replay leaves bit-exact to the
oracle's.  Several layers' steps captured into one graph (a model's forward
pass) are checked the same way, layer by layer."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from conftest import host_bits
from oracle_side import bits_equal, host_state

TOL = {"f32": 1e-5, "bf16": 2e-2}

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _bits(t: torch.Tensor) -> torch.Tensor:
    """integer view, so NaN canaries compare by bit pattern"""
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def _oracle_want(batch, cascade_blocks=None):
    """The oracle's caches after the step and its output for the batch."""
    hs = host_state(batch)
    if batch.kind != "decode":
        return hs, oracle.varlen_prefill(hs.q, hs.k_cache, hs.v_cache, batch.cu_seqlens,
                                         batch.context_offsets, batch.block_tables, batch.scale)
    if cascade_blocks is not None:
        return hs, oracle.cascade_decode(hs.q, hs.k_cache, hs.v_cache, batch.block_tables,
                                         batch.context_lens, cascade_blocks, batch.scale)
    return hs, oracle.decode(hs.q, hs.k_cache, hs.v_cache, batch.block_tables,
                             batch.context_lens, batch.scale)


def _oracle_check(batch, out, k_cache, v_cache, hs_want):
    """out (one replay's result) and the caches it left against the oracle."""
    hs, want = hs_want
    assert bits_equal(host_bits(k_cache), hs.k_cache), "cache differs from the oracle's"
    assert bits_equal(host_bits(v_cache), hs.v_cache), "cache differs from the oracle's"
    got = out.float().cpu().numpy().astype(np.float64)
    if batch.kind == "decode":
        err = float(np.abs(got - want).max())
    else:
        cu = batch.cu_seqlens
        err = max(float(np.abs(got[int(cu[i]):int(cu[i + 1])] - w).max()) for i, w in want.items())
    say("replay vs oracle max abs err", err)
    assert err <= TOL[batch.dtype], err


def _replays(make_batch, run, n_replays=4, cascade=False):
    from device_batch import DeviceBatch
    batch = make_batch()
    say(batch.name, "graph replays", n_replays)
    db = DeviceBatch(batch)
    k0, v0 = db.k_cache.clone(), db.v_cache.clone()
    eager = run(db).clone()
    torch.cuda.synchronize()
    k_eager, v_eager = db.k_cache.clone(), db.v_cache.clone()
    # every replay equals the eager call bit for bit, so this checks them all
    _oracle_check(batch, eager, k_eager, v_eager,
                  _oracle_want(batch, batch.notes["prefix_tokens"] // 16 if cascade else None))

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
                                            suffix_range=(1, 1500)), run, cascade=True)


def test_graph_cascade_single_partition_rest(gpu):
    # >= 1024 (sequence, kv head) pairs with short private parts: the prefix
    # pass, the single-partition kernel writing one partial per pair, and the
    # merge, captured together
    def run(db, out=None):
        db.write_new()
        return db.cascade(out)
    _replays(lambda: W.shared_prefix_decode(seed=59, n=130, prefix_blocks=20,
                                            suffix_range=(1, 1500)), run, cascade=True)


def test_graph_prefill_only_step(gpu):
    # a packed step with no single-token rows, the row count passed: slot
    # mapping, store, the prefill plan and the prefill kernel only
    def run(db, out=None):
        db.write_new()
        return db.attend(out)
    _replays(W.prefill_only, run)


@pytest.mark.parametrize("name", ["llama2", "gqa", "mixed"])
def test_graph_several_layers_in_one_graph(gpu, name):
    """Three layers' steps (each layer its own caches and values, one set of
    block tables) captured into one graph, replayed three times with eager
    work between: every layer's output and caches against the oracle after
    each replay."""
    from device_batch import DeviceBatch
    make = {"llama2": W.llama2_decode, "gqa": W.gqa_decode, "mixed": W.mixed_step}[name]
    base = make()
    layers = [base.with_layer(l) for l in range(3)]
    say(base.name, "3 layers in one graph")
    dbs = [DeviceBatch(b) for b in layers]
    fused = base.kind == "decode"
    snap = [(d.k_cache.clone(), d.v_cache.clone()) for d in dbs]
    outs = [torch.empty_like(d.q) for d in dbs]

    def run_all():
        for d, o in zip(dbs, outs):
            if fused:
                d.fused_step(o)
            else:
                d.write_new()
                d.attend(o)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_all()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    wants = [_oracle_want(b) for b in layers]
    for r in range(3):
        for d, (k0, v0), o in zip(dbs, snap, outs):
            d.k_cache.copy_(k0)
            d.v_cache.copy_(v0)
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for b, d, o, w in zip(layers, dbs, outs, wants):
            say("replay", r, "layer", b.layer)
            _oracle_check(b, o, d.k_cache, d.v_cache, w)
        torch.randn(1 << 20, device="cuda").sum().item()
