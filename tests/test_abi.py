"""The C-ABI library loads, exports what include/pa.h declares, and rejects bad
arguments on the host.  No call here reaches the GPU: every error path returns
before anything is enqueued, and zero-size calls return before any HIP call."""
import ctypes
import subprocess

import pytest

import paged_kv_cache_token_amd as pa

L = pa.lib
FAKE = 0x1000  # a non-null pointer value that is never dereferenced on the host


def test_exports_every_declared_function():
    names = pa.header_functions()
    assert {"pa_build_slot_mapping", "pa_write_kv", "pa_decode", "pa_decode_workspace_size",
            "pa_varlen_prefill", "pa_varlen_workspace_size", "pa_status_string",
            "pa_version"} <= set(names)
    syms = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    exported = {line.split()[-1] for line in syms.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_version_and_status_strings():
    assert pa.version() == 100
    assert pa.status_string(0) == "ok"
    for s in range(1, 9):
        assert pa.status_string(s) not in ("ok", "unknown status")
    assert pa.status_string(99) == "unknown status"


def test_decode_workspace_size():
    # a context that fits the shortest partition (256 tokens) needs no workspace
    assert L.pa_decode_workspace_size(64, 32, 128, 256, pa.PA_BF16) == 0
    assert L.pa_decode_workspace_size(64, 32, 128, 257, pa.PA_BF16) > 0
    # sized for the shortest partition (256 tokens): 513 tokens -> 3 partitions of
    # (m, l, acc[128]) per (seq, q head), plus the item count and the
    # (seq, partition) list
    assert L.pa_decode_workspace_size(4, 8, 128, 513, pa.PA_BF16) == \
        4 * 8 * 3 * 130 * 4 + 8 + 4 * 3 * 8
    assert L.pa_decode_workspace_size(4, 8, 96, 513, pa.PA_BF16) == 0        # unsupported d
    assert L.pa_varlen_workspace_size(10, 100, 32, 8, 128, 2000, pa.PA_BF16) > 0
    # fp32 / head_dim 64: every row through the decode kernels, sized per row
    assert L.pa_varlen_workspace_size(10, 100, 32, 8, 128, 2000, pa.PA_F32) > 0
    assert L.pa_varlen_workspace_size(10, 100, 32, 8, 64, 2000, pa.PA_BF16) > 0
    assert L.pa_varlen_workspace_size(10, 100, 32, 8, 96, 2000, pa.PA_BF16) == 0


def _decode(**over):
    args = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, ctx=FAKE, n=4, hq=8, hkv=2, d=128,
                bs=16, maxb=8, maxctx=100, nblocks=64, scale=0.1, dtype=pa.PA_BF16, ws=None,
                wsb=0, stream=None)
    args.update(over)
    return L.pa_decode(args["out"], args["q"], args["k"], args["v"], args["bt"], args["ctx"],
                       args["n"], args["hq"], args["hkv"], args["d"], args["bs"], args["maxb"],
                       args["maxctx"], args["nblocks"], args["scale"], args["dtype"], args["ws"],
                       args["wsb"], args["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(d=96), 2), (dict(bs=32), 2), (dict(dtype=7), 2), (dict(hq=12, hkv=8), 2),
    (dict(hq=32, hkv=2), 2), (dict(n=-1), 3), (dict(maxb=0), 3), (dict(maxctx=-5), 3),
    (dict(nblocks=0), 3), (dict(q=None), 1), (dict(bt=None), 1), (dict(out=None), 1),
    (dict(maxctx=4000, wsb=10), 4), (dict(maxctx=4000, wsb=1 << 30), 1),
    (dict(maxctx=300, wsb=0), 4),
    (dict(n=0, q=None), 0),
])
def test_decode_host_errors(over, status):
    assert _decode(**over) == status


def test_write_kv_host_errors():
    w = L.pa_write_kv
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 8, 100, 16, 64, pa.PA_BF16, None) == 2
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 8, 128, 8, 64, pa.PA_BF16, None) == 2
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 16, 64, pa.PA_BF16, None) == 3
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 0, 128, 16, 64, pa.PA_BF16, None) == 3
    assert w(None, FAKE, FAKE, FAKE, FAKE, 10, 8, 128, 16, 64, pa.PA_BF16, None) == 1
    assert w(FAKE, FAKE, FAKE, FAKE, None, 10, 8, 128, 16, 64, pa.PA_F32, None) == 1
    assert w(None, None, None, None, None, 0, 8, 128, 16, 64, pa.PA_F32, None) == 0


def test_slot_mapping_host_errors():
    s = L.pa_build_slot_mapping
    assert s(FAKE, FAKE, FAKE, FAKE, 4, 10, 8, 32, None) == 2
    assert s(FAKE, FAKE, FAKE, FAKE, -1, 10, 8, 16, None) == 3
    assert s(None, FAKE, FAKE, FAKE, 4, 10, 8, 16, None) == 1
    assert s(FAKE, FAKE, FAKE, FAKE, 4, 10, 0, 16, None) == 3
    assert s(None, None, None, None, 0, 0, 8, 16, None) == 0


@pytest.mark.parametrize("rows", [None, -1, 0, 3])
def test_varlen_host_errors(rows):
    """pa_varlen_prefill and pa_varlen_prefill_ex (any single-row count)
    refuse the same host-visible faults before launching anything."""
    def call(dtype=pa.PA_BF16, d=128, ws=FAKE, wsb=1 << 30, q=FAKE, n=4, total=40, maxq=20):
        if rows is None:
            return L.pa_varlen_prefill(FAKE, q, FAKE, FAKE, FAKE, FAKE, FAKE, n, total, maxq, 600,
                                       32, 8, d, 16, 64, 1000, 0.1, dtype, ws, wsb, None)
        return L.pa_varlen_prefill_ex(FAKE, q, FAKE, FAKE, FAKE, FAKE, FAKE, n, total, maxq, 600,
                                      32, 8, d, 16, 64, 1000, 0.1, dtype, rows, ws, wsb, None)
    assert call(dtype=7) == 2
    assert call(d=80) == 2
    assert call(dtype=pa.PA_F32, q=None) == 1   # fp32 is supported: the pointer check decides
    assert call(q=None) == 1
    assert call(wsb=16) == 4
    assert call(ws=None) == 1
    assert call(n=-2) == 3
    assert call(n=0, q=None) == 0


def test_cascade_workspace_size():
    ws = L.pa_cascade_workspace_size
    dec = L.pa_decode_workspace_size
    # no common prefix, or a type without the matrix-core pass: pa_decode's size
    assert ws(4, 8, 2, 128, 513, 0, pa.PA_BF16) == dec(4, 8, 128, 513, pa.PA_BF16)
    assert ws(4, 8, 2, 128, 513, 8, pa.PA_F32) == dec(4, 8, 128, 513, pa.PA_F32)
    assert ws(4, 8, 2, 64, 513, 8, pa.PA_BF16) == dec(4, 8, 64, 513, pa.PA_BF16)
    # 8 prefix blocks = 128 keys = at most 2 prefix splits, then the rest of
    # a 300-token context in one 256-token partition: 3 slots of (m, l, acc[128])
    # per (seq, q head), the item count and the (seq, partition) list
    assert ws(4, 8, 2, 128, 300, 8, pa.PA_BF16) == 4 * 8 * 3 * 130 * 4 + 8 + 4 * 3 * 8
    # a context that fits one partition still needs partial slots
    assert dec(4, 8, 128, 200, pa.PA_BF16) == 0 and ws(4, 8, 2, 128, 200, 4, pa.PA_BF16) > 0
    assert ws(4, 8, 2, 128, 300, -1, pa.PA_BF16) == 0


def test_cascade_host_errors():
    def call(p=4, dtype=pa.PA_BF16, d=128, q=FAKE, n=4, ws=FAKE, wsb=1 << 30, maxb=8):
        return L.pa_cascade_decode(FAKE, q, FAKE, FAKE, FAKE, FAKE, n, 8, 2, d, 16, maxb, 300,
                                   64, p, 0.1, dtype, ws, wsb, None)
    assert call(dtype=7) == 2
    assert call(d=96) == 2
    assert call(p=-1) == 3
    assert call(p=9) == 3          # more common blocks than a table row holds
    assert call(n=-1) == 3
    assert call(q=None) == 1
    assert call(wsb=16) == 4
    assert call(ws=None) == 1
    assert call(n=0, q=None) == 0


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        pa.decode(torch.zeros(1, 1, 64), torch.zeros(1, 1, 16, 64), torch.zeros(1, 1, 16, 64),
                  torch.zeros(1, 1, dtype=torch.int32), torch.ones(1, dtype=torch.int32), 1)


def test_swap_blocks_rejects_pageable_host_tensors():
    """pa_swap_blocks reaches host memory only when it is pinned: the binding
    refuses plain host tensors before calling the library."""
    import torch
    with pytest.raises(ValueError):
        pa.swap_blocks(torch.zeros(4, 2, 16, 8), torch.zeros(4, 2, 16, 8),
                       torch.zeros(1, 2, dtype=torch.int64))


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), -float("inf")])
def test_attention_calls_refuse_non_finite_scale(scale):
    """A NaN or infinite softmax scale defines no weights: every attention
    call refuses it with PA_ERR_INVALID_ARGUMENT before launching anything
    (any finite scale, zero and negative included, is taken)."""
    assert _decode(scale=scale) == 3
    assert L.pa_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 2, 128, 16, 8,
                            100, 64, scale, pa.PA_BF16, None, 0, None) == 3
    assert L.pa_cascade_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 2, 128, 16, 8, 300, 64,
                               4, scale, pa.PA_BF16, FAKE, 1 << 30, None) == 3
    assert L.pa_varlen_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 40, 20, 600, 32, 8,
                               128, 16, 64, 1000, scale, pa.PA_BF16, FAKE, 1 << 30, None) == 3
    assert L.pa_varlen_prefill_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 40, 20, 600, 32,
                                  8, 128, 16, 64, 1000, scale, pa.PA_BF16, 0, FAKE, 1 << 30,
                                  None) == 3
