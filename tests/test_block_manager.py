"""CPU tests of the host-side block manager (include/pa_blocks.h).

Pins: the pages' worked values (ceil(17/16) = 2 blocks; the 16 / 8 / 0 block
table and its slots, tests/golden/), the oracle's own slot mapping for the
metadata a step is built from, and a brute-force model of the documented
rules (FIFO free queue, reference counts, whole-block prefix sharing,
nothing changed by a failing call) driven through random operation
sequences."""
import collections
import json
import os

import numpy as np
import pytest

import oracle
import paged_kv_cache_token_amd as pa
from conftest import GOLDEN, route_block_manager

# under test_block_manager_sanitized.py: the pa_bm_* calls go to the
# AddressSanitizer / UndefinedBehaviorSanitizer build of pa_blocks.cpp
route_block_manager(pa)


def test_allocate_slots_worked_example():
    """[VI] allocate_slots: 17 new tokens need ceil(17/16) = 2 blocks."""
    g = json.load(open(os.path.join(GOLDEN, "allocate_slots_worked_example.json")))
    for case in g["cases"]:
        bm = pa.BlockManager(8, g["block_size"])
        assert bm.allocate_slots(7, case["new_tokens"])
        assert bm.info(7) == (case["new_tokens"], case["blocks"])
        assert bm.num_free_blocks == 8 - case["blocks"]


def test_block_table_example_16_8_0():
    """[KW] §1.2: a request of 24 tokens whose table holds blocks 1, 2, 3 with
    16, 8 and 0 tokens; its slots, the next token's and position 32's."""
    g = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    bm = pa.BlockManager(8)
    assert bm.allocate_slots(100, 1)          # another request takes block 0
    # 24 tokens plus room for 9 more: ceil(33/16) = 3 blocks, filled 16 / 8 / 0
    assert bm.allocate_slots(1, g["expected"]["length"], num_lookahead_tokens=9)
    assert list(bm.block_table(1)) == g["table"]
    tokens, blocks = bm.info(1)
    per_block = [min(max(tokens - 16 * i, 0), 16) for i in range(blocks)]
    assert per_block == g["tokens_per_block"]
    st = bm.build_step([1], [tokens], max_blocks_per_seq=4)
    assert list(st["slot_mapping"]) == g["expected"]["slots_of_positions_0_to_23"]
    assert bm.allocate_slots(1, 1)            # the next token: no new block needed
    assert bm.info(1) == (25, 3)
    assert list(bm.build_step([1], [1], 4)["slot_mapping"]) == [g["expected"]["slot_of_next_token_position_24"]]
    assert bm.allocate_slots(1, 8)            # grow to position 32
    assert list(bm.build_step([1], [1], 4)["slot_mapping"]) == [g["expected"]["slot_of_position_32_after_growth"]]


def test_failed_allocation_changes_nothing():
    bm = pa.BlockManager(4)
    assert bm.allocate_slots(1, 40)           # 3 blocks
    before = (bm.num_free_blocks, bm.info(1), [bm.refcount(b) for b in range(4)])
    assert not bm.allocate_slots(1, 40)       # needs 3 more, 1 free
    assert not bm.allocate_slots(2, 17)       # a new sequence needing 2
    assert (bm.num_free_blocks, bm.info(1), [bm.refcount(b) for b in range(4)]) == before
    with pytest.raises(pa.PAError):
        bm.info(2)                            # the refused sequence was not created


def test_allocate_batch_equals_one_by_one():
    """pa_bm_allocate_batch serves sequences in order exactly as one call per
    sequence, and stops at the first the free queue cannot serve, leaving it
    and the rest untouched."""
    rng = np.random.default_rng(9)
    ids = [5, 1, 9, 2, 7, 3]
    new = rng.integers(1, 40, size=len(ids))
    a, b = pa.BlockManager(64), pa.BlockManager(64)
    assert a.allocate_batch(ids, new) == len(ids)
    for i, k in zip(ids, new):
        assert b.allocate_slots(i, int(k))
    for i in ids:
        assert a.info(i) == b.info(i) and list(a.block_table(i)) == list(b.block_table(i))
    assert a.num_free_blocks == b.num_free_blocks
    # a short queue: 3 free blocks, asks of 1, 2, 2 blocks -> the first two served
    c = pa.BlockManager(3)
    assert c.allocate_batch([0, 1, 2], [16, 17, 20]) == 2
    assert c.info(0) == (16, 1) and c.info(1) == (17, 2) and c.num_free_blocks == 0
    with pytest.raises(pa.PAError):
        c.info(2)
    assert c.allocate_batch([], []) == 0
    d = pa.BlockManager(8)
    with pytest.raises(pa.PAError):
        d.allocate_batch([0, 1], [1, -1])    # an invalid count: the ones before it are served
    assert d.info(0) == (1, 1) and d.num_free_blocks == 7


def test_free_returns_blocks_fifo():
    bm = pa.BlockManager(6)
    assert bm.allocate_slots(1, 32)           # blocks 0, 1
    assert bm.allocate_slots(2, 16)           # block 2
    bm.free(1)                                # queue: 3, 4, 5, 0, 1
    assert bm.num_free_blocks == 5
    assert bm.allocate_slots(3, 16 * 5)
    assert list(bm.block_table(3)) == [3, 4, 5, 0, 1]


def test_prefix_sharing_refcounts():
    """[KW] §1.3: blocks of a common prefix referenced read-only by several
    tables; [KW] §2.1: a block returns to the pool when its last user goes."""
    bm = pa.BlockManager(16)
    assert bm.allocate_slots(1, 40)           # blocks 0, 1, 2 (2 partial)
    bm.share_prefix(1, 2, 40)                 # whole blocks only: 0, 1
    assert bm.info(2) == (32, 2)
    assert list(bm.block_table(2)) == [0, 1]
    assert [bm.refcount(b) for b in range(3)] == [2, 2, 1]
    assert bm.allocate_slots(2, 8)            # dst's own third block
    assert list(bm.block_table(2)) == [0, 1, 3]
    free0 = bm.num_free_blocks
    bm.free(1)                                # only the private block 2 returns
    assert bm.num_free_blocks == free0 + 1
    assert [bm.refcount(b) for b in range(4)] == [1, 1, 0, 1]
    bm.free(2)
    assert bm.num_free_blocks == 16
    with pytest.raises(pa.PAError):
        bm.share_prefix(5, 6, 1)              # unknown source
    assert bm.allocate_slots(7, 20)
    with pytest.raises(pa.PAError):
        bm.share_prefix(7, 7, 16)             # onto itself
    with pytest.raises(pa.PAError):
        bm.share_prefix(7, 8, 21)             # past the source's tokens


def test_build_step_matches_oracle_slot_mapping():
    """The metadata of a packed step: the oracle's slot mapping over the
    built block tables / offsets gives the same slots."""
    rng = np.random.default_rng(5)
    bm = pa.BlockManager(400)
    ids = list(range(10, 22))
    ctx = rng.integers(0, 200, size=len(ids))
    for s, c in zip(ids, ctx):
        assert bm.allocate_slots(s, int(c))
    q = rng.integers(0, 40, size=len(ids))
    for s, l in zip(ids, q):
        assert bm.allocate_slots(s, int(l))
    st = bm.build_step(ids, q, max_blocks_per_seq=20)
    assert list(st["cu_seqlens"]) == [0] + list(np.cumsum(q))
    assert list(st["context_offsets"]) == list(ctx)
    assert list(st["context_lens"]) == list(ctx + q)
    want = oracle.slot_mapping(st["block_tables"], st["cu_seqlens"], st["context_offsets"])
    assert np.array_equal(st["slot_mapping"], want)
    for i, s in enumerate(ids):
        row = st["block_tables"][i]
        nb = bm.info(s)[1]
        assert list(row[:nb]) == list(bm.block_table(s)) and (row[nb:] == -1).all()


def test_error_cases():
    with pytest.raises(pa.PAError):
        pa.BlockManager(0)
    with pytest.raises(pa.PAError):
        pa.BlockManager(8, block_size=32)
    bm = pa.BlockManager(8)
    with pytest.raises(pa.PAError):
        bm.allocate_slots(1, -1)
    with pytest.raises(pa.PAError):
        bm.free(1)
    assert bm.allocate_slots(1, 40)
    with pytest.raises(pa.PAError):
        bm.build_step([1], [41], 4)           # more new tokens than the sequence has
    with pytest.raises(pa.PAError):
        bm.build_step([1], [1], 2)            # table longer than the row
    assert bm.refcount(-1) == -1 and bm.refcount(8) == -1


_OOM_SCRIPT = r"""
import resource, sys
sys.path.insert(0, sys.argv[1])
import paged_kv_cache_token_amd as pa

def vm_bytes():
    for line in open("/proc/self/status"):
        if line.startswith("VmSize:"):
            return int(line.split()[1]) * 1024

def status_of(f):
    try:
        f()
    except pa.PAError as e:
        return e.status
    return 0

bm = pa.BlockManager(1 << 26)
assert bm.allocate_slots(1, 100)
free0 = bm.num_free_blocks
# from here on, at most 64 MiB more address space
resource.setrlimit(resource.RLIMIT_AS, (vm_bytes() + (64 << 20), resource.RLIM_INFINITY))
big = ((1 << 26) - 64) * 16      # tokens whose block list needs ~256 MiB
assert status_of(lambda: pa.BlockManager((1 << 31) - 1)) == pa.PA_ERR_HOST_MEMORY
assert status_of(lambda: bm.allocate_slots(2, big)) == pa.PA_ERR_HOST_MEMORY   # a new sequence
assert status_of(lambda: bm.info(2)) == 3                                        # not created
assert status_of(lambda: bm.allocate_slots(1, big)) == pa.PA_ERR_HOST_MEMORY   # a longer list
assert bm.info(1) == (100, 7) and bm.num_free_blocks == free0                    # nothing changed
assert bm.allocate_slots(3, 40) and bm.info(3) == (40, 3)                        # still usable
print("ok")
"""


def test_host_allocation_failure_changes_nothing():
    """Under an address-space limit (a child process), creating a huge manager
    and growing a block list fail with PA_ERR_HOST_MEMORY instead of letting
    a C++ exception out, and the manager is left as it was."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _OOM_SCRIPT, root], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


class Model:
    """Brute-force model of the documented rules."""

    def __init__(self, n):
        self.free = collections.deque(range(n))
        self.ref = [0] * n
        self.seqs = {}

    def allocate(self, s, new, look):
        tokens, blocks = self.seqs.get(s, (0, []))
        need = -(-(tokens + new + look) // 16) - len(blocks)
        if need > len(self.free):
            return False
        blocks = list(blocks)
        for _ in range(max(need, 0)):
            b = self.free.popleft()
            self.ref[b] = 1
            blocks.append(b)
        self.seqs[s] = (tokens + new, blocks)
        return True

    def share(self, src, dst, n):
        tokens, blocks = self.seqs[src]
        full = n // 16
        for b in blocks[:full]:
            self.ref[b] += 1
        self.seqs[dst] = (16 * full, list(blocks[:full]))

    def release(self, s):
        for b in self.seqs.pop(s)[1]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)


def test_random_operations_match_model():
    rng = np.random.default_rng(11)
    n = 64
    bm, model = pa.BlockManager(n), Model(n)
    next_id = 0
    for _ in range(600):
        live = list(model.seqs)
        op = rng.integers(0, 4)
        if op == 0 or not live:
            s = next_id if (not live or rng.random() < 0.5) else int(rng.choice(live))
            next_id += s == next_id
            new, look = int(rng.integers(0, 70)), int(rng.integers(0, 20))
            assert bm.allocate_slots(s, new, look) == model.allocate(s, new, look)
        elif op == 1:
            s = int(rng.choice(live))
            model.release(s)
            bm.free(s)
        elif op == 2:
            src = int(rng.choice(live))
            n_tok = int(rng.integers(0, model.seqs[src][0] + 1))
            dst = next_id
            next_id += 1
            bm.share_prefix(src, dst, n_tok)
            model.share(src, dst, n_tok)
        else:
            ids = [int(x) for x in rng.choice(live, size=min(len(live), 5), replace=False)]
            q = [int(rng.integers(0, model.seqs[s][0] + 1)) for s in ids]
            maxb = max(len(model.seqs[s][1]) for s in ids) + 1
            st = bm.build_step(ids, q, maxb)
            want = oracle.slot_mapping(st["block_tables"], st["cu_seqlens"], st["context_offsets"])
            assert np.array_equal(st["slot_mapping"], want)
        assert bm.num_free_blocks == len(model.free)
        assert [bm.refcount(b) for b in range(n)] == model.ref
        for s, (tokens, blocks) in model.seqs.items():
            assert bm.info(s) == (tokens, len(blocks))
            assert list(bm.block_table(s)) == blocks
