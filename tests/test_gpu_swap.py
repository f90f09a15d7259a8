"""GPU parity of pa_swap_blocks against the oracle's block copy, bit for bit:
swap out (device -> pinned host), swap in (pinned host -> device), copies
inside one device pool, pair lists in pinned host memory, out-of-range
pairs skipped, NaN canaries of untouched blocks intact."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_token_amd as pa

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16 if t.element_size() == 2 else torch.int32).numpy().copy()


def _pool(n, hkv, d, dtype, seed, device, pinned=False):
    g = torch.Generator(device="cpu").manual_seed(seed)
    t = torch.randn(n, hkv, 16, d, generator=g).to(dtype)
    if pinned:
        return t.pin_memory()
    return t.to(device)


@pytest.mark.parametrize("dtype,hkv,d", [(torch.bfloat16, 8, 128), (torch.float32, 4, 64)])
def test_swap_out_and_in(gpu, dtype, hkv, d):
    say("swap", dtype, hkv, d)
    rng = np.random.default_rng(41)
    dev_pool = _pool(300, hkv, d, dtype, 1, "cuda")
    host_pool = torch.full((120, hkv, 16, d), float("nan"), dtype=dtype).pin_memory()
    src_ids = rng.choice(300, size=100, replace=False)
    dst_ids = rng.choice(120, size=100, replace=False)
    pairs = np.stack([src_ids, dst_ids], 1).astype(np.int64)
    pairs = np.concatenate([pairs, [[-1, 3], [5, 120], [300, 0]]])  # skipped
    want = _bits(host_pool)
    oracle.swap_blocks(want, _bits(dev_pool), pairs)
    pa.swap_blocks(host_pool, dev_pool, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(host_pool), want), "swap out differs"

    # swap in from the host copies into fresh device blocks; pairs in pinned memory
    back = torch.full((200, hkv, 16, d), float("nan"), dtype=dtype, device="cuda")
    in_pairs = np.stack([dst_ids, rng.choice(200, size=100, replace=False)], 1).astype(np.int64)
    want = _bits(back)
    oracle.swap_blocks(want, _bits(host_pool), in_pairs)
    pa.swap_blocks(back, host_pool, torch.from_numpy(in_pairs).pin_memory())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(back), want), "swap in differs"


def test_copy_inside_one_pool(gpu):
    say("copy inside one pool")
    rng = np.random.default_rng(42)
    pool = _pool(500, 8, 128, torch.bfloat16, 2, "cuda")
    ids = rng.permutation(500)
    pairs = np.stack([ids[:150], ids[150:300]], 1).astype(np.int64)  # disjoint sources / targets
    want = _bits(pool)
    oracle.swap_blocks(want, want.copy(), pairs)
    pa.swap_blocks(pool, pool, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(pool), want)


def test_empty_and_errors(gpu):
    pool = _pool(4, 2, 64, torch.float32, 3, "cuda")
    pa.swap_blocks(pool, pool, torch.zeros(0, 2, dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError):
        pa.swap_blocks(pool, torch.zeros(4, 2, 16, 64), torch.zeros(1, 2, dtype=torch.int64,
                                                                   device="cuda"))
    with pytest.raises(ValueError):
        pa.swap_blocks(pool, _pool(4, 2, 32, torch.float32, 3, "cuda"),
                       torch.zeros(1, 2, dtype=torch.int64, device="cuda"))
