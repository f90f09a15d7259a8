"""The block manager's step metadata drives the device path: the slot
mapping pa_build_slot_mapping computes on the GPU from the manager's block
tables equals the manager's own, and a decode over a cache written through
those slots matches the oracle over the same pools."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_token_amd as pa

pytestmark = pytest.mark.gpu


def test_manager_metadata_on_device(gpu):
    print("[case] block manager -> device slot mapping + decode", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(31)
    hkv, hq, d = 4, 8, 128
    bm = pa.BlockManager(300)
    ids = list(range(12))
    prompt = rng.integers(1, 300, size=len(ids))
    bm.allocate_slots(100, 50)                      # an unrelated request holds blocks first
    for s, p in zip(ids, prompt):
        assert bm.allocate_slots(s, int(p))
    bm.free(100)
    bm.share_prefix(0, 50, int(prompt[0]))          # a request forked from sequence 0
    ids.append(50)
    for s in ids:
        assert bm.allocate_slots(s, 1)              # one decode token each
    maxb = max(bm.info(s)[1] for s in ids)
    st = bm.build_step(ids, [1] * len(ids), maxb)
    hist = bm.build_step(ids, [bm.info(s)[0] for s in ids], maxb)   # every token ever stored

    dev = torch.device("cuda")
    bt = torch.from_numpy(hist["block_tables"]).to(dev)
    slots = pa.build_slot_mapping(torch.from_numpy(hist["cu_seqlens"]).to(dev),
                                  torch.zeros(len(ids), dtype=torch.int32, device=dev), bt,
                                  int(hist["cu_seqlens"][-1]))
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), hist["slot_mapping"])
    step_slots = pa.build_slot_mapping(torch.from_numpy(st["cu_seqlens"]).to(dev),
                                       torch.from_numpy(st["context_offsets"]).to(dev), bt, len(ids))
    torch.cuda.synchronize()
    assert np.array_equal(step_slots.cpu().numpy(), st["slot_mapping"])

    # the forked request shares sequence 0's whole prompt blocks: write each
    # slot once (a shared slot holds one token, written by its owner)
    slot_all = hist["slot_mapping"]
    uniq, first = np.unique(slot_all, return_index=True)
    g = torch.Generator(device="cpu").manual_seed(31)
    total = slot_all.shape[0]
    k = torch.randn(total, hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(total, hkv, d, generator=g).to(torch.bfloat16)
    kc = torch.full((300, hkv, 16, d), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full_like(kc, float("nan"))
    rows = torch.from_numpy(first).long()
    pa.write_kv(k[rows].to(dev), v[rows].to(dev), kc, vc, torch.from_numpy(uniq).to(dev))
    q = torch.randn(len(ids), hq, d, generator=g).to(torch.bfloat16)
    lens = torch.from_numpy(hist["context_lens"]).to(dev)
    out = pa.decode(q.to(dev), kc, vc, bt, lens, int(lens.max()), d ** -0.5)
    torch.cuda.synchronize()
    want = oracle.decode(q.view(torch.int16).numpy().view(np.uint16),
                         kc.cpu().view(torch.int16).numpy().view(np.uint16),
                         vc.cpu().view(torch.int16).numpy().view(np.uint16),
                         hist["block_tables"], hist["context_lens"], d ** -0.5)
    err = float(np.abs(out.float().cpu().numpy() - want).max())
    print("[case] max abs err", err, flush=True)
    assert err <= 2e-2
