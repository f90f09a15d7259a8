"""Pins for the CPU oracle: it is checked against things other than itself.

* the pages' printed values (tests/golden/*.json, each with its citation):
  ceil(17/16) = 2 blocks; the 16 / 8 / 0 block-table example;
* hand-written expected layouts for the slot/cache/gather conventions;
* brute force: pure-Python loops over the unpaged K/V on tiny inputs;
* a library routine: torch's scaled_dot_product_attention in float64 on the
  CPU (with its own grouped-query head mapping) on the unpaged K/V;
* closed forms: one key -> V[0]; q = 0 or equal keys -> mean(V); two keys ->
  logistic weights;
* invariants the pages fix: physical placement, read-only sharing, ignored
  tail entries and slots, super-sequence isolation and chunking.

The last test plants plausible mistakes in the oracle (on the CPU) and checks
that each one is caught by at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.paged_attention as opa
from conftest import GOLDEN

BS = 16


# --------------------------------------------------------------------------
# small helpers (test data only; no oracle arithmetic)
# --------------------------------------------------------------------------

def _rand_case(seed, lens, hq, hkv, d, pool_extra=5):
    """Logical (unpaged) K/V per sequence, q, and a random paged placement."""
    rng = np.random.default_rng(seed)
    need = [-(-n // BS) for n in lens]
    pool = sum(need) + pool_extra
    perm = rng.permutation(pool)
    maxb = max(need) + 2
    bt = np.zeros((len(lens), maxb), np.int32)
    cur = 0
    for i, nb in enumerate(need):
        bt[i, :nb] = perm[cur:cur + nb]
        bt[i, nb:] = rng.integers(0, pool, size=maxb - nb)  # in-range garbage tail
        cur += nb
    ks = [rng.standard_normal((n, hkv, d)) for n in lens]
    vs = [rng.standard_normal((n, hkv, d)) for n in lens]
    return dict(pool=pool, bt=bt, ks=ks, vs=vs, lens=np.array(lens), hq=hq, hkv=hkv, d=d)


def _paged(case, dtype=np.float64):
    """Pool built through the oracle's own slot mapping and write (pinned
    separately below against hand-written layouts)."""
    hkv, d = case["hkv"], case["d"]
    kc = np.full((case["pool"], hkv, BS, d), np.nan, dtype)
    vc = np.full((case["pool"], hkv, BS, d), np.nan, dtype)
    lens = case["lens"]
    cu = np.concatenate([[0], np.cumsum(lens)])
    slots = oracle.slot_mapping(case["bt"], cu, np.zeros(len(lens), np.int64))
    key = np.concatenate(case["ks"]).astype(dtype) if len(lens) else np.zeros((0, hkv, d))
    val = np.concatenate(case["vs"]).astype(dtype) if len(lens) else np.zeros((0, hkv, d))
    oracle.write_kv(kc, vc, key, val, slots)
    return kc, vc


def _brute_attention(qrow, k, v, n, scale, hq, hkv):
    """Pure-Python loops: out[h][e] = sum_t w_t v[t][kv(h)][e], w = softmax."""
    d = len(qrow[0])
    out = []
    g = hq // hkv
    for h in range(hq):
        kv = h // g
        if n == 0:
            out.append([0.0] * d)
            continue
        s = []
        for t in range(n):
            acc = 0.0
            for e in range(d):
                acc += float(qrow[h][e]) * float(k[t][kv][e])
            s.append(acc * scale)
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = sum(w)
        row = []
        for e in range(d):
            acc = 0.0
            for t in range(n):
                acc += w[t] * float(v[t][kv][e])
            row.append(acc / z)
        out.append(row)
    return np.array(out)


def _sdpa(q_rows, k, v, visible, scale):
    """torch SDPA (float64, CPU) with an explicit visibility mask and grouped
    query heads; q_rows [R, Hq, d], k/v [L, Hkv, d]."""
    qt = torch.from_numpy(q_rows).permute(1, 0, 2).unsqueeze(0)        # [1, Hq, R, d]
    kt = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0)             # [1, Hkv, L, d]
    vt = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0)
    mask = torch.arange(k.shape[0])[None, :] < torch.from_numpy(np.asarray(visible))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


# --------------------------------------------------------------------------
# pins (plain functions so the mutation test can rerun them)
# --------------------------------------------------------------------------

def pin_allocate_slots_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "allocate_slots_worked_example.json")))
    for c in g["cases"]:
        assert opa.blocks_needed(c["new_tokens"], g["block_size"]) == c["blocks"]


def pin_blocks_needed_closed_form():
    # exact fill, one over, partial last block, empty
    for n, want in [(0, 0), (1, 1), (15, 1), (16, 1), (17, 2), (32, 2), (33, 3), (100, 7)]:
        assert opa.blocks_needed(n) == want, n
    assert [opa.blocks_needed(n) for n in (1, 16, 17, 100)] == [1, 1, 2, 7]


def pin_block_table_example():
    g = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    table = np.array([g["table"]], np.int32)
    length = sum(g["tokens_per_block"])
    exp = g["expected"]
    assert length == exp["length"]
    assert opa.blocks_needed(length, g["block_size"]) == exp["live_blocks"]
    slots = opa.slot_mapping(table, np.array([0, length]), np.array([0]))
    assert slots.tolist() == exp["slots_of_positions_0_to_23"]
    nxt = opa.slot_mapping(table, np.array([0, 1]), np.array([length]))
    assert nxt.tolist() == [exp["slot_of_next_token_position_24"]]
    grown = opa.slot_mapping(table, np.array([0, 1]), np.array([32]))
    assert grown.tolist() == [exp["slot_of_position_32_after_growth"]]


def pin_slot_mapping_packed_layout():
    # two sequences packed: seq 0 brings 3 tokens at positions 14..16 (crossing
    # a block edge), seq 1 brings 1 token at position 0.
    bt = np.array([[7, 2, 9], [4, 0, 0]], np.int32)
    slots = opa.slot_mapping(bt, np.array([0, 3, 4]), np.array([14, 0]))
    assert slots.tolist() == [7 * 16 + 14, 7 * 16 + 15, 2 * 16 + 0, 4 * 16 + 0]


def pin_write_kv_layout():
    kc = np.full((4, 2, BS, 3), -1.0, np.float32)
    vc = np.full((4, 2, BS, 3), -2.0, np.float32)
    key = np.arange(4 * 2 * 3, dtype=np.float32).reshape(4, 2, 3)
    val = 1000 + key
    # token 1 is padding (slot -1): nothing may be stored for it anywhere
    opa.write_kv(kc, vc, key, val, np.array([17, -1, 3, 62]))
    want_k = np.full_like(kc, -1.0)
    want_v = np.full_like(vc, -2.0)
    want_k[1, :, 1, :] = key[0]
    want_k[0, :, 3, :] = key[2]
    want_k[3, :, 14, :] = key[3]
    want_v[1, :, 1, :] = val[0]
    want_v[0, :, 3, :] = val[2]
    want_v[3, :, 14, :] = val[3]
    assert np.array_equal(kc, want_k) and np.array_equal(vc, want_v)


def pin_write_kv_bits():
    # bf16 patterns incl. a NaN payload and negative zero are copied bit for bit
    kc = np.full((2, 1, BS, 4), 0x7FC1, np.uint16)
    vc = kc.copy()
    key = np.array([[[0x7FA5, 0x8000, 0x3F80, 0x0001]]], np.uint16)
    opa.write_kv(kc, vc, key, key, np.array([16 + 5]))
    assert kc[1, 0, 5].tolist() == [0x7FA5, 0x8000, 0x3F80, 0x0001]
    assert (kc[0] == 0x7FC1).all() and (np.delete(kc[1, 0], 5, axis=0) == 0x7FC1).all()


def pin_swap_blocks_layout():
    # block b of a pool holds 10*b + 0.5 in every element; pairs move them by
    # hand-picked ids, one out-of-range pair is skipped, untouched blocks stay
    src = np.zeros((3, 2, BS, 2))
    for b in range(3):
        src[b] = 10 * b + 0.5
    dst = np.full((4, 2, BS, 2), -1.0)
    opa.swap_blocks(dst, src, np.array([[2, 0], [0, 3], [1, 9], [7, 1]]))
    assert (dst[0] == 20.5).all() and (dst[3] == 0.5).all()
    assert (dst[1] == -1.0).all() and (dst[2] == -1.0).all()
    # bit copy of bf16 patterns inside one pool (NaN payload, -0)
    pool = np.zeros((2, 1, BS, 2), np.uint16)
    pool[0, 0, 3] = [0x7FA5, 0x8000]
    opa.swap_blocks(pool, pool, np.array([[0, 1]]))
    assert pool[1, 0, 3].tolist() == [0x7FA5, 0x8000] and (pool[1, 0, :3] == 0).all()


def _cascade_case(seed=11):
    """Three sequences sharing their first 2 physical blocks (32 tokens) and a
    fourth whose context (14 tokens) ends inside them; private blocks and a
    garbage tail after each row's live entries.  Built by hand (no oracle
    code): pool [10, 2, 16, 4] of float64."""
    rng = np.random.default_rng(seed)
    hq, hkv, d = 4, 2, 4
    kc = rng.standard_normal((10, hkv, BS, d))
    vc = rng.standard_normal((10, hkv, BS, d))
    lens = np.array([37, 52, 32, 14])
    bt = np.array([[6, 2, 9, 0, 5],
                   [6, 2, 4, 8, 1],
                   [6, 2, 3, 3, 3],
                   [6, 7, 7, 7, 7]], np.int32)   # row 3: one live block, so entry 1 is dead
    q = rng.standard_normal((4, hq, d))
    return q, kc, vc, bt, lens, hq, hkv, d


def pin_cascade_split_identity():
    # the prefix keys attended on their own and the private rest on their own,
    # combined with weights e^(m_part - M), by brute-force loops over the
    # hand-built pool, equal the cascade result
    q, kc, vc, bt, lens, hq, hkv, d = _cascade_case()
    scale = 0.5
    got = opa.cascade_decode(q, kc, vc, bt, lens, 2, scale)
    g = hq // hkv
    for i, n in enumerate(lens):
        keys = [kc[bt[i, t // BS], :, t % BS] for t in range(n)]
        vals = [vc[bt[i, t // BS], :, t % BS] for t in range(n)]
        for h in range(hq):
            parts = []
            for lo, hi in ((0, min(n, 32)), (32, n)):
                if hi <= lo:
                    continue
                s = [scale * sum(q[i, h, e] * keys[t][h // g][e] for e in range(d))
                     for t in range(lo, hi)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                acc = [sum(w[t - lo] * vals[t][h // g][e] for t in range(lo, hi))
                       for e in range(d)]
                parts.append((m, sum(w), acc))
            big = max(p[0] for p in parts)
            z = sum(math.exp(p[0] - big) * p[1] for p in parts)
            want = [sum(math.exp(p[0] - big) * p[2][e] for p in parts) / z for e in range(d)]
            assert np.allclose(got[i, h], want, rtol=0, atol=1e-12), (i, h)


def pin_cascade_precondition():
    q, kc, vc, bt, lens, hq, hkv, d = _cascade_case()
    # row 3 differs from row 0 only in entry 1, past its one live block: accepted
    opa.cascade_decode(q, kc, vc, bt, lens, 2, 0.5)
    bad = bt.copy()
    bad[1, 1] = 5                                  # a live prefix entry differs

    def rejected(table, p):
        try:
            opa.cascade_decode(q, kc, vc, table, lens, p, 0.5)
        except ValueError:
            return True
        return False
    assert rejected(bad, 2)
    assert rejected(bt, 6)                         # more blocks than the table holds
    # no common prefix: the plain decode
    assert np.array_equal(opa.cascade_decode(q, kc, vc, bad, lens, 0, 0.5),
                          opa.decode(q, kc, vc, bad, lens, 0.5))


def pin_gather_layout():
    # slot value = 100 * physical block + offset, in every head and dim
    cache = np.zeros((3, 2, BS, 2))
    for b in range(3):
        for o in range(BS):
            cache[b, :, o, :] = 100 * b + o
    got = opa.gather(cache, np.array([2, 0, 1]), 20)
    want = [200 + o for o in range(16)] + [0, 1, 2, 3]
    assert got.shape == (20, 2, 2)
    assert got[:, 1, 0].tolist() == want and got[:, 0, 1].tolist() == want


def pin_bruteforce_decode():
    case = _rand_case(11, [1, 5, 16, 17, 37], hq=4, hkv=2, d=8)
    kc, vc = _paged(case)
    q = np.random.default_rng(12).standard_normal((5, 4, 8))
    scale = 0.3
    got = opa.decode(q, kc, vc, case["bt"], case["lens"], scale)
    for i, n in enumerate(case["lens"]):
        want = _brute_attention(q[i].tolist(), case["ks"][i].tolist(), case["vs"][i].tolist(),
                                int(n), scale, 4, 2)
        assert np.abs(got[i] - want).max() < 1e-12, i


def pin_bruteforce_prefill():
    # seq lens = context + chunk; two chunks with context, one plain prefill
    ctx = [0, 9, 20]
    ql = [5, 8, 3]
    case = _rand_case(21, [c + l for c, l in zip(ctx, ql)], hq=2, hkv=1, d=4)
    kc, vc = _paged(case)
    q = np.random.default_rng(22).standard_normal((sum(ql), 2, 4))
    cu = np.concatenate([[0], np.cumsum(ql)])
    scale = 0.7
    got = opa.varlen_prefill(q, kc, vc, cu, np.array(ctx), case["bt"], scale)
    for i in range(3):
        for j in range(ql[i]):
            want = _brute_attention(q[cu[i] + j].tolist(), case["ks"][i].tolist(),
                                    case["vs"][i].tolist(), ctx[i] + j + 1, scale, 2, 1)
            assert np.abs(got[i][j] - want).max() < 1e-12, (i, j)


def pin_sdpa_library_decode_gqa():
    case = _rand_case(31, [3, 16, 40, 70], hq=8, hkv=2, d=16)
    kc, vc = _paged(case)
    q = np.random.default_rng(32).standard_normal((4, 8, 16))
    got = opa.decode(q, kc, vc, case["bt"], case["lens"], 0.25)
    for i, n in enumerate(case["lens"]):
        want = _sdpa(q[i:i + 1], case["ks"][i], case["vs"][i], [n], 0.25)[0]
        assert np.abs(got[i] - want).max() < 1e-12, i


def pin_sdpa_library_prefill():
    ctx, ql = [0, 13, 31], [17, 4, 20]
    case = _rand_case(41, [c + l for c, l in zip(ctx, ql)], hq=4, hkv=4, d=8)
    kc, vc = _paged(case)
    q = np.random.default_rng(42).standard_normal((sum(ql), 4, 8))
    cu = np.concatenate([[0], np.cumsum(ql)])
    got = opa.varlen_prefill(q, kc, vc, cu, np.array(ctx), case["bt"], 0.35)
    for i in range(3):
        vis = ctx[i] + np.arange(ql[i]) + 1
        want = _sdpa(q[cu[i]:cu[i + 1]], case["ks"][i], case["vs"][i], vis, 0.35)
        assert np.abs(got[i] - want).max() < 1e-12, i


def pin_closed_forms():
    rng = np.random.default_rng(51)
    case = _rand_case(52, [1, 9, 9, 2], hq=2, hkv=2, d=6)
    # seq 2: all keys equal; seq 3: two keys
    case["ks"][2][:] = case["ks"][2][0]
    kc, vc = _paged(case)
    q = rng.standard_normal((4, 2, 6))
    q[1] = 0.0
    scale = 0.5
    got = opa.decode(q, kc, vc, case["bt"], case["lens"], scale)
    assert np.array_equal(got[0], case["vs"][0][0])                     # one key -> V[0]
    assert np.abs(got[1] - case["vs"][1].mean(axis=0)).max() < 1e-14   # q = 0 -> mean V
    assert np.abs(got[2] - case["vs"][2].mean(axis=0)).max() < 1e-14   # equal keys -> mean V
    k3, v3 = case["ks"][3], case["vs"][3]
    for h in range(2):
        s0 = scale * k3[0, h] @ q[3, h]
        s1 = scale * k3[1, h] @ q[3, h]
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        want = p0 * v3[0, h] + (1 - p0) * v3[1, h]
        assert np.abs(got[3, h] - want).max() < 1e-14


def pin_zero_context():
    kc = np.full((2, 1, BS, 4), np.nan)
    got = opa.decode(np.ones((1, 2, 4)), kc, kc, np.array([[0]]), np.array([0]), 1.0)
    assert np.array_equal(got, np.zeros((1, 2, 4)))


def pin_placement_invariance():
    case = _rand_case(61, [7, 33, 50], hq=4, hkv=1, d=8)
    q = np.random.default_rng(62).standard_normal((3, 4, 8))
    kc, vc = _paged(case)
    base = opa.decode(q, kc, vc, case["bt"], case["lens"], 0.4)
    # move every physical block to a new random place and relabel the tables
    rng = np.random.default_rng(63)
    perm = rng.permutation(case["pool"])
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = perm[case["bt"]]
    moved = opa.decode(q, kc2, vc2, bt2, case["lens"], 0.4)
    assert np.array_equal(base, moved)


def pin_shared_blocks_invariance():
    # three sequences share two prefix blocks read-only vs private copies
    rng = np.random.default_rng(71)
    hkv, d = 2, 8
    prefix = rng.standard_normal((2, hkv, BS, d))
    priv = rng.standard_normal((3, hkv, BS, d))
    shared_pool = np.concatenate([prefix, priv])                  # blocks 0,1 shared; 2,3,4
    bt_shared = np.array([[0, 1, 2], [0, 1, 3], [0, 1, 4]])
    copies = np.concatenate([prefix, priv[0:1], prefix, priv[1:2], prefix, priv[2:3]])
    bt_copy = np.array([[0, 1, 2], [3, 4, 5], [6, 7, 8]])
    q = rng.standard_normal((3, 4, d))
    lens = np.array([40, 33, 48])
    a = opa.decode(q, shared_pool, shared_pool, bt_shared, lens, 0.3)
    b = opa.decode(q, copies, copies, bt_copy, lens, 0.3)
    assert np.array_equal(a, b)


def pin_ignores_tail_and_unreferenced():
    case = _rand_case(81, [5, 21], hq=2, hkv=2, d=4)
    q = np.random.default_rng(82).standard_normal((2, 2, 4))
    kc, vc = _paged(case)                     # NaN everywhere not written
    got = opa.decode(q, kc, vc, case["bt"], case["lens"], 0.5)
    assert np.isfinite(got).all()
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[np.isnan(kc2)] = 1e30                 # a different garbage value
    vc2[np.isnan(vc2)] = -7.0
    bt2 = case["bt"].copy()
    bt2[:, 2:] = 0                            # different dead table entries
    assert np.array_equal(got, opa.decode(q, kc2, vc2, bt2, case["lens"], 0.5))


def pin_prefill_row_equals_decode():
    ctx, ql = [12], [9]
    case = _rand_case(91, [21], hq=4, hkv=2, d=8)
    kc, vc = _paged(case)
    q = np.random.default_rng(92).standard_normal((9, 4, 8))
    pre = opa.varlen_prefill(q, kc, vc, np.array([0, 9]), np.array(ctx), case["bt"], 0.3)[0]
    for j in range(9):
        dec = opa.decode(q[j:j + 1], kc, vc, case["bt"][:1], np.array([ctx[0] + j + 1]), 0.3)
        assert np.array_equal(pre[j], dec[0]), j


def pin_packing_and_chunking():
    ctx, ql = [0, 5, 40], [30, 1, 11]
    case = _rand_case(101, [c + l for c, l in zip(ctx, ql)], hq=2, hkv=2, d=8)
    kc, vc = _paged(case)
    q = np.random.default_rng(102).standard_normal((sum(ql), 2, 8))
    cu = np.concatenate([[0], np.cumsum(ql)])
    packed = opa.varlen_prefill(q, kc, vc, cu, np.array(ctx), case["bt"], 0.4)
    for i in range(3):                          # each sequence alone
        solo = opa.varlen_prefill(q[cu[i]:cu[i + 1]], kc, vc, np.array([0, ql[i]]),
                                  np.array([ctx[i]]), case["bt"][i:i + 1], 0.4)[0]
        assert np.array_equal(packed[i], solo)
    # sequence 0 split into two chunks of 18 + 12 with the second one after 18 cached
    two = opa.varlen_prefill(q[:30], kc, vc, np.array([0, 18, 30]), np.array([0, 18]),
                             np.stack([case["bt"][0], case["bt"][0]]), 0.4)
    assert np.array_equal(np.concatenate([two[0], two[1]]), packed[0])


def pin_bf16_widening():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F80], np.uint16)
    got = opa.widen(bits)
    assert got[0] == 1.0 and got[1] == -1.0
    assert got[2] == 3.140625                       # 0x4049 -> 3.140625 exactly
    assert got[3] == 2.0 ** -133                    # smallest bf16 subnormal
    assert got[4] == np.inf


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__[4:])
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# --------------------------------------------------------------------------

def _mut_attend(kind):
    def attend(q_rows, k, v, visible, scale):
        r_count, hq, d = q_rows.shape
        hkv = k.shape[1]
        group = hq // hkv
        out = np.zeros((r_count, hq, d))
        for r in range(r_count):
            n = int(visible[r])
            if kind == "drop_last_key":
                n -= 1
            if n <= 0:
                continue
            for h in range(hq):
                kvh = h % hkv if kind == "gqa_modulo" else h // group
                s = (k[:n, kvh] @ q_rows[r, h]) * (1.0 if kind == "no_scale" else scale)
                p = np.exp(s - s.max())
                z = n if kind == "wrong_norm" else p.sum()
                out[r, h] = (p @ v[:n, kvh]) / z
        return out
    return attend


def _mut_varlen_offset(kind):
    def varlen_prefill(q, k_cache, v_cache, cu_seqlens, context_offsets, block_tables,
                       scale, seqs=None, block_size=BS):
        qf = opa.widen(q)
        res = {}
        for i in (range(len(context_offsets)) if seqs is None else seqs):
            lo, hi = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
            c = int(context_offsets[i])
            k = opa.widen(opa.gather(k_cache, block_tables[i], c + hi - lo))
            v = opa.widen(opa.gather(v_cache, block_tables[i], c + hi - lo))
            if kind == "causal_off_by_one":
                vis = c + np.arange(hi - lo)
            elif kind == "ignore_context":
                vis = np.arange(hi - lo) + 1
            else:  # "no_causal"
                vis = np.full(hi - lo, c + hi - lo)
            res[i] = opa.attend(qf[lo:hi], k, v, vis, scale)
        return res
    return varlen_prefill


def _mut_slot_swap(block_tables, cu_seqlens, context_offsets, block_size=BS):
    cu = np.asarray(cu_seqlens, np.int64)
    c = np.asarray(context_offsets, np.int64)
    seq = np.repeat(np.arange(len(c)), cu[1:] - cu[:-1])
    pos = c[seq] + np.arange(int(cu[-1])) - cu[:-1][seq]
    return np.asarray(block_tables)[seq, pos % block_size].astype(np.int64) * block_size + pos // block_size


def _mut_write_no_skip(k_cache, v_cache, key, value, slots, block_size=BS):
    slots = np.asarray(slots, np.int64)
    k_cache[slots // block_size, :, slots % block_size, :] = key
    v_cache[slots // block_size, :, slots % block_size, :] = value


def _mut_swap_reversed(dst, src, block_pairs):
    for s_blk, d_blk in np.asarray(block_pairs, np.int64).reshape(-1, 2):
        if 0 <= d_blk < src.shape[0] and 0 <= s_blk < dst.shape[0]:
            dst[s_blk] = src[d_blk]


def _mut_cascade_checks_dead_entries(q, k_cache, v_cache, block_tables, context_lens,
                                     num_common_prefix_blocks, scale, seqs=None, block_size=BS):
    p = int(num_common_prefix_blocks)
    if (np.asarray(block_tables)[:, :p] != np.asarray(block_tables)[0, :p]).any():
        raise ValueError("prefix differs")
    return opa.decode(q, k_cache, v_cache, block_tables, context_lens, scale, seqs, block_size)


def _mut_cascade_prefix_twice(q, k_cache, v_cache, block_tables, context_lens,
                              num_common_prefix_blocks, scale, seqs=None, block_size=BS):
    # the shared keys counted once more in every row that holds them
    qf = opa.widen(q)
    p = int(num_common_prefix_blocks) * block_size
    out = np.zeros(qf.shape)
    for i, n in enumerate(context_lens):
        n = int(n)
        k = opa.widen(opa.gather(k_cache, block_tables[i], n, block_size))
        v = opa.widen(opa.gather(v_cache, block_tables[i], n, block_size))
        kk = np.concatenate([k[:min(n, p)], k])
        vv = np.concatenate([v[:min(n, p)], v])
        out[i] = opa.attend(qf[i:i + 1], kk, vv, np.array([len(kk)]), scale)[0]
    return out


def _mut_gather_identity(cache, table_row, length, block_size=BS):
    nb = opa.blocks_needed(length, block_size)
    if nb == 0:
        return np.zeros((0, cache.shape[1], cache.shape[3]), cache.dtype)
    seq = np.concatenate([cache[b] for b in range(nb)], axis=1)
    return np.ascontiguousarray(seq[:, :length].transpose(1, 0, 2))


def _mut_gather_transposed(cache, table_row, length, block_size=BS):
    nb = opa.blocks_needed(length, block_size)
    if nb == 0:
        return np.zeros((0, cache.shape[1], cache.shape[3]), cache.dtype)
    seq = np.concatenate([cache[int(b)].transpose(1, 0, 2) for b in table_row[:nb]], axis=1)
    return np.ascontiguousarray(seq[:, :length])


MUTATIONS = {
    "ceil_as_floor": ("blocks_needed", lambda n, block_size=BS: int(n) // block_size),
    "slot_block_offset_swapped": ("slot_mapping", _mut_slot_swap),
    "write_ignores_padding": ("write_kv", _mut_write_no_skip),
    "gather_ignores_table": ("gather", _mut_gather_identity),
    "swap_pair_reversed": ("swap_blocks", _mut_swap_reversed),
    "cascade_checks_dead_entries": ("cascade_decode", _mut_cascade_checks_dead_entries),
    "cascade_prefix_twice": ("cascade_decode", _mut_cascade_prefix_twice),
    "gather_transposed": ("gather", _mut_gather_transposed),
    "attend_no_scale": ("attend", _mut_attend("no_scale")),
    "attend_gqa_modulo": ("attend", _mut_attend("gqa_modulo")),
    "attend_wrong_norm": ("attend", _mut_attend("wrong_norm")),
    "attend_drops_last_key": ("attend", _mut_attend("drop_last_key")),
    "prefill_causal_off_by_one": ("varlen_prefill", _mut_varlen_offset("causal_off_by_one")),
    "prefill_ignores_context": ("varlen_prefill", _mut_varlen_offset("ignore_context")),
    "prefill_not_causal": ("varlen_prefill", _mut_varlen_offset("no_causal")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(opa, attr, fn)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # an assertion, or the mistake breaking a shape
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
