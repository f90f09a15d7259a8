"""The binding refuses arrays whose shapes disagree with the counts it passes
to the library (the kernels index every array by those counts, so a shorter
array would be read or written past its end).  Every case raises before any
launch."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def _decode_args(n=3, hq=8, hkv=2, d=128, nb=16, maxb=4):
    dev = torch.device("cuda")
    q = torch.zeros(n, hq, d, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(nb, hkv, 16, d, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    bt = torch.zeros(n, maxb, dtype=torch.int32, device=dev)
    lens = torch.ones(n, dtype=torch.int32, device=dev)
    return q, kc, vc, bt, lens


@pytest.mark.parametrize("bad", ["table_rows", "lens", "out", "v_cache"])
def test_decode_calls_reject_mismatched_shapes(gpu, bad):
    pa = gpu
    print("[case] binding shape check", bad, flush=True)
    q, kc, vc, bt, lens = _decode_args()
    out = None
    if bad == "table_rows":
        bt = bt[:2].contiguous()
    elif bad == "lens":
        lens = lens[:2].contiguous()
    elif bad == "out":
        out = torch.empty(2, *q.shape[1:], dtype=q.dtype, device=q.device)
    else:
        vc = vc[:8].contiguous()
    key = torch.zeros(q.shape[0], kc.shape[1], kc.shape[3], dtype=q.dtype, device=q.device)
    with pytest.raises(ValueError):
        pa.decode(q, kc, vc, bt, lens, 16, out=out)
    with pytest.raises(ValueError):
        pa.decode_step(q, key, key.clone(), kc, vc, bt, lens, 16, out=out)
    with pytest.raises(ValueError):
        pa.cascade_decode(q, kc, vc, bt, lens, 16, 1, out=out)


@pytest.mark.parametrize("bad", ["cu_seqlens", "table_rows", "out"])
def test_varlen_rejects_mismatched_shapes(gpu, bad):
    pa = gpu
    print("[case] varlen shape check", bad, flush=True)
    dev = torch.device("cuda")
    q, kc, vc, bt, _ = _decode_args(n=3)
    cu = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device=dev)
    co = torch.zeros(3, dtype=torch.int32, device=dev)
    out = None
    if bad == "cu_seqlens":
        cu = cu[:3].contiguous()
    elif bad == "table_rows":
        bt = bt[:2].contiguous()
    else:
        out = torch.empty(2, *q.shape[1:], dtype=q.dtype, device=dev)
    with pytest.raises(ValueError):
        pa.varlen_prefill(q, kc, vc, cu, co, bt, 1, 16, out=out)


@pytest.mark.parametrize("bad", ["cu_seqlens", "table_rows", "out"])
def test_slot_mapping_rejects_mismatched_shapes(gpu, bad):
    pa = gpu
    print("[case] slot mapping shape check", bad, flush=True)
    dev = torch.device("cuda")
    cu = torch.tensor([0, 2, 5], dtype=torch.int32, device=dev)
    co = torch.zeros(2, dtype=torch.int32, device=dev)
    bt = torch.zeros(2, 4, dtype=torch.int32, device=dev)
    out = torch.empty(5, dtype=torch.int64, device=dev)
    if bad == "cu_seqlens":
        cu = cu[:2].contiguous()
    elif bad == "table_rows":
        bt = bt[:1].contiguous()
    else:
        out = out[:4]
    with pytest.raises(ValueError):
        pa.build_slot_mapping(cu, co, bt, 5, out=out)
