"""Shared test plumbing: repo root on sys.path, GPU gating, tensor views."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def host_bits(t):
    """A torch tensor as the numpy array the oracle takes: bf16 -> its uint16
    bit patterns, fp32 -> float32, integers unchanged (copied to the host)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is present; fail loudly if it is but the library is not."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_token_amd as pa  # raises if the HIP library is missing
    return pa


def route_block_manager(pa):
    """When PA_TEST_BLOCKS_LIB names a host-only build of the block manager
    (csrc/pa_blocks.cpp under the sanitizers), send the binding's pa_bm_*
    calls to it; every other call keeps going to libpa.so."""
    path = os.environ.get("PA_TEST_BLOCKS_LIB")
    if not path:
        return
    import ctypes
    san = ctypes.CDLL(path)
    real = pa.lib

    class Routed:
        def __getattr__(self, name):
            fn = getattr(real, name)
            if not name.startswith("pa_bm_"):
                return fn
            alt = getattr(san, name)
            alt.restype, alt.argtypes = fn.restype, fn.argtypes
            return alt

    pa.lib = Routed()
