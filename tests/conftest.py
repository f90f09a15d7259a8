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
