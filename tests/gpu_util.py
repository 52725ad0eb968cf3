"""Helpers shared by the GPU tests (device transfer, the device fixture)."""

import sys

import numpy as np
import pytest


def device():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import linear_attention_la_amd as la

    la.lib()  # raises if the HIP library is missing: no fallback path exists
    return torch.device("cuda:0")


def to_dev(x, dtype, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dtype).contiguous()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
