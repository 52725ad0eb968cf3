"""Host-side checks of the torch-facing wrappers that need no GPU."""

import numpy as np
import pytest

import linear_attention_la_amd as la


def test_attention_rejects_host_tensors():
    import torch

    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="device tensor"):
        la.attention(q, q, q, np.array([0, 4], np.int32), np.ones(2, np.float32))


def test_attention_function_is_differentiable_op():
    import torch

    fn = la._binding._attention_function()
    assert issubclass(fn, torch.autograd.Function)
    assert fn is la._binding._attention_function()  # defined once
