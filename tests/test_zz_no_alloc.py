"""GPU check of la_prefill_segmented_noalloc (the segmented prefill whose
workspace is the library's static device scratch) against
la_prefill_segmented with a caller workspace, through the C ABI: two calls
in a row, the second on a smaller input, each equal bit for bit to the
entry point it varies (same kernels, same order of sums)."""

import numpy as np
import pytest

from la_inputs import cu_seqlens, host_qkv, random_states
from tests.gpu_util import device, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _case(dev, lengths, H, d, seed, segment_len, kv_init, out_f32):
    import torch
    import linear_attention_la_amd as la

    say(f"case noalloc lengths={lengths} H={H} d={d} segment_len={segment_len} "
        f"kv_init={kv_init} out_f32={out_f32}")
    T = int(sum(lengths))
    decay = np.linspace(1.0, 0.8, H).astype(np.float32)
    q, k, v = host_qkv(T, H, d, seed, "bf16")
    cu = cu_seqlens(lengths)
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    kv0 = to_dev(random_states(len(lengths), H, d, seed + 1, scale=0.1), torch.float32, dev) \
        if kv_init else None
    od = torch.float32 if out_f32 else None
    o_ref, kv_ref = la.prefill_segmented(qd, kd, vd, cu, decay, segment_len, kv_init=kv0,
                                         out_dtype=od)
    # the no-allocation call writes into buffers given to it
    o = torch.full_like(o_ref, float("nan"))
    kv = torch.full_like(kv_ref, float("nan"))
    o_, kv_ = la.prefill_segmented_noalloc(qd, kd, vd, cu, decay, segment_len, kv_init=kv0,
                                           out_dtype=od, out=o, kv_final=kv)
    torch.cuda.synchronize()
    assert o_ is o and kv_ is kv
    assert torch.equal(o, o_ref), "O differs from la_prefill_segmented"
    assert torch.equal(kv, kv_ref), "final state differs from la_prefill_segmented"
    return o, kv


def test_noalloc_two_calls_second_smaller(dev):
    """A larger call (3 sequences incl. an empty one, 4 heads, d = 128,
    initial states, fp32 output) and then a smaller one (one sequence, 2
    heads, d = 64): the scratch keeps the first call's contents, which the
    second must not depend on."""
    _case(dev, [700, 0, 333], 4, 128, 9101, 128, kv_init=True, out_f32=True)
    _case(dev, [200], 2, 64, 9102, 64, kv_init=False, out_f32=False)


def test_noalloc_wide_then_small(dev):
    """256 (segment, head) chains (the one-workgroup-per-chain kernel in both
    passes), then a one-segment call."""
    _case(dev, [4096], 64, 128, 9103, 1024, kv_init=False, out_f32=False)
    _case(dev, [64], 1, 128, 9104, 64, kv_init=True, out_f32=False)


def test_noalloc_rejects_oversize(dev):
    import torch
    import linear_attention_la_amd as la

    q = torch.zeros((9, 64, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(la.LAError, match="scratch"):  # 9 x 64 chains need 72 MiB
        la.prefill_segmented_noalloc(q, q, q, list(range(10)), np.full(64, 0.9, np.float32), 64)
