"""HIP graph capture of the library's launches (needs an MI355X).

The library allocates nothing and issues no memset or copy, so its calls can
be captured into a graph (torch.cuda.CUDAGraph) and replayed.  Each graph is
replayed several times with eager work and synchronisations between the
replays, and every replay is compared bit for bit with the eager call on the
same inputs: la_prefill_segmented_noalloc (the chained scan at d = 128, the
four-kernel path at d = 64; the plan kernel re-zeroes the scan's control
words on every replay), la_prefill, and la_decode on a state reset before
each replay."""

import numpy as np
import pytest

from la_inputs import cu_seqlens, host_qkv, random_states
from tests.gpu_util import device, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _capture(fn):
    """Capture fn() into a graph after one eager warm-up call on a side
    stream (torch requires the warm-up before capture)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _eager_noise(dev):
    """Unrelated eager work between replays."""
    import torch

    a = torch.randn(512, 512, device=dev)
    (a @ a).sum().item()


@pytest.mark.parametrize("d", [64, 128])
def test_graph_segmented_noalloc(dev, d):
    import torch
    import linear_attention_la_amd as la

    lengths, H, seg = [700, 0, 300, 64], 4, 128
    say(f"case graph noalloc d={d} lengths={lengths}")
    T, S = sum(lengths), len(lengths)
    q, k, v = (to_dev(x, torch.bfloat16, dev) for x in host_qkv(T, H, d, 611 + d, "bf16"))
    kv0 = to_dev(random_states(S, H, d, 612 + d, scale=0.1), torch.float32, dev)
    cu_h = cu_seqlens(lengths)
    cu = torch.from_numpy(cu_h).to(dev)
    decay = np.array([1.0, 0.99, 0.9, 0.6], np.float32)
    o = torch.empty_like(q)
    kvf = torch.empty_like(kv0)

    def call():
        la.prefill_segmented_noalloc(q, k, v, cu, decay, seg, kv_init=kv0, out=o, kv_final=kvf,
                                     cu_seqlens_host=cu_h)

    call()
    torch.cuda.synchronize()
    ref_o, ref_kv = o.clone(), kvf.clone()
    g = _capture(call)
    for r in range(3):
        o.zero_()
        kvf.zero_()
        _eager_noise(dev)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), f"replay {r}: output differs"
        assert torch.equal(kvf, ref_kv), f"replay {r}: final state differs"


def test_graph_prefill_and_decode(dev):
    import torch
    import linear_attention_la_amd as la

    lengths, H, d = [333, 64, 1], 64, 128
    say(f"case graph prefill + decode lengths={lengths}")
    T, S = sum(lengths), len(lengths)
    q, k, v = (to_dev(x, torch.bfloat16, dev) for x in host_qkv(T, H, d, 621, "bf16"))
    cu_h = cu_seqlens(lengths)
    cu = torch.from_numpy(cu_h).to(dev)
    decay = np.exp(-np.linspace(0.001, 0.1, H)).astype(np.float32)
    o = torch.empty_like(q)
    kv = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
    q1, k1, v1 = (to_dev(x[:S * H].reshape(S, H, d), torch.bfloat16, dev)
                  for x in host_qkv(S * H, 1, d, 622, "bf16"))
    o1 = torch.empty_like(q1)

    def call():
        la.prefill(q, k, v, cu, decay, out=o, kv_final=kv, cu_seqlens_host=cu_h)
        la.decode(q1, k1, v1, kv, decay, out=o1)  # continues from the prefill's states

    call()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (o, kv, o1)]
    g = _capture(call)
    for r in range(3):
        for x in (o, kv, o1):
            x.zero_()
        _eager_noise(dev)
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("o", "kv", "o1"), (o, kv, o1), ref):
            assert torch.equal(x, y), f"replay {r}: {name} differs"
