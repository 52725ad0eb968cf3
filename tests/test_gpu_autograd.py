"""attention(): the autograd wrapper over prefill / prefill_backward (needs
an MI355X).  Its forward and gradients must be the direct calls' results bit
for bit (it only marshals arguments), and match the fp64 oracle backward."""

import numpy as np
import pytest

import oracle
from la_inputs import cu_seqlens, host_qkv, random_states
from tests import parity
from tests.gpu_util import device, say, to_dev, to_np

pytestmark = pytest.mark.gpu

LENGTHS = [1, 63, 64, 65, 129, 0, 300, 17]
DECAY = np.array([1.0, 0.99, 0.9, 0.5], np.float32)


@pytest.fixture(scope="module")
def dev():
    return device()


def _inputs(dev, d, seed, kv_init=True):
    import torch

    T, H, S = sum(LENGTHS), len(DECAY), len(LENGTHS)
    q, k, v = host_qkv(T, H, d, seed, "bf16")
    w_o = host_qkv(T, H, d, seed + 1, "bf16")[0]          # bf16-exact upstream dO
    w_kv = random_states(S, H, d, seed + 2, scale=0.1)    # upstream dS_L
    kv0 = random_states(S, H, d, seed + 3, scale=0.1) if kv_init else None
    t = dict(q=to_dev(q, torch.bfloat16, dev), k=to_dev(k, torch.bfloat16, dev),
             v=to_dev(v, torch.bfloat16, dev), w_o=to_dev(w_o, torch.bfloat16, dev),
             w_kv=to_dev(w_kv, torch.float32, dev),
             kv0=None if kv0 is None else to_dev(kv0, torch.float32, dev))
    host = dict(q=q, k=k, v=v, w_o=w_o, w_kv=w_kv, kv0=kv0)
    return t, host


def _autograd(t, segment_len=None, use_kv=True):
    import torch
    import linear_attention_la_amd as la

    leaves = [x.clone().requires_grad_(True) for x in (t["q"], t["k"], t["v"])]
    kv0 = None if t["kv0"] is None else t["kv0"].clone().requires_grad_(True)
    o, kv = la.attention(*leaves, cu_seqlens(LENGTHS), DECAY, kv_init=kv0,
                         segment_len=segment_len)
    loss = (o.float() * t["w_o"].float()).sum()
    if use_kv:
        loss = loss + (kv * t["w_kv"]).sum()
    loss.backward()
    torch.cuda.synchronize()
    grads = [x.grad for x in leaves] + [None if kv0 is None else kv0.grad]
    return o.detach(), kv.detach(), grads


def _direct(t, segment_len=None, use_kv=True):
    import torch
    import linear_attention_la_amd as la

    cu = cu_seqlens(LENGTHS)
    if segment_len is None:
        o, kv = la.prefill(t["q"], t["k"], t["v"], cu, DECAY, kv_init=t["kv0"])
        g = la.prefill_backward(t["q"], t["k"], t["v"], t["w_o"], cu, DECAY, kv_init=t["kv0"],
                                dkv_final=t["w_kv"] if use_kv else None,
                                init_grad=t["kv0"] is not None)
    else:
        o, kv = la.prefill_segmented(t["q"], t["k"], t["v"], cu, DECAY, segment_len,
                                     kv_init=t["kv0"])
        g = la.prefill_backward_segmented(t["q"], t["k"], t["v"], t["w_o"], cu, DECAY,
                                          segment_len, kv_init=t["kv0"],
                                          dkv_final=t["w_kv"] if use_kv else None,
                                          init_grad=t["kv0"] is not None)
    torch.cuda.synchronize()
    return o, kv, list(g)


def _same(a, b, what):
    import torch

    if a is None or b is None:
        assert a is None and b is None, what
        return
    assert a.dtype == b.dtype and a.shape == b.shape, what
    assert torch.equal(a, b), f"{what}: autograd differs from the direct call"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("segment_len", [None, 64])
def test_autograd_equals_direct_calls(dev, d, segment_len):
    say(f"case autograd d={d} segment_len={segment_len}")
    t, _ = _inputs(dev, d, 700 + d)
    ao, akv, ag = _autograd(t, segment_len)
    do_, dkv, dg = _direct(t, segment_len)
    _same(ao, do_, "o")
    _same(akv, dkv, "kv_final")
    for name, a, b in zip(("dq", "dk", "dv", "dkv_init"), ag, dg):
        _same(a, b, name)


def test_autograd_output_only_no_initial_state(dev):
    """Only o enters the loss (the final-state gradient is None) and there is
    no initial state (no dkv_init is formed)."""
    say("case autograd o only, no kv_init")
    t, _ = _inputs(dev, 128, 811, kv_init=False)
    ao, akv, ag = _autograd(t, None, use_kv=False)
    do_, dkv, dg = _direct(t, None, use_kv=False)
    _same(ao, do_, "o")
    _same(akv, dkv, "kv_final")
    for name, a, b in zip(("dq", "dk", "dv"), ag[:3], dg[:3]):
        _same(a, b, name)
    assert ag[3] is None


def test_autograd_final_state_only(dev):
    """Only the final state enters the loss: dO is zero, and dQ with it."""
    import torch
    import linear_attention_la_amd as la

    say("case autograd kv only")
    t, _ = _inputs(dev, 128, 823)
    leaves = [x.clone().requires_grad_(True) for x in (t["q"], t["k"], t["v"])]
    kv0 = t["kv0"].clone().requires_grad_(True)
    _, kv = la.attention(*leaves, cu_seqlens(LENGTHS), DECAY, kv_init=kv0)
    (kv * t["w_kv"]).sum().backward()
    torch.cuda.synchronize()
    g = la.prefill_backward(t["q"], t["k"], t["v"], torch.zeros_like(t["q"]), cu_seqlens(LENGTHS),
                            DECAY, kv_init=t["kv0"], dkv_final=t["w_kv"])
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dkv_init"), [x.grad for x in leaves] + [kv0.grad],
                          g):
        _same(a, b, name)
    assert not torch.any(leaves[0].grad)


def test_autograd_against_oracle(dev):
    """Gradients of the autograd path against the fp64 oracle backward."""
    say("case autograd vs oracle")
    t, h = _inputs(dev, 128, 845)
    _, _, ag = _autograd(t)
    ref = oracle.backward_varlen(h["q"], h["k"], h["v"], h["w_o"], cu_seqlens(LENGTHS), DECAY,
                                 kv_init=h["kv0"], dkv_final=h["w_kv"])
    stats = []
    for name, a, b in zip(("dq", "dk", "dv"), ag[:3], ref[:3]):
        stats.append(parity.check(to_np(a), b, 1, 1e-2, out_bf16=True, what=f"autograd {name}"))
    stats.append(parity.check(to_np(ag[3]), ref[3], 1, 1e-2, what="autograd dkv_init"))
    say("autograd vs oracle", stats)
