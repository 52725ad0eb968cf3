"""Invariants of the GPU path at full size (needs an MI355X): scaling,
continuation and packing order, each bit for bit.

The method is multilinear in its inputs: O(a q, b k, c v) = abc O(q, k, v)
and the state scales by bc (with an initial state scaled by bc).  For powers
of two every product, sum and rounding of the computation scales exactly --
the bf16 hi/lo splits, the fp32 accumulations and the final rounding commute
with the scale while nothing overflows or becomes subnormal -- so the scaled
call must return the unscaled result times the scale bit for bit.  This
holds at any size, so it is checked on the launches the bench times (no
oracle needed): both prefill kernels, the chained scan, decode and the
backward.  Continuation at a block boundary and the order in which
sequences are packed also leave every result bit-identical."""

import numpy as np
import pytest

from tests.gpu_util import device, say

pytestmark = pytest.mark.gpu

A, B, C = 8.0, 4.0, 2.0  # scales of q, k, v (powers of two)


@pytest.fixture(scope="module")
def dev():
    return device()


def _inputs(name, dev, H=64):
    import torch
    from la_inputs import cu_seqlens, device_qkv, device_states, workload

    w = workload(name)
    cu_h = cu_seqlens(w["lengths"])
    T, S = int(cu_h[-1]), len(w["lengths"])
    q, k, v = device_qkv(T, H, 128, w["seed"], dev)
    kv0 = device_states(S, H, 128, w["seed"] + 5, dev, scale=0.1)
    return q, k, v, kv0, cu_h, torch.from_numpy(cu_h).to(dev), np.asarray(w["decay"][:H])


@pytest.mark.parametrize("name", ["n8k", "batch8_n8k"])
def test_prefill_scaling(dev, name):
    """la_prefill on the 32-column kernel (B=1, H=64, N=8192) and on the
    one-workgroup-per-chain kernel (8 x 8192)."""
    import torch
    import linear_attention_la_amd as la

    say(f"case prefill scaling {name}")
    q, k, v, kv0, cu_h, cu, decay = _inputs(name, dev)
    o1, s1 = la.prefill(q, k, v, cu, decay, kv_init=kv0, cu_seqlens_host=cu_h)
    o2, s2 = la.prefill(q * A, k * B, v * C, cu, decay, kv_init=kv0 * (B * C),
                        cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.isfinite(s1).all()
    assert torch.equal(o2, o1 * (A * B * C)), "output"
    assert torch.equal(s2, s1 * (B * C)), "final state"


def test_segmented_scan_scaling(dev):
    """la_prefill_segmented (the chained scan) on one 64K-token sequence x 8
    heads in 4K segments (128 items)."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv, workload

    say("case segmented scaling")
    w = workload("sweep65536")
    N, H = 65536, 8
    q, k, v = device_qkv(N, H, 128, w["seed"], dev)
    cu_h = np.array([0, N], np.int32)
    cu = torch.from_numpy(cu_h).to(dev)
    decay = np.asarray(w["decay"][:H])
    o1, s1 = la.prefill_segmented(q, k, v, cu, decay, 4096, cu_seqlens_host=cu_h)
    o2, s2 = la.prefill_segmented(q * A, k * B, v * C, cu, decay, 4096, cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1 * (A * B * C)), "output"
    assert torch.equal(s2, s1 * (B * C)), "final state"


def test_decode_scaling(dev):
    """la_decode on the 256 x 64 serving batch."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv, device_states, workload

    say("case decode scaling")
    w = workload("mixed_decode")
    Bt, H, d = w["batch"], w["H"], w["d"]
    kv = device_states(Bt, H, d, w["seed"], dev, scale=0.5)
    q, k, v = (x.view(Bt, H, d) for x in device_qkv(Bt, H, d, w["seed"] + 1, dev))
    kv2 = kv * (B * C)
    o1 = la.decode(q, k, v, kv, w["decay"])
    o2 = la.decode(q * A, k * B, v * C, kv2, w["decay"])
    torch.cuda.synchronize()
    assert torch.equal(o2, o1 * (A * B * C)), "output"
    assert torch.equal(kv2, kv * (B * C)), "updated state"


def test_backward_scaling(dev):
    """la_prefill_backward at B=1, H=64, N=8192 with S0 and dS_L: with dO
    scaled by E, S0 by BC and dS_L by AE, dQ scales by EBC, dK by EAC, dV by
    ABE and dS0 by AE."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv, device_states

    E = 16.0
    say("case backward scaling")
    q, k, v, kv0, cu_h, cu, decay = _inputs("n8k", dev)
    do = device_qkv(8192, 64, 128, 77, dev)[0]
    g = device_states(1, 64, 128, 78, dev, scale=0.1)
    r1 = la.prefill_backward(q, k, v, do, cu, decay, kv_init=kv0, dkv_final=g,
                             cu_seqlens_host=cu_h)
    r2 = la.prefill_backward(q * A, k * B, v * C, do * E, cu, decay, kv_init=kv0 * (B * C),
                             dkv_final=g * (A * E), cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    for name, x1, x2, f in zip(("dq", "dk", "dv", "dkv_init"), r1, r2,
                               (E * B * C, E * A * C, A * B * E, A * E)):
        assert torch.isfinite(x1).all(), name
        assert torch.equal(x2, x1 * f), name


@pytest.mark.parametrize("name", ["n8k", "batch8_n8k"])
def test_continuation_bitwise(dev, name):
    """Prefilling the first 4096 tokens of every sequence, then the rest from
    the returned states (kv_final written over kv_init in place), gives the
    one-call result bit for bit: the split falls on a block boundary, the
    state crosses it in fp32 either way, and each call runs the same kernel."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import cu_seqlens

    say(f"case continuation bitwise {name}")
    q, k, v, kv0, cu_h, cu, decay = _inputs(name, dev)
    S = len(cu_h) - 1
    o_full, s_full = la.prefill(q, k, v, cu, decay, kv_init=kv0, cu_seqlens_host=cu_h)
    first = np.concatenate([np.arange(cu_h[s], cu_h[s] + 4096) for s in range(S)])
    rest = np.concatenate([np.arange(cu_h[s] + 4096, cu_h[s + 1]) for s in range(S)])
    fi, ri = (torch.from_numpy(x).to(dev) for x in (first, rest))
    half = cu_seqlens([4096] * S)
    st = kv0.clone()
    o1, _ = la.prefill(q[fi].contiguous(), k[fi].contiguous(), v[fi].contiguous(), half, decay,
                       kv_init=st, kv_final=st)
    o2, _ = la.prefill(q[ri].contiguous(), k[ri].contiguous(), v[ri].contiguous(),
                       cu_seqlens([int(cu_h[s + 1] - cu_h[s] - 4096) for s in range(S)]), decay,
                       kv_init=st, kv_final=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o_full[fi]), "first part"
    assert torch.equal(o2, o_full[ri]), "continued part"
    assert torch.equal(st, s_full), "final state"


def test_packing_order_bitwise(dev):
    """Eight 8K sequences packed in reverse order give, for every sequence,
    the same rows and final state bit for bit (one workgroup per chain either
    way; a chain's result does not depend on where its sequence sits)."""
    import torch
    import linear_attention_la_amd as la

    say("case packing order bitwise")
    q, k, v, kv0, cu_h, cu, decay = _inputs("batch8_n8k", dev)
    S = len(cu_h) - 1
    o1, s1 = la.prefill(q, k, v, cu, decay, kv_init=kv0, cu_seqlens_host=cu_h)
    order = list(range(S))[::-1]
    rows = np.concatenate([np.arange(cu_h[s], cu_h[s + 1]) for s in order])
    idx = torch.from_numpy(rows).to(dev)
    o2, s2 = la.prefill(q[idx].contiguous(), k[idx].contiguous(), v[idx].contiguous(), cu_h,
                        decay, kv_init=kv0[order].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o2, o1[idx]), "outputs"
    assert torch.equal(s2, s1[order]), "final states"


def test_backward_chains_are_forward_runs(dev):
    """Without S0 and dS_L the backward's three chains are forward runs of
    the same one-workgroup-per-chain kernel body: dQ = prefill(dO, V, K),
    dK = flip(prefill(flip V, flip dO, flip Q)) and dV = flip(prefill(flip K,
    flip Q, flip dO)), flip reversing the tokens of every sequence.  Checked
    bit for bit on eight 8K sequences x 64 heads (512 chains: la_prefill and
    la_prefill_backward both take that kernel)."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv

    say("case backward chains vs forward runs")
    q, k, v, _, cu_h, cu, decay = _inputs("batch8_n8k", dev)
    do = device_qkv(int(cu_h[-1]), 64, 128, 91, dev)[0]
    dq, dk, dv, _ = la.prefill_backward(q, k, v, do, cu, decay, cu_seqlens_host=cu_h)
    rows = np.concatenate([np.arange(cu_h[s + 1] - 1, cu_h[s] - 1, -1)
                           for s in range(len(cu_h) - 1)])
    fl = torch.from_numpy(rows).to(dev)  # token reversal within each sequence (an involution)

    def fwd(a, b, c):
        return la.prefill(a.contiguous(), b.contiguous(), c.contiguous(), cu, decay,
                          cu_seqlens_host=cu_h, final_state=False)[0]

    ref_dq = fwd(do, v, k)
    ref_dk = fwd(v[fl], do[fl], q[fl])[fl]
    ref_dv = fwd(k[fl], q[fl], do[fl])[fl]
    torch.cuda.synchronize()
    assert torch.equal(dq, ref_dq), "dq"
    assert torch.equal(dk, ref_dk), "dk"
    assert torch.equal(dv, ref_dv), "dv"
