"""GPU parity of la_prefill_backward (dQ, dK, dV, dS_init) against the fp64
oracle backward (needs an MI355X)."""

import numpy as np
import pytest

import oracle
from la_inputs import cu_seqlens, host_qkv, random_states, workload
from tests import parity
from tests.gpu_util import device, say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _run(dev, lengths, H, d, decay, seed, kv_init, dkv_final, f32_grads=False, heads=None):
    import torch
    import linear_attention_la_amd as la

    say(f"case backward lengths={list(lengths)[:8]} H={H} d={d} kv_init={kv_init} "
        f"dkv_final={dkv_final} f32_grads={f32_grads}")
    T = int(sum(lengths))
    S = len(lengths)
    q, k, v = host_qkv(T, H, d, seed, "bf16")
    do = host_qkv(T, H, d, seed + 1, "bf16")[0]
    cu = cu_seqlens(lengths)
    kv0 = random_states(S, H, d, seed + 7, scale=0.1) if kv_init else None
    g = random_states(S, H, d, seed + 9, scale=0.1) if dkv_final else None
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v, do))
    out = la.prefill_backward(qd, kd, vd, dod, cu, decay,
                              kv_init=to_dev(kv0, torch.float32, dev) if kv_init else None,
                              dkv_final=to_dev(g, torch.float32, dev) if dkv_final else None,
                              grad_dtype=torch.float32 if f32_grads else None)
    torch.cuda.synchronize()
    ref = oracle.backward_varlen(q, k, v, do, cu, decay, kv_init=kv0, dkv_final=g, heads=heads)
    return [to_np(x) for x in out], ref


def _check(gpu, ref, f32_grads, heads=None, what=""):
    sel = (lambda x: x) if heads is None else (lambda x: x[:, list(heads)])
    stats = []
    for name, a, b in zip(("dq", "dk", "dv"), gpu[:3], ref[:3]):
        stats.append(parity.check(sel(a), sel(b), 1, 1e-2, out_bf16=not f32_grads,
                                  what=f"{what} {name}"))
    stats.append(parity.check(sel(gpu[3]), sel(ref[3]), 1, 1e-2, what=f"{what} dkv_init"))
    return stats


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kv_init,dkv_final", [(False, False), (True, True), (False, True),
                                                (True, False)])
def test_backward_ragged(dev, d, kv_init, dkv_final):
    """Ragged lengths around the 64-token block (empty, 1, 63..65, several
    blocks plus a tail), decays from none to strong, with and without an
    initial state and a final-state gradient."""
    lengths = [1, 63, 64, 65, 129, 0, 300, 17]
    decay = np.array([1.0, 0.99, 0.9, 0.5], np.float32)
    gpu, ref = _run(dev, lengths, 4, d, decay, 51 + d, kv_init, dkv_final)
    say("backward ragged", _check(gpu, ref, False, what="ragged"))


def test_backward_fp32_grads(dev):
    lengths = [200, 0, 513]
    decay = np.array([0.999, 0.97, 0.8], np.float32)
    gpu, ref = _run(dev, lengths, 3, 128, decay, 83, True, True, f32_grads=True)
    say("backward fp32 grads", _check(gpu, ref, True, what="fp32 grads"))


def test_backward_n8k_sampled_heads(dev):
    """B=1, H=64, N=8192, d=128 with the seeded decays (initial state and
    final-state gradient): three heads (no, mid and strongest decay
    included) against the oracle's two-chain backward."""
    w = workload("n8k")
    heads = [0, int(np.argmin(w["decay"])), int(np.argmax(w["decay"]))]
    gpu, ref = _run(dev, w["lengths"], 64, 128, w["decay"], 1002, True, True, heads=heads)
    say("backward n8k", _check(gpu, ref, False, heads=heads, what="n8k"))


@pytest.mark.parametrize("kv_init,dkv_final,f32_grads", [(False, False, False), (True, True, False),
                                                         (True, True, True)])
def test_backward_wide_path(dev, kv_init, dkv_final, f32_grads):
    """Eight ragged sequences x 64 heads (512 chains: at least one per CU,
    1536 workgroups in the one launch of the d = 128 backward); every head
    against the oracle."""
    import torch

    lengths = [1, 63, 64, 65, 0, 300, 129, 17]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert len(lengths) * 64 >= cus
    decay = np.asarray(workload("n8k")["decay"], np.float32).copy()
    decay[0], decay[1] = 1.0, 0.5
    gpu, ref = _run(dev, lengths, 64, 128, decay, 61 + kv_init + 2 * f32_grads, kv_init, dkv_final,
                    f32_grads=f32_grads)
    say("backward wide", _check(gpu, ref, f32_grads, what="wide"))


def test_backward_single_chain(dev):
    """One sequence, one head: three workgroups, none in a whole group of
    XCD-placed items; a 64-token block boundary plus a tail."""
    decay = np.array([0.95], np.float32)
    gpu, ref = _run(dev, [130], 1, 128, decay, 141, True, True)
    say("backward single chain", _check(gpu, ref, False, what="single chain"))


@pytest.mark.parametrize("d", [64, 128])
def test_backward_extreme_decays(dev, d):
    """Decays down to the smallest one allowed with a final-state gradient
    (2^-64, whose 1/lambda = 2^64 scales dS_L into the reverse chains), next
    to no decay and a moderate one."""
    decay = np.array([1.0, 2.0 ** -64, 1e-10, 0.5, 0.999], np.float32)
    gpu, ref = _run(dev, [1, 64, 130, 0, 257], 5, d, decay, 151 + d, True, True)
    say("backward extreme decays", _check(gpu, ref, False, what="extreme decays"))


@pytest.mark.parametrize("segmented", [False, True])
def test_backward_without_initial_state_gradient(dev, segmented):
    """init_grad=False (dkv_init NULL): dq, dk and dv are exactly those of
    the call that also returns dS0."""
    import torch
    import linear_attention_la_amd as la

    lengths = [200, 70]
    decay = np.array([0.97, 0.8], np.float32)
    say(f"case backward without dS0 segmented={segmented}")
    T = sum(lengths)
    q, k, v = host_qkv(T, 2, 128, 161, "bf16")
    do = host_qkv(T, 2, 128, 162, "bf16")[0]
    cu = cu_seqlens(lengths)
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v, do))
    g = to_dev(random_states(2, 2, 128, 163, scale=0.1), torch.float32, dev)
    call = ((lambda **kw: la.prefill_backward_segmented(qd, kd, vd, dod, cu, decay, 128, **kw))
            if segmented else (lambda **kw: la.prefill_backward(qd, kd, vd, dod, cu, decay, **kw)))
    full = call(dkv_final=g)
    part = call(dkv_final=g, init_grad=False)
    torch.cuda.synchronize()
    assert part[3] is None
    for a, b in zip(full[:3], part[:3]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("segmented", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_all_sequences_empty(dev, segmented, d):
    """Sequences of length 0 only: no gradient rows, and dS0 = dS_L (its
    1/lambda and lambda scalings cancel up to rounding), against the oracle."""
    import torch
    import linear_attention_la_amd as la

    lengths = [0, 0, 0]
    decay = np.array([1.0, 0.9, 0.3], np.float32)
    say(f"case backward all empty d={d} segmented={segmented}")
    q = np.zeros((0, 3, d), np.float32)
    qd = torch.zeros((0, 3, d), dtype=torch.bfloat16, device=dev)
    cu = cu_seqlens(lengths)
    kv0 = random_states(3, 3, d, 171, scale=0.1)
    g = random_states(3, 3, d, 173, scale=0.1)
    kv0d, gd = to_dev(kv0, torch.float32, dev), to_dev(g, torch.float32, dev)
    if segmented:
        out = la.prefill_backward_segmented(qd, qd, qd, qd, cu, decay, 64, kv_init=kv0d,
                                            dkv_final=gd)
    else:
        out = la.prefill_backward(qd, qd, qd, qd, cu, decay, kv_init=kv0d, dkv_final=gd)
    torch.cuda.synchronize()
    assert all(x.shape[0] == 0 for x in out[:3])
    ref = oracle.backward_varlen(q, q, q, q, cu, decay, kv_init=kv0, dkv_final=g)
    parity.check(to_np(out[3]), ref[3], 1, 1e-5, what="all empty dkv_init")
