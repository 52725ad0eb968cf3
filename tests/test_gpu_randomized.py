"""Seeded randomized GPU parity (needs an MI355X): many small configurations
of la_prefill (both bf16 kernels and the fp32 path), la_prefill_segmented
(and its no-allocation form), la_prefill_backward (plain and segmented),
la_prefill_normed and the state pool (prefill then decode) against the fp64
oracle, and la_prefill's choice of kernels across chain counts.
Each case draws its batch shape, lengths (block edges 0, 1, 63, 64, 65
included often), head count, d, decays, initial states and output dtype
from its own seed, and prints them before it runs."""

import numpy as np
import pytest

import oracle
from la_inputs import cu_seqlens, host_qkv, random_states
from tests import parity
from tests.gpu_util import device, say, to_dev, to_np

pytestmark = pytest.mark.gpu

EDGES = (0, 1, 63, 64, 65, 127, 128, 129)


@pytest.fixture(scope="module")
def dev():
    return device()


def _lengths(rng, S, max_len):
    out = []
    for _ in range(S):
        if rng.random() < 0.4:
            out.append(int(rng.choice(EDGES)))
        else:
            out.append(int(rng.integers(0, max_len + 1)))
    return out


def _decays(rng, H):
    kind = rng.integers(0, 3, size=H)
    d = np.where(kind == 0, 1.0,
                 np.where(kind == 1, rng.uniform(0.5, 1.0, size=H),
                          1.0 - 10.0 ** rng.uniform(-6, -1, size=H)))
    return d.astype(np.float32)


def _case(seed, wide=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    if wide:  # enough (sequence, head) chains for the one-workgroup-per-chain kernel
        S, H, d = int(rng.integers(6, 9)), int(rng.integers(48, 65)), 128
        lengths = _lengths(rng, S, 200)
    else:
        S, H, d = int(rng.integers(1, 13)), int(rng.integers(1, 9)), int(rng.choice([64, 128]))
        lengths = _lengths(rng, S, 400)
    return rng, lengths, H, d, _decays(rng, H)


@pytest.mark.parametrize("case", range(24))
def test_random_prefill(dev, case):
    import torch
    import linear_attention_la_amd as la

    wide = case % 6 == 5
    rng, lengths, H, d, decay = _case(7000 + case, wide)
    fp32_in = (not wide) and case % 4 == 1
    kv_init = bool(rng.random() < 0.5)
    out_f32 = fp32_in or bool(rng.random() < 0.5)
    in_place = kv_init and bool(rng.random() < 0.5)
    say(f"random prefill case {case}: lengths={lengths} H={H} d={d} fp32_in={fp32_in} "
        f"kv_init={kv_init} out_f32={out_f32} in_place={in_place} decay={decay.tolist()[:4]}...")
    T = sum(lengths)
    q, k, v = host_qkv(T, H, d, 8000 + case, "fp32" if fp32_in else "bf16")
    cu = cu_seqlens(lengths)
    kv0 = random_states(len(lengths), H, d, 9000 + case, scale=0.1) if kv_init else None
    tdt = torch.float32 if fp32_in else torch.bfloat16
    qd, kd, vd = (to_dev(x, tdt, dev) for x in (q, k, v))
    kv0d = to_dev(kv0, torch.float32, dev) if kv_init else None
    o, kv = la.prefill(qd, kd, vd, cu, decay, kv_init=kv0d,
                       out_dtype=torch.float32 if out_f32 else None,
                       kv_final=kv0d if in_place else None)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, kv_init=kv0)
    tol = 1e-5 if fp32_in else 1e-2
    s1 = parity.check(to_np(o), o_ref, 1, tol, out_bf16=not out_f32, what=f"case {case} o")
    s2 = parity.check(to_np(kv), kv_ref, 1, tol, what=f"case {case} kv")
    say("  ", s1, s2)


@pytest.mark.parametrize("case", range(10))
def test_random_kernel_choice(dev, monkeypatch, case):
    """la_prefill at d = 128 over 32 to 1280 (sequence, head) chains, equal or
    mixed lengths: the library picks the 32-column kernel, one workgroup per
    chain, or whole waves of the latter with the remaining sequences in
    slices.  Every sequence's rows and final state equal, bit for bit, those
    of the kernel that la_prefill_kernel_plan names for it, forced for the
    whole call (LA_NDV), and the call matches the oracle."""
    import torch
    import linear_attention_la_amd as la

    rng = np.random.Generator(np.random.PCG64(7600 + case))
    S = int(rng.integers(2, 21))
    H = int(rng.choice([16, 24, 32, 48, 64]))
    if rng.random() < 0.5:
        lengths = [int(rng.integers(1, 401))] * S
    else:
        lengths = _lengths(rng, S, 400)
    decay = _decays(rng, H)
    kv_init = bool(rng.random() < 0.5)
    say(f"random kernel choice case {case}: chains={S * H} lengths={lengths} H={H} "
        f"kv_init={kv_init}")
    T = sum(lengths)
    q, k, v = host_qkv(T, H, 128, 8600 + case, "bf16")
    cu = cu_seqlens(lengths)
    kv0 = random_states(S, H, 128, 9600 + case, scale=0.1) if kv_init else None
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    kv0d = to_dev(kv0, torch.float32, dev) if kv_init else None

    def run(ndv):
        if ndv is None:
            monkeypatch.delenv("LA_NDV", raising=False)
        else:
            monkeypatch.setenv("LA_NDV", ndv)
        o, kv = la.prefill(qd, kd, vd, cu, decay, kv_init=kv0d, out_dtype=torch.float32)
        torch.cuda.synchronize()
        return o, kv

    o, kv = run(None)
    forced = [run("1"), run("4")]
    monkeypatch.delenv("LA_NDV")
    n_wide, order = la.kernel_plan(cu, H, 128)  # the plan for this device
    for pos, s in enumerate(order.tolist()):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        fo, fkv = forced[0] if pos < n_wide else forced[1]
        assert torch.equal(o[rows], fo[rows]) and torch.equal(kv[s], fkv[s]), \
            f"sequence {s} did not run on the kernel la_prefill_kernel_plan names"
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, kv_init=kv0)
    s1 = parity.check(to_np(o), o_ref, 1, 1e-2, what=f"case {case} o")
    s2 = parity.check(to_np(kv), kv_ref, 1, 1e-2, what=f"case {case} kv")
    say("  ", s1, s2)


@pytest.mark.parametrize("case", range(8))
def test_random_segmented(dev, case):
    import torch
    import linear_attention_la_amd as la

    rng, lengths, H, d, decay = _case(7100 + case, wide=case == 7)
    segment_len = int(rng.choice([64, 128, 192, 256]))
    kv_init = bool(rng.random() < 0.5)
    out_f32 = bool(rng.random() < 0.5)
    say(f"random segmented case {case}: lengths={lengths} H={H} d={d} "
        f"segment_len={segment_len} kv_init={kv_init} out_f32={out_f32}")
    T = sum(lengths)
    q, k, v = host_qkv(T, H, d, 8100 + case, "bf16")
    cu = cu_seqlens(lengths)
    kv0 = random_states(len(lengths), H, d, 9100 + case, scale=0.1) if kv_init else None
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    o, kv = la.prefill_segmented(qd, kd, vd, cu, decay, segment_len,
                                 kv_init=to_dev(kv0, torch.float32, dev) if kv_init else None,
                                 out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, kv_init=kv0)
    s1 = parity.check(to_np(o), o_ref, 1, 1e-2, out_bf16=not out_f32, what=f"case {case} o")
    s2 = parity.check(to_np(kv), kv_ref, 1, 1e-2, what=f"case {case} kv")
    say("  ", s1, s2)


@pytest.mark.parametrize("case", range(8))
def test_random_backward(dev, case):
    import torch
    import linear_attention_la_amd as la

    rng, lengths, H, d, decay = _case(7200 + case, wide=case == 7)
    kv_init = bool(rng.random() < 0.5)
    dkv_final = bool(rng.random() < 0.5)
    f32 = bool(rng.random() < 0.5)
    say(f"random backward case {case}: lengths={lengths} H={H} d={d} kv_init={kv_init} "
        f"dkv_final={dkv_final} f32_grads={f32}")
    T = sum(lengths)
    S = len(lengths)
    q, k, v = host_qkv(T, H, d, 8200 + case, "bf16")
    do = host_qkv(T, H, d, 8300 + case, "bf16")[0]
    cu = cu_seqlens(lengths)
    kv0 = random_states(S, H, d, 9200 + case, scale=0.1) if kv_init else None
    g = random_states(S, H, d, 9300 + case, scale=0.1) if dkv_final else None
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v, do))
    out = la.prefill_backward(qd, kd, vd, dod, cu, decay,
                              kv_init=to_dev(kv0, torch.float32, dev) if kv_init else None,
                              dkv_final=to_dev(g, torch.float32, dev) if dkv_final else None,
                              grad_dtype=torch.float32 if f32 else None)
    torch.cuda.synchronize()
    ref = oracle.backward_varlen(q, k, v, do, cu, decay, kv_init=kv0, dkv_final=g)
    stats = [parity.check(to_np(a), b, 1, 1e-2, out_bf16=not f32, what=f"case {case} {n}")
             for n, a, b in zip(("dq", "dk", "dv"), out[:3], ref[:3])]
    stats.append(parity.check(to_np(out[3]), ref[3], 1, 1e-2, what=f"case {case} dkv_init"))
    say("  ", stats)


@pytest.mark.parametrize("case", range(8))
def test_random_backward_segmented(dev, case):
    import torch
    import linear_attention_la_amd as la

    rng, lengths, H, d, decay = _case(7300 + case, wide=case == 7)
    segment_len = int(rng.choice([64, 128, 192, 320]))
    kv_init = bool(rng.random() < 0.5)
    dkv_final = bool(rng.random() < 0.5)
    f32 = bool(rng.random() < 0.5)
    say(f"random segmented backward case {case}: lengths={lengths} H={H} d={d} "
        f"segment_len={segment_len} kv_init={kv_init} dkv_final={dkv_final} f32_grads={f32}")
    T = sum(lengths)
    S = len(lengths)
    q, k, v = host_qkv(T, H, d, 8400 + case, "bf16")
    do = host_qkv(T, H, d, 8500 + case, "bf16")[0]
    cu = cu_seqlens(lengths)
    kv0 = random_states(S, H, d, 9400 + case, scale=0.1) if kv_init else None
    g = random_states(S, H, d, 9500 + case, scale=0.1) if dkv_final else None
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v, do))
    out = la.prefill_backward_segmented(
        qd, kd, vd, dod, cu, decay, segment_len,
        kv_init=to_dev(kv0, torch.float32, dev) if kv_init else None,
        dkv_final=to_dev(g, torch.float32, dev) if dkv_final else None,
        grad_dtype=torch.float32 if f32 else None)
    torch.cuda.synchronize()
    ref = oracle.backward_varlen(q, k, v, do, cu, decay, kv_init=kv0, dkv_final=g)
    stats = [parity.check(to_np(a), b, 1, 1e-2, out_bf16=not f32, what=f"case {case} {n}")
             for n, a, b in zip(("dq", "dk", "dv"), out[:3], ref[:3])]
    stats.append(parity.check(to_np(out[3]), ref[3], 1, 1e-2, what=f"case {case} dkv_init"))
    say("  ", stats)


def _weights(rng, H, d):
    return rng.uniform(0.5, 1.5, (H, d)).astype(np.float32)


@pytest.mark.parametrize("case", range(8))
def test_random_prefill_normed(dev, case):
    """la_prefill_normed: the one-workgroup-per-chain path (every second case)
    or the chained scan, random gate, eps, kv_init and output dtype."""
    import torch
    import linear_attention_la_amd as la

    wide = case % 2 == 1
    rng = np.random.Generator(np.random.PCG64(7400 + case))
    if wide:
        S, H = int(rng.integers(5, 9)), int(rng.integers(48, 65))
        lengths = _lengths(rng, S, 200)
    else:
        S, H = int(rng.integers(1, 5)), int(rng.integers(1, 9))
        lengths = _lengths(rng, S, 900)
    d = 128
    decay = _decays(rng, H)
    gate = bool(rng.random() < 0.6)
    kv_init = bool(rng.random() < 0.5)
    out_f32 = bool(rng.random() < 0.5)
    eps = float(10.0 ** rng.uniform(-6, -3))
    heads = sorted({0, H - 1, int(rng.integers(0, H))})
    say(f"random normed prefill case {case}: lengths={lengths} H={H} gate={gate} "
        f"kv_init={kv_init} out_f32={out_f32} eps={eps:.2e}")
    T = sum(lengths)
    q, k, v = host_qkv(T, H, d, 8600 + case, "bf16")
    g = host_qkv(T, H, d, 8700 + case, "bf16")[0] * 30.0 if gate else None
    cu = cu_seqlens(lengths)
    kv0 = random_states(S, H, d, 9600 + case, scale=0.1) if kv_init else None
    w = _weights(rng, H, d)
    gd = to_dev(g, torch.bfloat16, dev) if gate else None
    y, kv = la.prefill_normed(*(to_dev(x, torch.bfloat16, dev) for x in (q, k, v)), cu, decay,
                              to_dev(w, torch.float32, dev), eps, gd,
                              kv_init=to_dev(kv0, torch.float32, dev) if kv_init else None,
                              out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.prefill_varlen(q[:, heads], k[:, heads], v[:, heads], cu,
                                          decay[heads],
                                          kv_init=None if kv0 is None else kv0[:, heads])
    y_ref = oracle.norm_gate(o_ref, w[heads], eps, to_np(gd)[:, heads] if gate else None)
    s1 = parity.check(to_np(y)[:, heads], y_ref, 1, 1e-2, out_bf16=not out_f32,
                      what=f"case {case} y")
    s2 = parity.check(to_np(kv)[:, heads], kv_ref, 1, 1e-2, what=f"case {case} kv")
    say("  ", s1, s2)


@pytest.mark.parametrize("case", range(8))
def test_random_pool_prefill_then_decode(dev, case):
    """A chunk of la_prefill_pool on random slots, then la_decode_pool on a
    random subset of those slots: every output and every pool entry against
    the oracle's pool functions."""
    import torch
    import linear_attention_la_amd as la

    rng = np.random.Generator(np.random.PCG64(7500 + case))
    S, H, d = int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.choice([64, 128]))
    P = S + int(rng.integers(0, 6))
    lengths = _lengths(rng, S, 300)
    decay = _decays(rng, H)
    slots = rng.permutation(P)[:S].astype(np.int32)
    say(f"random pool case {case}: lengths={lengths} H={H} d={d} P={P} slots={slots.tolist()}")
    T = sum(lengths)
    q, k, v = host_qkv(T, H, d, 8800 + case, "bf16")
    cu = cu_seqlens(lengths)
    pool = random_states(P, H, d, 9800 + case, scale=0.1)
    pool_d = to_dev(pool, torch.float32, dev)
    o = la.prefill_pool(*(to_dev(x, torch.bfloat16, dev) for x in (q, k, v)), cu, decay, pool_d,
                        slots)
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle.prefill_pool(q, k, v, cu, decay, pool, slots)
    s1 = parity.check(to_np(o), o_ref, 1, 1e-2, out_bf16=True, what=f"case {case} prefill o")
    s2 = parity.check(to_np(pool_d), pool_ref, 1, 1e-2, what=f"case {case} pool after prefill")
    B = int(rng.integers(1, S + 1))
    dslots = rng.permutation(slots)[:B].astype(np.int32)
    q1, k1, v1 = (x[:B * H].reshape(B, H, d)
                  for x in host_qkv(B * H, 1, d, 8900 + case, "bf16"))
    pool_host = to_np(pool_d)
    o1 = la.decode_pool(*(to_dev(x, torch.bfloat16, dev) for x in (q1, k1, v1)), pool_d, dslots,
                        decay)
    torch.cuda.synchronize()
    o1_ref, pool1_ref = oracle.decode_pool(q1, k1, v1, pool_host, dslots, decay)
    s3 = parity.check(to_np(o1), o1_ref, 1, 1e-2, out_bf16=True, what=f"case {case} decode o")
    s4 = parity.check(to_np(pool_d), pool1_ref, 1, 1e-5, what=f"case {case} pool after decode")
    say("  ", s1, s2, s3, s4)


@pytest.mark.parametrize("case", range(6))
def test_random_segmented_noalloc(dev, case):
    """la_prefill_segmented_noalloc on random batches (its static scratch
    reused from call to call) against the oracle."""
    import torch
    import linear_attention_la_amd as la

    rng, lengths, H, d, decay = _case(7600 + case, wide=case == 5)
    segment_len = int(rng.choice([64, 128, 256]))
    kv_init = bool(rng.random() < 0.5)
    say(f"random noalloc case {case}: lengths={lengths} H={H} d={d} segment_len={segment_len} "
        f"kv_init={kv_init}")
    T = sum(lengths)
    q, k, v = host_qkv(T, H, d, 8950 + case, "bf16")
    cu = cu_seqlens(lengths)
    kv0 = random_states(len(lengths), H, d, 9900 + case, scale=0.1) if kv_init else None
    o, kv = la.prefill_segmented_noalloc(
        *(to_dev(x, torch.bfloat16, dev) for x in (q, k, v)), cu, decay, segment_len,
        kv_init=to_dev(kv0, torch.float32, dev) if kv_init else None)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, kv_init=kv0)
    s1 = parity.check(to_np(o), o_ref, 1, 1e-2, out_bf16=True, what=f"case {case} o")
    s2 = parity.check(to_np(kv), kv_ref, 1, 1e-2, what=f"case {case} kv")
    say("  ", s1, s2)
