"""GPU parity of la_decode, prefill->decode consistency, and the two-stream
mixed serving step (needs an MI355X)."""

import numpy as np
import pytest

import oracle
from la_inputs import (cu_seqlens, device_qkv, device_states, host_qkv, random_states,
                       workload)
from tests import parity
from tests.gpu_util import device, say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_random_states(dev, d, dtype):
    """Three successive decode steps on random states against the oracle."""
    import torch
    import linear_attention_la_amd as la

    B, H = 5, 3
    decay = np.array([1.0, 0.97, 0.5], np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kv = random_states(B, H, d, 41 + d)
    kvd = to_dev(kv, torch.float32, dev)
    kv_ref = kv.astype(np.float64)
    for step in range(3):
        say(f"decode d={d} dtype={dtype} step={step}")
        q, k, v = (x[:B * H].reshape(B, H, d)
                   for x in host_qkv(B * H, 1, d, 100 * step + d, dtype))
        o = la.decode(to_dev(q, tdt, dev), to_dev(k, tdt, dev), to_dev(v, tdt, dev), kvd, decay)
        torch.cuda.synchronize()
        # the oracle continues from the GPU's fp32 state of the previous step
        # only through values it computed itself: kv_ref is its own chain
        o_ref, kv_ref = oracle.decode_batch(q, k, v, kv_ref, decay)
        tol = 1e-5 if dtype == "fp32" else 1e-2
        parity.check(to_np(o), o_ref, 1, tol, out_bf16=(dtype == "bf16"), what="decode o")
        parity.check(to_np(kvd), kv_ref, 1, 1e-5, what="decode kv")


def test_prefill_then_decode(dev):
    """prefill(x[:L]) then decode(x[L]) matches the last row and state of the
    oracle's prefill over x[:L+1]; the GPU state is carried in place."""
    import torch
    import linear_attention_la_amd as la

    H, d = 4, 128
    lengths = [130, 64, 1, 257]
    decay = np.array([1.0, 0.99, 0.9, 0.6], np.float32)
    S = len(lengths)
    Ls = np.array(lengths)
    q, k, v = host_qkv(int(Ls.sum() + S), H, d, 77)
    # sequence s occupies rows [off_s, off_s + L_s + 1): prefix then one decode token
    offs = np.concatenate([[0], np.cumsum(Ls + 1)])[:-1]
    pre_idx = np.concatenate([np.arange(o, o + L) for o, L in zip(offs, Ls)])
    dec_idx = offs + Ls
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    _, kv = la.prefill(qd[pre_idx].contiguous(), kd[pre_idx].contiguous(),
                       vd[pre_idx].contiguous(), cu_seqlens(lengths), decay)
    o = la.decode(qd[dec_idx].contiguous(), kd[dec_idx].contiguous(), vd[dec_idx].contiguous(),
                  kv, decay)
    torch.cuda.synchronize()
    full = cu_seqlens(Ls + 1)
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, full, decay, beta=64)
    parity.check(to_np(o), o_ref[full[1:] - 1], 1, 1e-2, out_bf16=True, what="prefill+decode o")
    parity.check(to_np(kv), kv_ref, 1, 1e-2, what="prefill+decode kv")


def test_decode_full_batch_sampled(dev):
    """256 sequences x 64 heads x d=128 (the serving batch): sampled
    (sequence, head) pairs checked one by one against the oracle."""
    import torch
    import linear_attention_la_amd as la

    w = workload("mixed_decode")
    B, H, d = w["batch"], w["H"], w["d"]
    kvd = device_states(B, H, d, w["seed"], dev, scale=0.5)
    kv0 = kvd.clone()
    qd, kd, vd = (x.view(B, H, d) for x in device_qkv(B, H, d, w["seed"] + 1, dev))
    o = la.decode(qd, kd, vd, kvd, w["decay"])
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(9))
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 48), rng.integers(0, H, 48))]
    pairs += [(0, 0), (B - 1, H - 1)]
    for b, h in pairs:
        o_ref, s_ref = oracle.decode_step(to_np(qd[b, h]), to_np(kd[b, h]), to_np(vd[b, h]),
                                          to_np(kv0[b, h]), w["decay"][h])
        parity.check(to_np(o[b, h])[None], o_ref[None], 0, 1e-2, out_bf16=True,
                     what=f"decode ({b},{h}) o")
        parity.check(to_np(kvd[b, h])[None], s_ref[None], 0, 1e-5, what=f"decode ({b},{h}) kv")


def test_two_streams_bitwise(dev):
    """Decode on one stream concurrently with a packed prefill on another
    gives exactly the results each gives alone."""
    import torch
    import linear_attention_la_amd as la

    wp = workload("mixed_prefill")
    wd = workload("mixed_decode")
    B, H, d = wd["batch"], wd["H"], wd["d"]
    cu = cu_seqlens(wp["lengths"])
    T = int(cu[-1])
    say(f"two streams: prefill T={T}, decode B={B}")
    qp, kp, vp = device_qkv(T, H, d, wp["seed"], dev)
    qd, kd, vd = (x.view(B, H, d) for x in device_qkv(B, H, d, wd["seed"] + 1, dev))
    cu_s = cu_seqlens(wd["state_lengths"])
    qs, ks, vs = device_qkv(int(cu_s[-1]), H, d, wd["seed"] + 7, dev)
    _, kv_init = la.prefill(qs, ks, vs, torch.from_numpy(cu_s).to(dev), wd["decay"],
                            cu_seqlens_host=cu_s)
    cu_dev = torch.from_numpy(cu).to(dev)

    kv_a = kv_init.clone()
    o_dec_a = la.decode(qd, kd, vd, kv_a, wd["decay"])
    o_pre_a, kv_pre_a = la.prefill(qp, kp, vp, cu_dev, wp["decay"])
    torch.cuda.synchronize()

    sp, sd = torch.cuda.Stream(), torch.cuda.Stream()
    kv_b = kv_init.clone()
    o_pre_b = torch.empty_like(o_pre_a)
    kv_pre_b = torch.empty_like(kv_pre_a)
    o_dec_b = torch.empty_like(o_dec_a)
    torch.cuda.synchronize()
    for _ in range(3):
        kv_b.copy_(kv_init)
        torch.cuda.synchronize()
        la.prefill(qp, kp, vp, cu_dev, wp["decay"], stream=sp, out=o_pre_b, kv_final=kv_pre_b)
        la.decode(qd, kd, vd, kv_b, wd["decay"], stream=sd, out=o_dec_b)
        torch.cuda.synchronize()
        assert torch.equal(o_dec_a, o_dec_b)
        assert torch.equal(kv_a, kv_b)
        assert torch.equal(o_pre_a, o_pre_b)
        assert torch.equal(kv_pre_a, kv_pre_b)


def test_serving_step_two_streams_oracle(dev):
    """The mixed serving step -- the 256 x 64 decode batch, its states made by
    a seeded prefill of 256 sequences of U[256, 2048] tokens, beside a packed
    prefill of 8 sequences of U[1K, 32K] tokens (the one-workgroup-per-chain
    kernel) -- run concurrently on two streams, with either kernel submitted
    first, on plain streams and on streams restricted to disjoint sets of
    compute units: every run equals the solo run bit for bit, and the solo
    run matches the oracle (three heads over all 8 prefill sequences, with
    their final states; 50 sampled decode pairs, each from the oracle's own
    prefill of its state's sequence)."""
    import torch
    import linear_attention_la_amd as la

    wp = workload("mixed_prefill")
    wd = workload("mixed_decode")
    B, H, d = wd["batch"], wd["H"], wd["d"]
    cu = cu_seqlens(wp["lengths"])
    T = int(cu[-1])
    qp, kp, vp = device_qkv(T, H, d, wp["seed"], dev)
    qd, kd, vd = (x.view(B, H, d) for x in device_qkv(B, H, d, wd["seed"] + 1, dev))
    cu_s = cu_seqlens(wd["state_lengths"])
    qs, ks, vs = device_qkv(int(cu_s[-1]), H, d, wd["seed"] + 7, dev)
    _, kv_init = la.prefill(qs, ks, vs, torch.from_numpy(cu_s).to(dev), wd["decay"],
                            cu_seqlens_host=cu_s)
    cu_dev = torch.from_numpy(cu).to(dev)

    kv_solo = kv_init.clone()
    o_dec = la.decode(qd, kd, vd, kv_solo, wd["decay"])
    o_pre, kv_pre = la.prefill(qp, kp, vp, cu_dev, wp["decay"])
    torch.cuda.synchronize()

    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    n_dec = max(1, n_cu // 8)
    dec_mask = (1 << n_dec) - 1
    pre_mask = ((1 << n_cu) - 1) & ~dec_mask
    plain = (torch.cuda.Stream(), torch.cuda.Stream())
    masked = (la.cu_masked_stream(pre_mask), la.cu_masked_stream(dec_mask))
    for name, (sp, sd) in (("plain", plain), ("cu-masked", masked)):
        for decode_first in (True, False):
            say(f"serving step: {name} streams, decode first={decode_first}")
            kv_b = kv_init.clone()
            o_pre_b, kv_pre_b = torch.empty_like(o_pre), torch.empty_like(kv_pre)
            o_dec_b = torch.empty_like(o_dec)
            torch.cuda.synchronize()
            run_pre = lambda: la.prefill(qp, kp, vp, cu_dev, wp["decay"], stream=sp,  # noqa
                                         out=o_pre_b, kv_final=kv_pre_b, cu_seqlens_host=cu)
            run_dec = lambda: la.decode(qd, kd, vd, kv_b, wd["decay"], stream=sd,  # noqa
                                        out=o_dec_b)
            (run_dec, run_pre)[0 if decode_first else 1]()
            (run_pre, run_dec)[0 if decode_first else 1]()
            torch.cuda.synchronize()
            assert torch.equal(o_dec_b, o_dec) and torch.equal(kv_b, kv_solo)
            assert torch.equal(o_pre_b, o_pre) and torch.equal(kv_pre_b, kv_pre)

    heads = [0, 31, 63]
    q_h, k_h, v_h = (to_np(x[:, heads]) for x in (qp, kp, vp))
    dec_h = np.asarray(wp["decay"], np.float32)[heads]
    o_ref, kv_ref = oracle.prefill_varlen(q_h, k_h, v_h, cu, dec_h, beta=64)
    s1 = parity.check(to_np(o_pre[:, heads]), o_ref, 1, 1e-2, out_bf16=True,
                      what="serving prefill o")
    s2 = parity.check(to_np(kv_pre[:, heads]), kv_ref, 1, 1e-2, what="serving prefill kv")
    say("serving prefill", s1, s2)
    rng = np.random.Generator(np.random.PCG64(11))
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 48), rng.integers(0, H, 48))]
    pairs += [(0, 0), (B - 1, H - 1)]
    for b, h in pairs:
        rows = slice(int(cu_s[b]), int(cu_s[b + 1]))
        _, s0_ref = oracle.prefill_varlen(*(to_np(x[rows, h:h + 1]) for x in (qs, ks, vs)),
                                          [0, rows.stop - rows.start],
                                          np.asarray(wd["decay"])[h:h + 1])
        parity.check(to_np(kv_init[b, h])[None], s0_ref[0], 0, 1e-2,
                     what=f"serving state prefill ({b},{h})")
        od_ref, sd_ref = oracle.decode_step(to_np(qd[b, h]), to_np(kd[b, h]), to_np(vd[b, h]),
                                            s0_ref[0, 0], wd["decay"][h])
        parity.check(to_np(o_dec[b, h])[None], od_ref[None], 0, 1e-2, out_bf16=True,
                     what=f"serving decode ({b},{h}) o")
        parity.check(to_np(kv_solo[b, h])[None], sd_ref[None], 0, 1e-5,
                     what=f"serving decode ({b},{h}) kv")
