"""GPU parity of la_prefill_segmented (sequences cut into parallel segments)
against the fp64 oracle, and its agreement with la_prefill (needs an MI355X)."""

import numpy as np
import pytest

import oracle
from la_inputs import cu_seqlens, device_qkv, host_qkv, random_states, workload
from tests import parity
from tests.gpu_util import device, say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _run(dev, lengths, H, d, decay, seed, segment_len, kv_init=False, out_f32=False,
         in_place=False):
    import torch
    import linear_attention_la_amd as la

    say(f"case segmented lengths={list(lengths)[:8]} H={H} d={d} segment_len={segment_len} "
        f"kv_init={kv_init} out_f32={out_f32} in_place={in_place}")
    T = int(sum(lengths))
    q, k, v = host_qkv(T, H, d, seed, "bf16")
    cu = cu_seqlens(lengths)
    kv0 = random_states(len(lengths), H, d, seed + 7, scale=0.1) if kv_init else None
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    kv0d = to_dev(kv0, torch.float32, dev) if kv_init else None
    o, kv = la.prefill_segmented(qd, kd, vd, cu, decay, segment_len, kv_init=kv0d,
                                 out_dtype=torch.float32 if out_f32 else None,
                                 kv_final=kv0d if in_place else None)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, kv_init=kv0)
    return to_np(o), to_np(kv), o_ref, kv_ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("segment_len", [64, 128, 192])
def test_ragged_segments(dev, d, segment_len):
    """Lengths below, at and across segment boundaries (empty, 1, 63..65,
    several segments plus a tail), decays from none to strong."""
    lengths = [1, 63, 64, 65, 129, 0, 300, 17, 450]
    decay = np.array([1.0, 0.99, 0.9, 0.5], np.float32)
    o, kv, o_ref, kv_ref = _run(dev, lengths, 4, d, decay, 31 + d + segment_len, segment_len)
    s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what="segmented o")
    s2 = parity.check(kv, kv_ref, 1, 1e-2, what="segmented kv")
    say("segmented ragged", s1, s2)


@pytest.mark.parametrize("in_place", [False, True])
def test_kv_init_and_fp32_out(dev, in_place):
    """Initial states carried into the first segment; fp32 output; the final
    state written over kv_init (in-place continuation)."""
    lengths = [200, 0, 513]
    decay = np.array([0.999, 0.97, 0.8], np.float32)
    o, kv, o_ref, kv_ref = _run(dev, lengths, 3, 128, decay, 77, 128, kv_init=True, out_f32=True,
                                in_place=in_place)
    parity.check(o, o_ref, 1, 1e-2, what="segmented kv_init o")
    parity.check(kv, kv_ref, 1, 1e-2, what="segmented kv_init kv")


def test_long_sequence_two_heads(dev):
    """One 65,536-token sequence, 2 heads, 16 segments of 4096: every output
    and the final state against the oracle."""
    w = workload("sweep65536")
    decay = np.asarray(w["decay"][:2], np.float32)
    o, kv, o_ref, kv_ref = _run(dev, [65536], 2, 128, decay, 91, 4096)
    s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what="segmented 64K o")
    s2 = parity.check(kv, kv_ref, 1, 1e-2, what="segmented 64K kv")
    say("segmented 64K", s1, s2)


def test_matches_unsegmented_n8k(dev):
    """B=1, H=64, N=8192 with 4 segments agrees with la_prefill to the
    oracle tolerance on every head (same inputs, different fp32 sum order)."""
    import torch
    import linear_attention_la_amd as la

    w = workload("n8k")
    say("case segmented vs la_prefill n8k")
    q, k, v = device_qkv(8192, 64, 128, w["seed"], dev)
    cu = torch.tensor([0, 8192], dtype=torch.int32, device=dev)
    o1, kv1 = la.prefill(q, k, v, cu, w["decay"], cu_seqlens_host=[0, 8192])
    o2, kv2 = la.prefill_segmented(q, k, v, cu, w["decay"], 2048, cu_seqlens_host=[0, 8192])
    torch.cuda.synchronize()
    s1 = parity.check(to_np(o2), to_np(o1), 1, 1e-2, out_bf16=True, what="seg vs plain o")
    s2 = parity.check(to_np(kv2), to_np(kv1), 1, 1e-2, what="seg vs plain kv")
    say("segmented vs plain", s1, s2)


def test_caller_workspace_reused(dev):
    """A caller-provided workspace serves two calls of different sizes."""
    import torch
    import linear_attention_la_amd as la

    decay = np.array([0.95, 0.6], np.float32)
    big = la.prefill_segmented_workspace_size(cu_seqlens([700, 300]), 2, 128, 128)
    ws = torch.empty(big, dtype=torch.uint8, device=dev)
    for lengths, seed in (([700, 300], 5), ([130], 6)):
        say(f"case workspace reuse lengths={lengths}")
        T = sum(lengths)
        q, k, v = host_qkv(T, 2, 128, seed, "bf16")
        cu = cu_seqlens(lengths)
        qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
        o, kv = la.prefill_segmented(qd, kd, vd, cu, decay, 128, workspace=ws)
        torch.cuda.synchronize()
        o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay)
        parity.check(to_np(o), o_ref, 1, 1e-2, out_bf16=True, what="workspace reuse o")
        parity.check(to_np(kv), kv_ref, 1, 1e-2, what="workspace reuse kv")


@pytest.mark.parametrize("d", [64, 128])
def test_many_sequences(dev, d):
    """1,100 sequences of 0..160 tokens: the plan spreads more than 1,024
    sequences over its threads (two per thread) and every wave of its
    prefix sum carries segments."""
    rng = np.random.default_rng(1234 + d)
    lengths = [int(x) for x in rng.integers(0, 161, size=1100)]
    decay = np.array([0.97], np.float32)
    o, kv, o_ref, kv_ref = _run(dev, lengths, 1, d, decay, 41 + d, 64)
    s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what="segmented many o")
    s2 = parity.check(kv, kv_ref, 1, 1e-2, what="segmented many kv")
    say("segmented many sequences", s1, s2)


def test_bench_config_one_million_tokens(dev):
    """The segmented launch the bench times: B=1, H=8, N=1,048,576, d=128,
    segments of 32,768 (256 (segment, head) items of the chained scan); the
    heads of strongest and weakest decay checked over all 1M tokens, and the
    final states of all heads."""
    import torch
    import linear_attention_la_amd as la

    w = workload("n1m")
    N, H = w["lengths"][0], 8
    decay = np.asarray(w["decay"][:H], np.float32)
    say("case segmented bench config H=8 N=1M")
    qd, kd, vd = device_qkv(N, H, 128, 1006, dev)
    cu = np.array([0, N], np.int32)
    o, kv = la.prefill_segmented(qd, kd, vd, cu, decay, 32768)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    heads = sorted({int(np.argmin(decay)), int(np.argmax(decay))})
    for h in heads:
        sl = lambda x: to_np(x[:, h, :])[:, None, :]  # noqa: E731
        o_ref, kv_ref = oracle.prefill_varlen(sl(qd), sl(kd), sl(vd), cu, decay[h:h + 1], beta=256)
        s1 = parity.check(to_np(o[:, h, :])[:, None, :], o_ref, 1, 1e-2, out_bf16=True,
                          what=f"segmented 1M o head {h}")
        s2 = parity.check(to_np(kv[:, h])[:, None], kv_ref, 1, 1e-2,
                          what=f"segmented 1M kv head {h}")
        say("segmented 1M head", h, s1, s2)
    del qd, kd, vd, o, kv
    torch.cuda.empty_cache()


def test_auto_segment_len_bitwise(dev):
    """segment_len 0 lets the library choose about one (segment, head) item per
    compute unit: the forward (the chained scan) and the segmented backward
    then equal, bit for bit, the calls with that length given explicitly."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv, device_states

    lengths, H = [5000, 0, 2304, 640], 8
    cu_h = cu_seqlens(lengths)
    T, S = int(cu_h[-1]), len(lengths)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    seg = max(64, -(-(-(-T * H // cus)) // 64) * 64)
    say(f"case auto segment_len lengths={lengths} H={H} -> {seg}")
    q, k, v = device_qkv(T, H, 128, 531, dev)
    do = device_qkv(T, H, 128, 532, dev)[0]
    kv0 = device_states(S, H, 128, 533, dev, scale=0.1)
    g = device_states(S, H, 128, 534, dev, scale=0.1)
    cu = torch.from_numpy(cu_h).to(dev)
    decay = np.exp(-np.linspace(0.001, 0.1, H)).astype(np.float32)
    assert la.prefill_segmented_workspace_size(cu_h, H, 128, 0) == \
        la.prefill_segmented_workspace_size(cu_h, H, 128, seg)
    o0, s0 = la.prefill_segmented(q, k, v, cu, decay, 0, kv_init=kv0, cu_seqlens_host=cu_h)
    o1, s1 = la.prefill_segmented(q, k, v, cu, decay, seg, kv_init=kv0, cu_seqlens_host=cu_h)
    b0 = la.prefill_backward_segmented(q, k, v, do, cu, decay, 0, kv_init=kv0, dkv_final=g,
                                       cu_seqlens_host=cu_h)
    b1 = la.prefill_backward_segmented(q, k, v, do, cu, decay, seg, kv_init=kv0, dkv_final=g,
                                       cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(s0, s1), "forward"
    for name, x0, x1 in zip(("dq", "dk", "dv", "dkv_init"), b0, b1):
        assert torch.equal(x0, x1), name
