"""GPU parity of la_prefill_backward_segmented (the backward with every
sequence cut into segments) against the fp64 oracle backward and against
la_prefill_backward (needs an MI355X)."""

import numpy as np
import pytest

import oracle
from la_inputs import cu_seqlens, host_qkv, random_states
from tests import parity
from tests.gpu_util import device, say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _inputs(dev, lengths, H, d, seed, kv_init, dkv_final):
    import torch

    T, S = int(sum(lengths)), len(lengths)
    q, k, v = host_qkv(T, H, d, seed, "bf16")
    do = host_qkv(T, H, d, seed + 1, "bf16")[0]
    kv0 = random_states(S, H, d, seed + 7, scale=0.1) if kv_init else None
    g = random_states(S, H, d, seed + 9, scale=0.1) if dkv_final else None
    dv_ = [to_dev(x, torch.bfloat16, dev) for x in (q, k, v, do)]
    kv0d = to_dev(kv0, torch.float32, dev) if kv_init else None
    gd = to_dev(g, torch.float32, dev) if dkv_final else None
    return (q, k, v, do, kv0, g), (*dv_, kv0d, gd)


def _check(gpu, ref, f32, heads=None, what=""):
    sel = (lambda x: x) if heads is None else (lambda x: x[:, list(heads)])
    stats = [parity.check(sel(to_np(a)), sel(b), 1, 1e-2, out_bf16=not f32, what=f"{what} {n}")
             for n, a, b in zip(("dq", "dk", "dv"), gpu[:3], ref[:3])]
    stats.append(parity.check(sel(to_np(gpu[3])), sel(ref[3]), 1, 1e-2, what=f"{what} dkv_init"))
    return stats


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("segment_len", [64, 128])
@pytest.mark.parametrize("kv_init,dkv_final", [(True, True), (False, True), (True, False),
                                                (False, False)])
def test_segmented_backward_ragged(dev, d, segment_len, kv_init, dkv_final):
    """Lengths around the segment and block edges (empty, 1, 63..65, 127..129,
    several segments plus a tail) against the oracle's backward."""
    import torch
    import linear_attention_la_amd as la

    lengths = [1, 63, 64, 65, 129, 0, 300, 127, 17]
    decay = np.array([1.0, 0.99, 0.9, 0.5], np.float32)
    say(f"case segmented backward d={d} segment_len={segment_len} kv_init={kv_init} "
        f"dkv_final={dkv_final}")
    host, devs = _inputs(dev, lengths, 4, d, 301 + d + segment_len, kv_init, dkv_final)
    cu = cu_seqlens(lengths)
    out = la.prefill_backward_segmented(*devs[:4], cu, decay, segment_len, kv_init=devs[4],
                                        dkv_final=devs[5])
    torch.cuda.synchronize()
    ref = oracle.backward_varlen(*host[:4], cu, decay, kv_init=host[4], dkv_final=host[5])
    say("  ", _check(out, ref, False, what="ragged"))


def test_segmented_backward_fp32_grads(dev):
    import torch
    import linear_attention_la_amd as la

    lengths = [700, 0, 130]
    decay = np.array([0.999, 0.97, 0.8], np.float32)
    say("case segmented backward fp32 grads")
    host, devs = _inputs(dev, lengths, 3, 128, 331, True, True)
    cu = cu_seqlens(lengths)
    out = la.prefill_backward_segmented(*devs[:4], cu, decay, 192, kv_init=devs[4],
                                        dkv_final=devs[5], grad_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.backward_varlen(*host[:4], cu, decay, kv_init=host[4], dkv_final=host[5])
    say("  ", _check(out, ref, True, what="fp32 grads"))


def test_segmented_backward_wide_path(dev):
    """One sequence of 16K tokens x 16 heads in segments of 1024: 256
    (segment, head) chains, so every pass runs the one-workgroup-per-chain
    kernel (reverse-time state pass included); three heads against the
    oracle."""
    import torch
    import linear_attention_la_amd as la

    H, N = 16, 16384
    rng = np.random.default_rng(17)
    decay = np.exp(-rng.uniform(0.001, 0.1, H)).astype(np.float32)
    decay[0] = 1.0
    heads = [0, int(np.argmin(decay)), 7]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert (N // 1024) * H >= cus
    say("case segmented backward wide path")
    host, devs = _inputs(dev, [N], H, 128, 341, True, True)
    cu = cu_seqlens([N])
    out = la.prefill_backward_segmented(*devs[:4], cu, decay, 1024, kv_init=devs[4],
                                        dkv_final=devs[5])
    torch.cuda.synchronize()
    ref = oracle.backward_varlen(*host[:4], cu, decay, kv_init=host[4], dkv_final=host[5],
                                 heads=heads)
    say("  ", _check(out, ref, False, heads=heads, what="wide"))


def test_segmented_backward_matches_plain(dev):
    """Against la_prefill_backward on the same inputs (every head): the two
    differ only in the order of fp32 sums."""
    import torch
    import linear_attention_la_amd as la

    lengths = [3000, 1100, 64]
    decay = np.array([1.0, 0.995, 0.95, 0.8, 0.6, 0.9], np.float32)
    say("case segmented backward vs plain")
    _, devs = _inputs(dev, lengths, 6, 128, 351, True, True)
    cu = cu_seqlens(lengths)
    seg = la.prefill_backward_segmented(*devs[:4], cu, decay, 256, kv_init=devs[4],
                                        dkv_final=devs[5], grad_dtype=torch.float32)
    plain = la.prefill_backward(*devs[:4], cu, decay, kv_init=devs[4], dkv_final=devs[5],
                                grad_dtype=torch.float32)
    torch.cuda.synchronize()
    stats = [parity.check(to_np(a), to_np(b).astype(np.float64), 1, 1e-4, what=n)
             for n, a, b in zip(("dq", "dk", "dv", "dkv_init"), seg, plain)]
    say("  ", stats)


def test_segmented_backward_side_stream_workspace_reuse(dev):
    """Two calls on a side stream sharing one workspace (a different batch
    each time, the second one smaller) give exactly what fresh calls on the
    default stream give."""
    import torch
    import linear_attention_la_amd as la

    decay = np.array([0.98, 0.9], np.float32)
    side = torch.cuda.Stream()
    cases = [([500, 64, 1], 371), ([200, 3], 381)]
    cu0 = cu_seqlens(cases[0][0])
    ws = torch.empty(la.prefill_backward_segmented_workspace_size(cu0, 2, 128, 128),
                     dtype=torch.uint8, device=dev)
    for lengths, seed in cases:
        say(f"case segmented backward side stream lengths={lengths}")
        _, devs = _inputs(dev, lengths, 2, 128, seed, True, True)
        cu = cu_seqlens(lengths)
        ref = la.prefill_backward_segmented(*devs[:4], cu, decay, 128, kv_init=devs[4],
                                            dkv_final=devs[5])
        torch.cuda.synchronize()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            out = la.prefill_backward_segmented(*devs[:4], cu, decay, 128, kv_init=devs[4],
                                                dkv_final=devs[5], stream=side, workspace=ws)
        side.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b)


def test_bench_config_one_million_tokens(dev):
    """The segmented backward the bench times: B=1, H=8, N=1,048,576, d=128,
    segments of 32,768, with S0 and dS_L.  dQ at a token depends only on the
    tokens up to it and S0, and dK, dV only on the tokens from it on and
    dS_L, so the oracle backward of the first 8192 tokens (with S0) gives dQ
    there and that of the last 8192 tokens (with dS_L) gives dK and dV there,
    for the heads of strongest and weakest decay; every output of every head
    is also compared with la_prefill_backward (fp32 gradients: the two differ
    only in the order of fp32 sums)."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv, device_states, workload

    w = workload("n1m")
    N, H, d, P = w["lengths"][0], 8, 128, 8192
    decay = np.asarray(w["decay"][:H], np.float32)
    say("case segmented backward bench config H=8 N=1M")
    q, k, v = device_qkv(N, H, d, 1007, dev)
    do = device_qkv(N, H, d, 1008, dev)[0]
    kv0 = device_states(1, H, d, 1009, dev, scale=0.1)
    g = device_states(1, H, d, 1010, dev, scale=0.1)
    cu = np.array([0, N], np.int32)
    seg = la.prefill_backward_segmented(q, k, v, do, cu, decay, 32768, kv_init=kv0, dkv_final=g,
                                        grad_dtype=torch.float32)
    torch.cuda.synchronize()
    heads = sorted({int(np.argmin(decay)), int(np.argmax(decay))})
    pre = [to_np(x[:P][:, heads]) for x in (q, k, v, do)]
    ref = oracle.backward_varlen(*pre, [0, P], decay[heads], kv_init=to_np(kv0[:, heads]))
    s1 = parity.check(to_np(seg[0][:P][:, heads]), ref[0], 1, 1e-2, what="1M dq (first 8K)")
    suf = [to_np(x[N - P:][:, heads]) for x in (q, k, v, do)]
    ref = oracle.backward_varlen(*suf, [0, P], decay[heads], dkv_final=to_np(g[:, heads]))
    s2 = parity.check(to_np(seg[1][N - P:][:, heads]), ref[1], 1, 1e-2, what="1M dk (last 8K)")
    s3 = parity.check(to_np(seg[2][N - P:][:, heads]), ref[2], 1, 1e-2, what="1M dv (last 8K)")
    say("  oracle", s1, s2, s3)
    plain = la.prefill_backward(q, k, v, do, cu, decay, kv_init=kv0, dkv_final=g,
                                grad_dtype=torch.float32)
    torch.cuda.synchronize()
    # per head on the device (1M x 8 x 128 is too large to move to the host
    # in float64): relative L2 and largest element over the head's rms
    for n, a, b in zip(("dq", "dk", "dv", "dkv_init"), seg, plain):
        a64 = a.double().transpose(0, 1).reshape(H, -1)
        b64 = b.double().transpose(0, 1).reshape(H, -1)
        nb = torch.linalg.vector_norm(b64, dim=1)
        rel = torch.linalg.vector_norm(a64 - b64, dim=1) / nb
        worst = (a64 - b64).abs().amax(dim=1) / (nb / b64.shape[1] ** 0.5)
        say("  vs plain", n, float(rel.max()), float(worst.max()))
        assert bool(torch.isfinite(rel).all()) and float(rel.max()) <= 1e-4, n
        assert float(worst.max()) <= 2e-2, n
    del q, k, v, do, seg, plain
    torch.cuda.empty_cache()
