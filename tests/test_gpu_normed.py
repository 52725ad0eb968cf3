"""GPU parity of the fused output normalisation (la_prefill_normed,
la_decode_normed) against the fp64 oracle: the oracle's prefill or decode
output passed through oracle.norm_gate (needs an MI355X)."""

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


def _weights(H, d, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.uniform(0.5, 1.5, (H, d)).astype(np.float32)


def _prefill_case(dev, lengths, H, decay, seed, gate, out_f32, kv_init, heads):
    import torch
    import linear_attention_la_amd as la

    d = 128
    say(f"case normed prefill lengths={lengths[:6]} H={H} gate={gate} out_f32={out_f32} "
        f"kv_init={kv_init}")
    T = int(sum(lengths))
    q, k, v = host_qkv(T, H, d, seed, "bf16")
    g = host_qkv(T, H, d, seed + 1, "bf16")[0] * 20.0 if gate else None  # gate logits ~ N(0, 3)
    cu = cu_seqlens(lengths)
    kv0 = random_states(len(lengths), H, d, seed + 2, scale=0.1) if kv_init else None
    w = _weights(H, d, seed + 3)
    eps = 1e-5
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    gd = to_dev(g, torch.bfloat16, dev) if gate else None
    g_exact = to_np(gd) if gate else None  # the gate values as the GPU sees them
    kv0d = to_dev(kv0, torch.float32, dev) if kv_init else None
    y, kv = la.prefill_normed(qd, kd, vd, cu, decay, to_dev(w, torch.float32, dev), eps, gd,
                              kv_init=kv0d, out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.prefill_varlen(q[:, heads], k[:, heads], v[:, heads], cu,
                                          np.asarray(decay)[heads],
                                          kv_init=None if kv0 is None else kv0[:, heads])
    y_ref = oracle.norm_gate(o_ref, w[heads], eps, None if g_exact is None else g_exact[:, heads])
    s1 = parity.check(to_np(y)[:, heads], y_ref, 1, 1e-2, out_bf16=not out_f32,
                      what="normed prefill y")
    s2 = parity.check(to_np(kv)[:, heads], kv_ref, 1, 1e-2, what="normed prefill kv")
    say("normed prefill", s1, s2)
    return y


@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("out_f32", [False, True])
def test_prefill_normed_wide(dev, gate, out_f32):
    """320 (sequence, head) pairs: one workgroup per pair, epilogue fused into
    its output write; ragged lengths incl. empty, 1 and block edges."""
    H = 64
    lengths = [1, 63, 300, 0, 129]
    decay = np.exp(-np.linspace(0.001, 0.1, H)).astype(np.float32)
    decay[0] = 1.0
    _prefill_case(dev, lengths, H, decay, 301 + gate + 2 * out_f32, gate, out_f32, kv_init=True,
                  heads=[0, 1, 31, 63])


@pytest.mark.parametrize("gate", [False, True])
def test_prefill_normed_scan(dev, gate):
    """Few pairs (3 sequences x 4 heads): the chained scan over segments of
    a length the library picks, epilogue fused into the output pass."""
    decay = np.array([1.0, 0.99, 0.9, 0.5], np.float32)
    _prefill_case(dev, [700, 0, 333], 4, decay, 311 + gate, gate, False, kv_init=True,
                  heads=[0, 1, 2, 3])


def test_prefill_normed_long_single(dev):
    """One 8192-token sequence x 16 heads (the scan, 16 segments a head)."""
    decay = np.exp(-np.linspace(0.001, 0.1, 16)).astype(np.float32)
    _prefill_case(dev, [8192], 16, decay, 321, True, False, kv_init=False, heads=[0, 7, 15])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("gate", [False, True])
def test_decode_normed(dev, d, dtype, gate):
    import torch
    import linear_attention_la_amd as la

    B, H = 5, 3
    decay = np.array([1.0, 0.97, 0.5], np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"case normed decode d={d} dtype={dtype} gate={gate}")
    kv = random_states(B, H, d, 331 + d)
    kvd = to_dev(kv, torch.float32, dev)
    q, k, v = (x[:B * H].reshape(B, H, d) for x in host_qkv(B * H, 1, d, 332 + d, dtype))
    g = host_qkv(B * H, 1, d, 333 + d, dtype)[0][:B * H].reshape(B, H, d) * 20.0 if gate else None
    w = _weights(H, d, 334)
    gd = to_dev(g, tdt, dev) if gate else None
    y = la.decode_normed(to_dev(q, tdt, dev), to_dev(k, tdt, dev), to_dev(v, tdt, dev), kvd, decay,
                         to_dev(w, torch.float32, dev), 1e-5, gd)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.decode_batch(to_np(to_dev(q, tdt, dev)), to_np(to_dev(k, tdt, dev)),
                                        to_np(to_dev(v, tdt, dev)), kv, decay)
    y_ref = oracle.norm_gate(o_ref, w, 1e-5, to_np(gd) if gate else None)
    tol = 1e-5 if dtype == "fp32" else 1e-2
    parity.check(to_np(y), y_ref, 1, tol, out_bf16=(dtype == "bf16"), what="normed decode y")
    parity.check(to_np(kvd), kv_ref, 1, 1e-5, what="normed decode kv")


def test_prefill_normed_unit_weight_matches_plain(dev):
    """With unit weights and no gate, the normed output of the wide path is
    the plain output normalised: checked against la_prefill's output rows
    normalised on the host (both from the same kernel's fp32 sums, so they
    agree to the output rounding)."""
    import torch
    import linear_attention_la_amd as la

    H, d, lengths = 64, 128, [200, 100, 57, 90]
    T = sum(lengths)
    q, k, v = (to_dev(x, torch.bfloat16, dev) for x in host_qkv(T, H, d, 341, "bf16"))
    decay = np.full(H, 0.95, np.float32)
    o, _ = la.prefill(q, k, v, cu_seqlens(lengths), decay, out_dtype=torch.float32)
    y, _ = la.prefill_normed(q, k, v, cu_seqlens(lengths), decay,
                             torch.ones((H, d), dtype=torch.float32, device=dev), 1e-6,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.norm_gate(to_np(o), np.ones((H, d)), 1e-6)
    parity.check(to_np(y), ref, 1, 1e-5, what="normed vs plain")


@pytest.mark.parametrize("name", ["n8k", "batch8_n8k"])
def test_prefill_normed_bench_shapes(dev, name):
    """The launches the bench times, at full size with a gate: B=1, H=64,
    N=8192 (the chained scan, segments of 2048) and eight 8K sequences
    (one workgroup per chain); three heads of every sequence against the
    oracle, on the bench's own device-generated inputs."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv, workload

    w = workload(name)
    H, d = 64, 128
    cu = cu_seqlens(w["lengths"])
    T = int(cu[-1])
    say(f"case normed bench shape {name} T={T}")
    q, k, v = device_qkv(T, H, d, w["seed"], dev)
    g = device_qkv(T, H, d, w["seed"] + 21, dev)[0]
    wt = _weights(H, d, 351)
    y, kv = la.prefill_normed(q, k, v, cu, w["decay"], to_dev(wt, torch.float32, dev), 1e-6, g)
    torch.cuda.synchronize()
    heads = [0, 37, 63]
    qh, kh, vh, gh = (to_np(x[:, heads]) for x in (q, k, v, g))
    o_ref, kv_ref = oracle.prefill_varlen(qh, kh, vh, cu, np.asarray(w["decay"])[heads])
    y_ref = oracle.norm_gate(o_ref, wt[heads], 1e-6, gh)
    s1 = parity.check(to_np(y[:, heads]), y_ref, 1, 1e-2, out_bf16=True, what=f"normed {name} y")
    s2 = parity.check(to_np(kv[:, heads]), kv_ref, 1, 1e-2, what=f"normed {name} kv")
    say(f"normed {name}", s1, s2)


def test_decode_normed_full_batch_sampled(dev):
    """la_decode_normed on the serving batch the bench times (256 sequences x
    64 heads x d=128, bf16, with a gate): sampled (sequence, head) pairs
    checked one by one against the oracle's decode step and norm_gate."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv, device_states, workload

    w = workload("mixed_decode")
    B, H, d = w["batch"], w["H"], w["d"]
    say(f"case normed decode full batch B={B} H={H}")
    kvd = device_states(B, H, d, w["seed"], dev, scale=0.5)
    kv0 = kvd.clone()
    qd, kd, vd = (x.view(B, H, d) for x in device_qkv(B, H, d, w["seed"] + 1, dev))
    gd = device_qkv(B, H, d, w["seed"] + 3, dev)[0].view(B, H, d)
    wt = _weights(H, d, 361)
    y = la.decode_normed(qd, kd, vd, kvd, w["decay"], to_dev(wt, torch.float32, dev), 1e-6, gd)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(19))
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 32), rng.integers(0, H, 32))]
    pairs += [(0, 0), (B - 1, H - 1)]
    for b, h in pairs:
        o_ref, s_ref = oracle.decode_step(to_np(qd[b, h]), to_np(kd[b, h]), to_np(vd[b, h]),
                                          to_np(kv0[b, h]), w["decay"][h])
        y_ref = oracle.norm_gate(o_ref[None, None], wt[h][None], 1e-6,
                                 to_np(gd[b, h])[None, None])[0]
        parity.check(to_np(y[b, h])[None], y_ref, 0, 1e-2, out_bf16=True,
                     what=f"normed decode ({b},{h}) y")
        parity.check(to_np(kvd[b, h])[None], s_ref[None], 0, 1e-5,
                     what=f"normed decode ({b},{h}) kv")


@pytest.mark.parametrize("name", ["n8k", "batch8_n8k"])
def test_gate_limits_bitwise(dev, name):
    """At the bench's launches: a gate of 0 gives sigmoid 1/2, so exactly half
    the ungated output, and a gate of 64 gives sigmoid 1 in fp32, so exactly
    the ungated output (both bit for bit: the scale 1/2 and the rounding
    commute)."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv, workload

    w = workload(name)
    cu = cu_seqlens(w["lengths"])
    T, H, d = int(cu[-1]), 64, 128
    say(f"case gate limits {name}")
    q, k, v = device_qkv(T, H, d, w["seed"], dev)
    wt = to_dev(_weights(H, d, 371), torch.float32, dev)
    y0, _ = la.prefill_normed(q, k, v, cu, w["decay"], wt, 1e-6, None)
    yz, _ = la.prefill_normed(q, k, v, cu, w["decay"], wt, 1e-6, torch.zeros_like(q))
    y1, _ = la.prefill_normed(q, k, v, cu, w["decay"], wt, 1e-6, torch.full_like(q, 64.0))
    torch.cuda.synchronize()
    assert torch.equal(yz, y0 * 0.5), "gate 0"
    assert torch.equal(y1, y0), "gate 64"


@pytest.mark.parametrize("lengths,H,tail", [([640] * 5, 64, [4]),
                                            ([600, 700, 640, 640, 640], 64, [0]),
                                            ([3072] * 33, 8, [32])])
def test_prefill_normed_split(dev, lengths, H, tail):
    """Pairs past one whole wave of the one-workgroup-per-pair kernel (320 or
    264 pairs on 256 compute units): the sequences of the wave run on that
    kernel, the remaining ones (consecutive in the index order) through the
    chained scan.  Every sequence's output and final state equal, bit for
    bit, those of a call on its own part alone (the wave's sequences: one
    workgroup per pair; the rest: the scan, with the same segments) and
    those of the same call in place, and the call matches the oracle on
    four heads."""
    import torch
    import linear_attention_la_amd as la

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"the split planned here assumes 256 compute units, not {cus}")
    d = 128
    say(f"case normed split lengths={lengths[:6]} H={H} tail={tail}")
    T, S = int(sum(lengths)), len(lengths)
    cu = cu_seqlens(lengths)
    q, k, v = host_qkv(T, H, d, 411, "bf16")
    g = host_qkv(T, H, d, 412, "bf16")[0] * 20.0
    kv0 = random_states(S, H, d, 413, scale=0.1)
    w = _weights(H, d, 414)
    decay = np.exp(-np.linspace(0.001, 0.1, H)).astype(np.float32)
    qd, kd, vd, gd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v, g))
    kv0d = to_dev(kv0, torch.float32, dev)
    wd = to_dev(w, torch.float32, dev)
    assert la.prefill_normed_workspace_size(cu, H, d) > 0, "no scan part planned"
    y, kv = la.prefill_normed(qd, kd, vd, cu, decay, wd, 1e-5, gd, kv_init=kv0d,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()

    def alone(seqs):
        rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
        idx = torch.from_numpy(rows).to(dev)
        part = [lengths[s] for s in seqs]
        yp, kvp = la.prefill_normed(qd[idx].contiguous(), kd[idx].contiguous(),
                                    vd[idx].contiguous(), cu_seqlens(part), decay, wd, 1e-5,
                                    gd[idx].contiguous(), kv_init=kv0d[seqs].contiguous(),
                                    out_dtype=torch.float32)
        torch.cuda.synchronize()
        return idx, yp, kvp

    for seqs in ([s for s in range(S) if s not in tail], tail):
        idx, yp, kvp = alone(seqs)
        assert torch.equal(y[idx], yp), f"sequences {seqs[:4]}...: rows"
        assert torch.equal(kv[seqs], kvp), f"sequences {seqs[:4]}...: final states"
    # in place (kv_final is kv_init): both parts read their initial states
    # before writing the final ones
    kv_ip = kv0d.clone()
    y_ip, _ = la.prefill_normed(qd, kd, vd, cu, decay, wd, 1e-5, gd, kv_init=kv_ip,
                                kv_final=kv_ip, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y_ip, y), "in place: rows"
    assert torch.equal(kv_ip, kv), "in place: final states"
    heads = [0, 1, H // 2, H - 1]
    o_ref, kv_ref = oracle.prefill_varlen(q[:, heads], k[:, heads], v[:, heads], cu,
                                          decay[heads], kv_init=kv0[:, heads])
    y_ref = oracle.norm_gate(o_ref, w[heads], 1e-5, to_np(gd)[:, heads])
    parity.check(to_np(y)[:, heads], y_ref, 1, 1e-2, what="normed split y")
    parity.check(to_np(kv)[:, heads], kv_ref, 1, 1e-2, what="normed split kv")
