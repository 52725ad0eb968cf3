"""GPU parity of la_prefill against the fp64 oracle (needs an MI355X)."""

import numpy as np
import pytest

import oracle
from la_inputs import (cu_seqlens, decay_from_seed, device_qkv, host_int_qkv, host_qkv,
                       random_states, rne_bf16, workload)
from tests import parity
from tests.gpu_util import device, say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _run(dev, lengths, H, d, dtype, decay, seed, kv_init=False, out_f32=False, beta=64,
         heads=None):
    import torch
    import linear_attention_la_amd as la

    say(f"case lengths={list(lengths)[:8]}{'...' if len(lengths) > 8 else ''} H={H} d={d} "
        f"dtype={dtype} kv_init={kv_init} out_f32={out_f32}")
    T = int(sum(lengths))
    q, k, v = host_qkv(T, H, d, seed, dtype)
    cu = cu_seqlens(lengths)
    kv0 = random_states(len(lengths), H, d, seed + 7, scale=0.1) if kv_init else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd, kd, vd = (to_dev(x, tdt, dev) for x in (q, k, v))
    kv0d = to_dev(kv0, torch.float32, dev) if kv_init else None
    o, kv = la.prefill(qd, kd, vd, cu, decay, kv_init=kv0d,
                       out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, kv_init=kv0, beta=beta,
                                          heads=heads)
    return to_np(o), to_np(kv), o_ref, kv_ref


def test_tiny_workload_fp32(dev):
    """N=256, H=2, d=64, fp32, decay {1.0, 0.9}: relative L2 <= 1e-5."""
    w = workload("tiny")
    o, kv, o_ref, kv_ref = _run(dev, w["lengths"], w["H"], w["d"], "fp32", w["decay"], w["seed"],
                                out_f32=True, beta=32)
    s1 = parity.check(o, o_ref, 1, 1e-5, what="tiny o")
    s2 = parity.check(kv, kv_ref, 1, 1e-5, what="tiny kv")
    say("tiny", s1, s2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kv_init", [False, True])
def test_fp32_ragged(dev, d, kv_init):
    lengths = [1, 31, 32, 33, 100, 0, 7]
    decay = np.array([1.0, 0.95, 0.5], np.float32)
    o, kv, o_ref, kv_ref = _run(dev, lengths, 3, d, "fp32", decay, 11 + d, kv_init=kv_init,
                                out_f32=True)
    parity.check(o, o_ref, 1, 1e-5, what="fp32 ragged o")
    parity.check(kv, kv_ref, 1, 1e-5, what="fp32 ragged kv")


def test_fp32_n8k_sampled_heads(dev):
    """fp32 inputs at the 8K shape (B=1, H=64, N=8192, d=128, seeded decays,
    initial state): 256 blocks of 32 tokens per chain on the fp32 kernel;
    head 0 and the weakest and strongest decays against the oracle at 1e-5."""
    w = workload("n8k")
    heads = [0, int(np.argmin(w["decay"])), int(np.argmax(w["decay"]))]
    o, kv, o_ref, kv_ref = _run(dev, w["lengths"], w["H"], w["d"], "fp32", w["decay"],
                                w["seed"] + 100, kv_init=True, out_f32=True, beta=32,
                                heads=heads)
    s1 = parity.check(o[:, heads], o_ref[:, heads], 1, 1e-5, what="fp32 n8k o")
    s2 = parity.check(kv[:, heads], kv_ref[:, heads], 1, 1e-5, what="fp32 n8k kv")
    say("fp32 n8k", s1, s2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("kv_init", [False, True])
def test_bf16_ragged(dev, d, out_f32, kv_init):
    """Ragged lengths around the 64-token block (empty, 1, 63..65, several
    blocks plus a tail), decays from none to strong."""
    lengths = [1, 63, 64, 65, 129, 0, 300, 17]
    decay = np.array([1.0, 0.99, 0.9, 0.5], np.float32)
    o, kv, o_ref, kv_ref = _run(dev, lengths, 4, d, "bf16", decay, 21 + d, kv_init=kv_init,
                                out_f32=out_f32)
    s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=not out_f32, what="bf16 ragged o")
    s2 = parity.check(kv, kv_ref, 1, 1e-2, what="bf16 ragged kv")
    say("bf16 ragged", s1, s2)


@pytest.mark.parametrize("nseq", [511, 512, 513, 700])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_many_sequences_dispatch_order(dev, nseq, dtype):
    """Batches at and past the largest one dispatched longest-first (512
    sequences; larger batches keep the index order): lengths 0..130 in a
    shuffled order, so the longest-first order differs from the index
    order, and every sequence and head against the oracle."""
    rng = np.random.default_rng(600 + nseq)
    lengths = rng.integers(0, 131, size=nseq)
    lengths[:3] = (0, 1, 130)
    rng.shuffle(lengths)
    decay = np.array([1.0, 0.8], np.float32)
    tol = 1e-2 if dtype == "bf16" else 1e-5
    o, kv, o_ref, kv_ref = _run(dev, lengths.tolist(), 2, 64, dtype, decay, 31 + nseq,
                                kv_init=True, out_f32=dtype == "fp32",
                                beta=64 if dtype == "bf16" else 32)
    s1 = parity.check(o, o_ref, 1, tol, out_bf16=dtype == "bf16", what=f"{nseq} seqs o")
    s2 = parity.check(kv, kv_ref, 1, tol, what=f"{nseq} seqs kv")
    say("many sequences", nseq, dtype, s1, s2)


def test_bf16_n8k_all_heads(dev):
    """B=1, H=64, N=8192, d=128, bf16, seeded decay: every head checked."""
    w = workload("n8k")
    o, kv, o_ref, kv_ref = _run(dev, w["lengths"], w["H"], w["d"], "bf16", w["decay"], w["seed"])
    s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what="n8k o")
    s2 = parity.check(kv, kv_ref, 1, 1e-2, what="n8k kv")
    say("n8k", s1, s2)


def test_exact_integer_inputs_bitwise(dev):
    """Entries in {-1, 0, 1} with decay 1 (sequences up to 256 tokens) or 0.5
    (up to 12 tokens) keep every intermediate exactly representable, so the
    GPU must equal the exact result bit for bit (fp32 output) and its
    round-to-nearest-even bf16 value (bf16 output)."""
    import torch
    import linear_attention_la_amd as la

    for lengths, decay in (([256, 100, 37, 0, 1, 64], np.array([1.0, 1.0], np.float32)),
                           ([12, 5, 1, 9], np.array([0.5, 0.5], np.float32))):
        say(f"exact case lengths={lengths} decay={decay.tolist()}")
        T = sum(lengths)
        q, k, v = host_int_qkv(T, 2, 128, 5)
        cu = cu_seqlens(lengths)
        qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
        o32, kv = la.prefill(qd, kd, vd, cu, decay, out_dtype=torch.float32)
        o16, _ = la.prefill(qd, kd, vd, cu, decay)
        torch.cuda.synchronize()
        o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, beta=64)
        assert np.array_equal(to_np(o32), o_ref)
        assert np.array_equal(to_np(kv), kv_ref)
        assert np.array_equal(to_np(o16), rne_bf16(o_ref.astype(np.float32)).astype(np.float64))


@pytest.mark.parametrize("d", [64, 128])
def test_max_heads_extreme_decays(dev, d):
    """LA_MAX_HEADS = 256 heads over three sequences (at d = 128 the 768
    chains take the one-workgroup-per-chain kernel, at d = 64 the 32-column
    kernel), with decays from 1 down to 1e-30, where lambda^2 already
    underflows in fp32 and each row keeps only its diagonal term
    (q_t . k_t) v_t."""
    H = 256
    decay = np.geomspace(1e-30, 1.0, H).astype(np.float32)
    decay[:4] = (1.0, 1e-30, 0.5, 0.999999)
    o, kv, o_ref, kv_ref = _run(dev, [130, 1, 64], H, d, "bf16", decay, 41 + d, kv_init=True)
    s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what="max heads o")
    s2 = parity.check(kv, kv_ref, 1, 1e-2, what="max heads kv")
    say("max heads", d, s1, s2)


def test_zero_length_sequences(dev):
    """All sequences empty: no rows, final state = initial state (or zero)."""
    import torch
    import linear_attention_la_amd as la

    H, d = 2, 128
    kv0 = random_states(3, H, d, 3)
    kv0d = to_dev(kv0, torch.float32, dev)
    qd = torch.empty((0, H, d), dtype=torch.bfloat16, device=dev)
    o, kv = la.prefill(qd, qd.clone(), qd.clone(), [0, 0, 0, 0], [0.9, 1.0], kv_init=kv0d)
    o2, kv2 = la.prefill(qd, qd.clone(), qd.clone(), [0, 0, 0, 0], [0.9, 1.0])
    torch.cuda.synchronize()
    assert o.shape == (0, H, d)
    assert np.array_equal(to_np(kv), kv0.astype(np.float64))
    assert np.all(to_np(kv2) == 0.0)


def test_continuation_in_place(dev):
    """Prefill A, then B from A's state (kv_final aliasing kv_init), equals
    one prefill of A||B within tolerance; both match the oracle."""
    import torch
    import linear_attention_la_amd as la

    H, d, L, cut = 4, 128, 1000, 321
    decay = np.array([1.0, 0.99, 0.9, 0.7], np.float32)
    q, k, v = host_qkv(L, H, d, 31)
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    o_full, kv_full = la.prefill(qd, kd, vd, [0, L], decay)
    o_a, kv = la.prefill(qd[:cut].contiguous(), kd[:cut].contiguous(), vd[:cut].contiguous(),
                         [0, cut], decay)
    o_b, kv_b = la.prefill(qd[cut:].contiguous(), kd[cut:].contiguous(), vd[cut:].contiguous(),
                           [0, L - cut], decay, kv_init=kv, kv_final=kv)
    torch.cuda.synchronize()
    assert kv_b.data_ptr() == kv.data_ptr()
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, np.array([0, L]), decay, beta=64)
    o_split = np.concatenate([to_np(o_a), to_np(o_b)])
    parity.check(o_split, o_ref, 1, 1e-2, out_bf16=True, what="continuation o")
    parity.check(to_np(kv), kv_ref, 1, 1e-2, what="continuation kv")
    parity.check(o_split, to_np(o_full), 1, 1e-2, out_bf16=True, what="split vs full")


def test_determinism_bitwise(dev):
    """Two runs of the same launch agree bit for bit (no atomics)."""
    import torch
    import linear_attention_la_amd as la

    w = workload("n8k")
    qd, kd, vd = device_qkv(8192, 64, 128, w["seed"], dev)
    o1, kv1 = la.prefill(qd, kd, vd, [0, 8192], w["decay"])
    o2, kv2 = la.prefill(qd, kd, vd, [0, 8192], w["decay"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(kv1, kv2)


def _check_heads(dev, qd, kd, vd, cu, decay, o, kv, heads, beta=256, what=""):
    """Full oracle check of the listed heads of a large device-resident run."""
    for h in heads:
        q = to_np(qd[:, h, :])[:, None, :]
        k = to_np(kd[:, h, :])[:, None, :]
        v = to_np(vd[:, h, :])[:, None, :]
        o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, np.array([decay[h]]), beta=beta)
        s1 = parity.check(to_np(o[:, h, :])[:, None, :], o_ref, 1, 1e-2, out_bf16=True,
                          what=f"{what} o head {h}")
        s2 = parity.check(to_np(kv[:, h])[:, None], kv_ref, 1, 1e-2, what=f"{what} kv head {h}")
        say(what, "head", h, s1, s2)


@pytest.mark.parametrize("name", ["sweep1024", "sweep4096", "sweep16384", "sweep65536",
                                  "sweep65536_nodecay"])
def test_length_sweep(dev, name):
    """B=1, H=64, d=128, N in {1K, 4K, 16K, 64K} (+ no decay at 64K): a spread
    of heads checked against the oracle over the whole sequence."""
    import torch
    import linear_attention_la_amd as la

    w = workload(name)
    N = w["lengths"][0]
    say(f"sweep {name} N={N}")
    qd, kd, vd = device_qkv(N, 64, 128, w["seed"], dev)
    o, kv = la.prefill(qd, kd, vd, [0, N], w["decay"])
    torch.cuda.synchronize()
    _check_heads(dev, qd, kd, vd, np.array([0, N]), w["decay"], o, kv, [0, 21, 42, 63],
                 what=name)


def test_one_million_tokens(dev):
    """B=1, H=64, N=1,048,576, d=128 in the benchmark's launch configuration;
    two heads (strongest and weakest decay) checked over all 1M tokens."""
    import torch
    import linear_attention_la_amd as la

    w = workload("n1m")
    N = w["lengths"][0]
    say("n1m: generating inputs")
    qd, kd, vd = device_qkv(N, 64, 128, w["seed"], dev)
    o, kv = la.prefill(qd, kd, vd, [0, N], w["decay"])
    torch.cuda.synchronize()
    say("n1m: kernel done, checking")
    assert torch.isfinite(o).all()
    heads = [int(np.argmin(w["decay"])), int(np.argmax(w["decay"]))]
    _check_heads(dev, qd, kd, vd, np.array([0, N]), w["decay"], o, kv, heads, beta=256,
                 what="n1m")
    del qd, kd, vd, o, kv
    torch.cuda.empty_cache()


def test_varlen_64_sequences(dev):
    """64 sequences, lengths log-uniform in [512, 131072], packed: every
    sequence of two heads checked."""
    import torch
    import linear_attention_la_amd as la

    w = workload("varlen64")
    cu = cu_seqlens(w["lengths"])
    T = int(cu[-1])
    say(f"varlen64 T={T}")
    qd, kd, vd = device_qkv(T, 64, 128, w["seed"] + 1, dev)
    o, kv = la.prefill(qd, kd, vd, cu, w["decay"])
    torch.cuda.synchronize()
    _check_heads(dev, qd, kd, vd, cu, w["decay"], o, kv, [5, 50], beta=256, what="varlen64")
    del qd, kd, vd, o, kv
    torch.cuda.empty_cache()


def test_binding_rejects_mismatched_outputs(dev):
    """The torch wrappers reject caller-supplied outputs and buffers that do
    not match what the library will write (shape, dtype, device, layout) and
    output dtypes it does not produce, before any call into the library: it
    writes through bare pointers and cannot see a tensor's size."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import cu_seqlens

    say("case binding rejects mismatched outputs")
    T, H, d = 130, 2, 64
    q, k, v = (to_dev(x, torch.bfloat16, dev) for x in host_qkv(T, H, d, 5, "bf16"))
    cu = cu_seqlens([100, 30])
    decay = np.array([0.9, 0.8], np.float32)
    bad_out = [torch.empty((T - 1, H, d), dtype=torch.bfloat16, device=dev),
               torch.empty((T, H, d), dtype=torch.float32, device=dev),
               torch.empty((T, H, 2 * d), dtype=torch.bfloat16, device=dev)[:, :, :d],
               torch.empty((T, H, d), dtype=torch.bfloat16)]
    for o in bad_out:
        with pytest.raises(ValueError):
            la.prefill(q, k, v, cu, decay, out=o)
    with pytest.raises(ValueError):  # fp32 output into a bf16 buffer
        la.prefill(q, k, v, cu, decay, out_dtype=torch.float32,
                   out=torch.empty((T, H, d), dtype=torch.bfloat16, device=dev))
    with pytest.raises(TypeError):
        la.prefill(q, k, v, cu, decay, out_dtype=torch.float16)
    with pytest.raises(ValueError):
        la.prefill(q, k, v, cu, decay, kv_final=torch.empty((1, H, d, d), device=dev))
    with pytest.raises(ValueError):
        la.prefill(q, k, v, cu, decay, kv_init=torch.zeros((2, H, d, d), device=dev).double())
    with pytest.raises(ValueError):  # host copy longer than the device cu_seqlens
        la.prefill(q, k, v, torch.from_numpy(cu[:2].copy()).to(dev), decay,
                   cu_seqlens_host=cu)
    with pytest.raises(ValueError):
        la.prefill_segmented(q, k, v, cu, decay, 64, workspace=torch.empty(1 << 20,
                                                                            dtype=torch.uint8))
    do = torch.empty_like(q)
    with pytest.raises(ValueError):
        la.prefill_backward(q, k, v, do, cu, decay,
                            dk=torch.empty((T, H, d), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        la.prefill_backward(q, k, v, do, cu, decay,
                            dkv_init=torch.empty((2, H, d, d), dtype=torch.bfloat16, device=dev))
    q1, k1, v1 = q[:4].contiguous(), k[:4].contiguous(), v[:4].contiguous()
    kv = torch.zeros((4, H, d, d), device=dev)
    with pytest.raises(ValueError):
        la.decode(q1, k1, v1, kv, decay, out=torch.empty((4, H, d), dtype=torch.float32,
                                                          device=dev))
    with pytest.raises(ValueError):
        la.decode(q1, k1, v1, kv[:3].contiguous(), decay)
    pool = torch.zeros((6, H, d, d), device=dev)
    with pytest.raises(ValueError):
        la.decode_pool(q1, k1, v1, pool, torch.tensor([0, 1, 2], dtype=torch.int32,
                                                      device=dev), decay)
    with pytest.raises(ValueError):
        la.prefill_pool(q, k, v, cu, decay, pool, [0, 1],
                        out=torch.empty((H, T, d), dtype=torch.bfloat16,
                                        device=dev).transpose(0, 1))
    # nothing was launched; a correct call still works
    o, kv_f = la.prefill(q, k, v, cu, decay)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(kv_f).all()


@pytest.mark.parametrize("d", [64, 128])
def test_block_size_variants_agree(dev, d, monkeypatch):
    """The compiled block sizes agree with one another, not only each with the
    oracle: the fp32 kernel (beta = 32), the 32-column bf16 kernel and, for
    d = 128, the one-workgroup-per-chain kernel (beta = 64 both, forced by
    LA_NDV) on the same bf16-valued inputs, fp32 outputs, ragged lengths
    across block edges, with initial states.  Each pair within 1e-4 relative
    L2 per head (both sit within ~3e-5 of the exact result), and each
    against the oracle at a block size none of them uses (beta = 100)."""
    import torch
    import linear_attention_la_amd as la

    lengths = [1, 63, 64, 65, 200, 0, 333]
    H = 3
    decay = np.array([1.0, 0.97, 0.6], np.float32)
    say(f"case block-size variants lengths={lengths} H={H} d={d}")
    T = int(sum(lengths))
    q, k, v = host_qkv(T, H, d, 51 + d, "bf16")  # bf16-representable fp32 arrays
    cu = cu_seqlens(lengths)
    kv0 = random_states(len(lengths), H, d, 58 + d, scale=0.1)
    kv0d = to_dev(kv0, torch.float32, dev)
    runs = {}
    for name, dt, ndv in (("fp32 beta=32", torch.float32, None),
                          ("32-column beta=64", torch.bfloat16, str(d // 32)),
                          ("one workgroup per chain beta=64", torch.bfloat16, "1")):
        if ndv == "1" and d != 128:
            continue
        if ndv is None:
            monkeypatch.delenv("LA_NDV", raising=False)
        else:
            monkeypatch.setenv("LA_NDV", ndv)
        qd, kd, vd = (to_dev(x, dt, dev) for x in (q, k, v))
        o, kv = la.prefill(qd, kd, vd, cu, decay, kv_init=kv0d, out_dtype=torch.float32)
        torch.cuda.synchronize()
        runs[name] = (to_np(o), to_np(kv))
    monkeypatch.delenv("LA_NDV", raising=False)
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, kv_init=kv0, beta=100)
    names = list(runs)
    for name in names:
        parity.check(runs[name][0], o_ref, 1, 1e-2, what=f"{name} o vs oracle")
        parity.check(runs[name][1], kv_ref, 1, 1e-2, what=f"{name} kv vs oracle")
    for i in range(len(names)):
        for j in range(i + 1, len(names)):
            a, b = runs[names[i]], runs[names[j]]
            s1 = parity.check(a[0], b[0], 1, 1e-4, what=f"{names[i]} vs {names[j]} o")
            s2 = parity.check(a[1], b[1], 1, 1e-4, what=f"{names[i]} vs {names[j]} kv")
            say(f"{names[i]} vs {names[j]}", s1, s2)
