"""GPU parity of the wide bf16 prefill kernel (one workgroup per chain, d = 128)
against the fp64 oracle (needs an MI355X).

The library takes the wide kernel when a call has more (sequence, head)
chains -- or (segment, head) chains in the segmented prefill -- than half the
GPU's compute units; every case here is sized past that point (64 heads and
enough sequences or segments), which the tests assert."""

import numpy as np
import pytest

import oracle
from la_inputs import cu_seqlens, host_int_qkv, host_qkv, random_states, rne_bf16, workload
from tests import parity
from tests.gpu_util import device, say, to_dev, to_np

pytestmark = pytest.mark.gpu

H = 64
D = 128


@pytest.fixture(scope="module")
def dev():
    return device()


def _assert_wide(chains):
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert 2 * chains > cus, f"{chains} chains <= {cus} / 2 compute units: the wide kernel is not used"


def _decay():
    d = np.asarray(workload("n8k")["decay"], np.float32).copy()
    d[0], d[1], d[2] = 1.0, 0.5, 0.9  # no decay, strong decay, medium
    return d


def _run(dev, lengths, seed, kv_init=False, out_f32=False, in_place=False, segment_len=None):
    import torch
    import linear_attention_la_amd as la

    say(f"case wide lengths={list(lengths)[:8]} kv_init={kv_init} out_f32={out_f32} "
        f"in_place={in_place} segment_len={segment_len}")
    T = int(sum(lengths))
    decay = _decay()
    q, k, v = host_qkv(T, H, D, seed, "bf16")
    cu = cu_seqlens(lengths)
    kv0 = random_states(len(lengths), H, D, seed + 7, scale=0.1) if kv_init else None
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    kv0d = to_dev(kv0, torch.float32, dev) if kv_init else None
    out_dtype = torch.float32 if out_f32 else None
    kv_final = kv0d if in_place else None
    if segment_len is None:
        _assert_wide(len(lengths) * H)
        o, kv = la.prefill(qd, kd, vd, cu, decay, kv_init=kv0d, out_dtype=out_dtype,
                           kv_final=kv_final)
    else:
        segs = sum(max(1, -(-n // segment_len)) for n in lengths)
        _assert_wide(segs * H)
        o, kv = la.prefill_segmented(qd, kd, vd, cu, decay, segment_len, kv_init=kv0d,
                                     out_dtype=out_dtype, kv_final=kv_final)
    torch.cuda.synchronize()
    if in_place:
        assert kv.data_ptr() == kv0d.data_ptr()
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, kv_init=kv0, beta=64)
    return to_np(o), to_np(kv), o_ref, kv_ref


@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("kv_init", [False, True])
def test_wide_ragged(dev, out_f32, kv_init):
    """Eight sequences x 64 heads: lengths 1, 63, 64, 65 (block edges), empty,
    several blocks with a tail; every head and sequence against the oracle."""
    lengths = [1, 63, 64, 65, 0, 300, 129, 17]
    o, kv, o_ref, kv_ref = _run(dev, lengths, 101 + 2 * out_f32 + kv_init, kv_init, out_f32)
    s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=not out_f32, what="wide o")
    s2 = parity.check(kv, kv_ref, 1, 1e-2, what="wide kv")
    say("wide ragged", s1, s2)


def test_wide_in_place_continuation(dev):
    """Final states written over kv_init (aliasing allowed)."""
    o, kv, o_ref, kv_ref = _run(dev, [200, 0, 513, 64], 111, kv_init=True, in_place=True)
    parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what="wide in-place o")
    parity.check(kv, kv_ref, 1, 1e-2, what="wide in-place kv")


@pytest.mark.parametrize("kv_init", [False, True])
def test_wide_segmented(dev, kv_init):
    """One 1000-token sequence cut into 4 segments of 256 (the last one
    ragged): both segmented passes run the wide kernel."""
    o, kv, o_ref, kv_ref = _run(dev, [1000], 121 + kv_init, kv_init=kv_init, segment_len=256)
    s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what="wide segmented o")
    s2 = parity.check(kv, kv_ref, 1, 1e-2, what="wide segmented kv")
    say("wide segmented", s1, s2)


def test_wide_exact_integer_inputs_bitwise(dev):
    """Entries in {-1, 0, 1} with decay 1 (sequences up to 256 tokens) or 0.5
    (up to 12 tokens): every intermediate is exact, so the wide kernel equals
    the exact result bit for bit (fp32 output, final state) and its
    round-to-nearest-even bf16 value (bf16 output)."""
    import torch
    import linear_attention_la_amd as la

    for lengths, lam in (([256, 100, 37, 1], 1.0), ([12, 5, 1, 9], 0.5)):
        say(f"exact wide case lengths={lengths} decay={lam}")
        _assert_wide(len(lengths) * H)
        decay = np.full(H, lam, np.float32)
        T = sum(lengths)
        q, k, v = host_int_qkv(T, H, D, 9)
        cu = cu_seqlens(lengths)
        qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
        o32, kv = la.prefill(qd, kd, vd, cu, decay, out_dtype=torch.float32)
        o16, _ = la.prefill(qd, kd, vd, cu, decay)
        torch.cuda.synchronize()
        o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, beta=64)
        assert np.array_equal(to_np(o32), o_ref)
        assert np.array_equal(to_np(kv), kv_ref)
        assert np.array_equal(to_np(o16), rne_bf16(o_ref.astype(np.float32)).astype(np.float64))


def test_wide_zero_length_sequences(dev):
    """Four empty sequences x 64 heads: no rows; final state = initial state."""
    import torch
    import linear_attention_la_amd as la

    _assert_wide(4 * H)
    kv0 = random_states(4, H, D, 13)
    kv0d = to_dev(kv0, torch.float32, dev)
    qd = torch.empty((0, H, D), dtype=torch.bfloat16, device=dev)
    o, kv = la.prefill(qd, qd.clone(), qd.clone(), [0, 0, 0, 0, 0], _decay(), kv_init=kv0d)
    torch.cuda.synchronize()
    assert o.shape == (0, H, D)
    assert np.array_equal(to_np(kv), kv0.astype(np.float64))


def test_wide_determinism_bitwise(dev):
    """Two runs of a wide launch agree bit for bit."""
    import torch
    import linear_attention_la_amd as la

    lengths = [700, 33, 64, 1500]
    _assert_wide(len(lengths) * H)
    q, k, v = host_qkv(sum(lengths), H, D, 17, "bf16")
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    cu = cu_seqlens(lengths)
    o1, kv1 = la.prefill(qd, kd, vd, cu, _decay())
    o2, kv2 = la.prefill(qd, kd, vd, cu, _decay())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(kv1, kv2)


@pytest.mark.parametrize("name", ["batch3_n8k", "batch5_n8k", "batch8_n8k"])
def test_wide_batch_n8k_benchmark_launch(dev, name):
    """Three, five or eight 8192-token sequences x 64 heads (the bench's
    launches; with five, the fifth sequence runs in 32-column slices after
    one wave of the wide kernel): three heads over all sequences against the
    oracle, and every output and final state against the 32-column kernel
    run one sequence at a time on the same inputs (64 chains per call)."""
    import torch
    import linear_attention_la_amd as la
    from la_inputs import device_qkv

    w = workload(name)
    cu = cu_seqlens(w["lengths"])
    T, S = int(cu[-1]), len(w["lengths"])
    _assert_wide(S * H)
    say(f"case wide {name} T={T}")
    qd, kd, vd = device_qkv(T, H, D, w["seed"], dev)
    o, kv = la.prefill(qd, kd, vd, cu, w["decay"])
    parts = [la.prefill(qd[cu[i]:cu[i + 1]].contiguous(), kd[cu[i]:cu[i + 1]].contiguous(),
                        vd[cu[i]:cu[i + 1]].contiguous(), [0, int(cu[i + 1] - cu[i])], w["decay"])
             for i in range(S)]
    o_slice = torch.cat([p_[0] for p_ in parts])
    kv_slice = torch.cat([p_[1] for p_ in parts])
    torch.cuda.synchronize()
    s1 = _compare_on_device(o, o_slice, bf16=True, what="wide vs 32-column o")
    s2 = _compare_on_device(kv, kv_slice, bf16=False, what="wide vs 32-column kv")
    say("wide vs 32-column", s1, s2)
    for h in (0, int(np.argmin(w["decay"])), int(np.argmax(w["decay"]))):
        q1, k1, v1 = (to_np(x[:, h, :])[:, None, :] for x in (qd, kd, vd))
        o_ref, kv_ref = oracle.prefill_varlen(q1, k1, v1, cu, np.array([w["decay"][h]]), beta=256)
        s3 = parity.check(to_np(o[:, h, :])[:, None, :], o_ref, 1, 1e-2, out_bf16=True,
                          what=f"o head {h}")
        s4 = parity.check(to_np(kv[:, h])[:, None], kv_ref, 1, 1e-2, what=f"kv head {h}")
        say(f"wide {name} head", h, s3, s4)


def _compare_on_device(a, b, bf16, what, rel_tol=1e-2, elem_tol=2e-2):
    """Per-head relative L2 <= rel_tol and elementwise |a - b| <= elem_tol *
    rms_h(b), on the GPU (head axis 1); for bf16 tensors an element past the
    elementwise bound passes only if a and b are at most one bf16 ulp apart
    (both are rounded results)."""
    import torch

    x = a.float().transpose(0, 1).reshape(a.shape[1], -1)
    y = b.float().transpose(0, 1).reshape(b.shape[1], -1)
    diff = x - y
    ny = torch.linalg.vector_norm(y, dim=1)
    rel = torch.linalg.vector_norm(diff, dim=1) / ny
    rms = ny / (y.shape[1] ** 0.5)
    assert bool(torch.all(rel <= rel_tol)), f"{what}: max relative L2 {rel.max().item():.3e}"
    over = diff.abs() > elem_tol * rms[:, None]
    n_over = int(over.sum().item())
    if n_over:
        assert bf16, f"{what}: {n_over} elements over {elem_tol} * rms"
        mag = torch.maximum(x.abs(), y.abs())
        ulp = torch.exp2(torch.floor(torch.log2(mag.clamp_min(1e-30))) - 7)
        bad = over & (diff.abs() > ulp)
        assert not bool(bad.any()), f"{what}: {int(bad.sum().item())} elements over the bound"
    return {"max_rel_l2": float(rel.max().item()), "format_explained": n_over}


def test_ndv_override_forces_either_kernel(dev, monkeypatch):
    """LA_NDV forces the kernel of la_prefill and la_prefill_pool.  A chain's
    result does not depend on the other chains of its call, so each kernel
    is recognised bit for bit: two sequences x 64 heads (128 chains, fewer
    than half the compute units: 32-column slices by default) run with
    LA_NDV=1 must equal those sequences inside a call padded to 384 chains
    (one workgroup per chain by default) and inside one of 192 chains (more
    than half the compute units: also one workgroup per chain by default),
    and the padded call with LA_NDV=4 must equal the unpadded default.  The
    two kernels differ in their last bits on these inputs (fp32 output), and
    both match the oracle."""
    import torch
    import linear_attention_la_amd as la

    lengths, pad = [300, 77], [64, 64, 64, 64]
    say(f"case LA_NDV override lengths={lengths} pad={pad}")
    _assert_wide(len(lengths + pad) * H)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert 2 * len(lengths) * H <= cus < 2 * (len(lengths) + 1) * H
    decay = _decay()
    T, Tp = sum(lengths), sum(lengths + pad)
    q, k, v = host_qkv(Tp, H, D, 131, "bf16")
    kv0 = random_states(len(lengths + pad), H, D, 132, scale=0.1)
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    kv0d = to_dev(kv0, torch.float32, dev)
    S = len(lengths)

    def run(n, ndv):
        if ndv is None:
            monkeypatch.delenv("LA_NDV", raising=False)
        else:
            monkeypatch.setenv("LA_NDV", ndv)
        cu = cu_seqlens((lengths + pad)[:n])
        tt = int(cu[-1])
        o, kv = la.prefill(qd[:tt], kd[:tt], vd[:tt], cu, decay, kv_init=kv0d[:n].contiguous(),
                           out_dtype=torch.float32)
        torch.cuda.synchronize()
        return o[:T], kv[:S]

    o_slices, kv_slices = run(S, None)
    o_wide, kv_wide = run(S, "1")
    o_pad_wide, kv_pad_wide = run(S + len(pad), None)
    o_pad_slices, kv_pad_slices = run(S + len(pad), "4")
    o_mid, kv_mid = run(S + 1, None)
    assert torch.equal(o_wide, o_pad_wide) and torch.equal(kv_wide, kv_pad_wide), \
        "LA_NDV=1 did not run the one-workgroup-per-chain kernel"
    assert torch.equal(o_mid, o_wide) and torch.equal(kv_mid, kv_wide), \
        "192 chains did not take the one-workgroup-per-chain kernel"
    assert torch.equal(o_pad_slices, o_slices) and torch.equal(kv_pad_slices, kv_slices), \
        "LA_NDV=4 did not run the 32-column kernel"
    assert not torch.equal(o_wide, o_slices), "the two kernels gave identical results"
    o_ref, kv_ref = oracle.prefill_varlen(q[:T], k[:T], v[:T], cu_seqlens(lengths), decay,
                                          kv_init=kv0[:S], beta=64)
    for name, o, kv in (("slices", o_slices, kv_slices), ("wide", o_wide, kv_wide)):
        parity.check(to_np(o), o_ref, 1, 1e-2, what=f"LA_NDV {name} o")
        parity.check(to_np(kv), kv_ref, 1, 1e-2, what=f"LA_NDV {name} kv")

    # la_prefill_pool takes the same override: its states sit in pool slots
    monkeypatch.setenv("LA_NDV", "1")
    pool = torch.zeros((5, H, D, D), dtype=torch.float32, device=dev)
    slots = [3, 1]
    pool[slots] = kv0d[:S]
    o_pool = la.prefill_pool(qd[:T], kd[:T], vd[:T], cu_seqlens(lengths), decay, pool, slots,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    monkeypatch.delenv("LA_NDV")
    assert torch.equal(o_pool, o_wide) and torch.equal(pool[slots], kv_wide), \
        "la_prefill_pool with LA_NDV=1 differs from la_prefill with LA_NDV=1"


@pytest.mark.parametrize("lengths,wide_seqs", [([640] * 5, [0, 1, 2, 3]),
                                               ([576, 640, 640, 640, 640], [1, 2, 3, 4]),
                                               ([640, 640, 640, 640, 320, 0], [0, 1, 2, 3])])
def test_split_launch(dev, monkeypatch, lengths, wide_seqs):
    """Five sequences x 64 heads (320 chains on 256 compute units): the four
    longest sequences fill one wave of the one-workgroup-per-chain kernel and
    the last one runs in 32-column slices in a second launch, rather than as
    an extra wave of the wide kernel.  Each sequence's rows and final state
    equal, bit for bit, those of the kernel it was given (forced for the
    whole call with LA_NDV), also on a state pool; the call matches the
    oracle.  The second case dispatches the sequences out of index order; the
    third (384 chains) sends a shorter and a zero-length sequence to the
    slices."""
    import torch
    import linear_attention_la_amd as la

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"the split planned here assumes 256 compute units, not {cus}")
    say(f"case split launch lengths={lengths}")
    decay = _decay()
    cu = cu_seqlens(lengths)
    T, S = int(cu[-1]), len(lengths)
    q, k, v = host_qkv(T, H, D, 141, "bf16")
    kv0 = random_states(S, H, D, 142, scale=0.1)
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    kv0d = to_dev(kv0, torch.float32, dev)

    def run(ndv):
        if ndv is None:
            monkeypatch.delenv("LA_NDV", raising=False)
        else:
            monkeypatch.setenv("LA_NDV", ndv)
        o, kv = la.prefill(qd, kd, vd, cu, decay, kv_init=kv0d, out_dtype=torch.float32)
        torch.cuda.synchronize()
        return o, kv

    o, kv = run(None)
    o_wide, kv_wide = run("1")
    o_slices, kv_slices = run("4")
    monkeypatch.delenv("LA_NDV")
    n_wide, order = la.kernel_plan(cu, H, D)
    assert n_wide == len(wide_seqs) and sorted(order[:n_wide].tolist()) == wide_seqs
    for s in range(S):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        ref_o, ref_kv = (o_wide, kv_wide) if s in wide_seqs else (o_slices, kv_slices)
        assert torch.equal(o[rows], ref_o[rows]), f"sequence {s}: rows"
        assert torch.equal(kv[s], ref_kv[s]), f"sequence {s}: final state"
    assert not torch.equal(o, o_wide) and not torch.equal(o, o_slices)
    o_ref, kv_ref = oracle.prefill_varlen(q, k, v, cu, decay, kv_init=kv0, beta=64)
    parity.check(to_np(o), o_ref, 1, 1e-2, what="split o")
    parity.check(to_np(kv), kv_ref, 1, 1e-2, what="split kv")

    pool = torch.zeros((7, H, D, D), dtype=torch.float32, device=dev)
    slots = [6, 0, 3, 5, 1, 2][:S]
    pool[slots] = kv0d
    o_pool = la.prefill_pool(qd, kd, vd, cu, decay, pool, slots, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_pool, o) and torch.equal(pool[slots], kv), "pool prefill differs"
