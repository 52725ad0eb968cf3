"""GPU parity of la_prefill_pool (prefill whose states live at slots of a
state pool) against the fp64 oracle (needs an MI355X)."""

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


def _chunk(dev, pool_dev, pool_ref, slots, lengths, H, d, decay, seed):
    """One pool prefill on the GPU and in the oracle; returns the outputs and
    advances the oracle's pool."""
    import torch
    import linear_attention_la_amd as la

    T = sum(lengths)
    q, k, v = host_qkv(T, H, d, seed, "bf16")
    cu = cu_seqlens(lengths)
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    o = la.prefill_pool(qd, kd, vd, cu, decay, pool_dev, slots)
    torch.cuda.synchronize()
    o_ref, pool_new = oracle.prefill_pool(q, k, v, cu, decay, pool_ref, slots)
    return to_np(o), o_ref, pool_new


@pytest.mark.parametrize("d", [64, 128])
def test_chunked_prefill_on_random_slots(dev, d):
    """Two chunks of the same sequences continue from their pooled states
    (ragged lengths, an empty chunk included); slots no sequence names stay
    bit-identical."""
    import torch

    H, P = 4, 20
    decay = np.array([1.0, 0.99, 0.9, 0.5], np.float32)
    pool0 = random_states(P, H, d, 61 + d, scale=0.1)
    pool_dev = to_dev(pool0, torch.float32, dev)
    slots = np.array([13, 2, 19, 7, 0], np.int32)
    say(f"case pool prefill d={d} slots={slots.tolist()}")
    ref = pool0.astype(np.float64)
    for step, lengths in enumerate(([65, 1, 200, 0, 64], [3, 130, 63, 17, 0])):
        o, o_ref, ref = _chunk(dev, pool_dev, ref, slots, lengths, H, d, decay, 70 + 10 * step + d)
        s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what=f"chunk {step} o")
        s2 = parity.check(to_np(pool_dev)[slots], ref[slots], 1, 1e-2, what=f"chunk {step} states")
        say("  chunk", step, s1, s2)
    untouched = np.setdiff1d(np.arange(P), slots)
    assert np.array_equal(to_np(pool_dev)[untouched], pool0.astype(np.float64)[untouched])


def test_identity_slots_match_in_place_prefill(dev):
    """Slots 0..S-1 of a pool of S states give exactly la_prefill with
    kv_init = kv_final = the pool (bit for bit)."""
    import torch
    import linear_attention_la_amd as la

    H, d = 3, 128
    lengths = [100, 0, 257, 64]
    S, T = len(lengths), sum(lengths)
    decay = np.array([0.999, 0.9, 0.6], np.float32)
    q, k, v = host_qkv(T, H, d, 91, "bf16")
    cu = cu_seqlens(lengths)
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    st0 = to_dev(random_states(S, H, d, 93, scale=0.1), torch.float32, dev)
    pool = st0.clone()
    kv = st0.clone()
    o1 = la.prefill_pool(qd, kd, vd, cu, decay, pool, np.arange(S, dtype=np.int32))
    o2, _ = la.prefill(qd, kd, vd, cu, decay, kv_init=kv, kv_final=kv)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(pool, kv)


def test_wide_path_on_random_slots(dev):
    """Eight sequences x 40 heads (320 chains: the one-workgroup-per-chain
    kernel) on random slots of a 12-state pool."""
    import torch

    H, d, P = 40, 128, 12
    rng = np.random.default_rng(5)
    decay = np.clip(rng.uniform(0.8, 1.0, H), 0.8, 1.0).astype(np.float32)
    decay[0] = 1.0
    pool0 = random_states(P, H, d, 95, scale=0.1)
    pool_dev = to_dev(pool0, torch.float32, dev)
    slots = rng.permutation(P)[:8].astype(np.int32)
    lengths = [130, 1, 64, 0, 77, 200, 63, 5]
    say(f"case pool prefill wide slots={slots.tolist()}")
    o, o_ref, ref = _chunk(dev, pool_dev, pool0.astype(np.float64), slots, lengths, H, d, decay, 97)
    s1 = parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what="wide pool o")
    s2 = parity.check(to_np(pool_dev)[slots], ref[slots], 1, 1e-2, what="wide pool states")
    say("  wide", s1, s2)


def test_prefill_then_decode_on_the_pool(dev):
    """The serving flow: a pool prefill writes the states that a pool decode
    then advances by one token, against the oracle's two steps."""
    import torch
    import linear_attention_la_amd as la

    H, d, P = 4, 128, 10
    decay = np.array([1.0, 0.97, 0.9, 0.7], np.float32)
    pool0 = np.zeros((P, H, d, d), np.float32)  # fresh sequences start from zeroed slots
    pool_dev = to_dev(pool0, torch.float32, dev)
    slots = np.array([4, 9, 1], np.int32)
    o, o_ref, ref = _chunk(dev, pool_dev, pool0.astype(np.float64), slots, [150, 64, 33], H, d,
                           decay, 99)
    parity.check(o, o_ref, 1, 1e-2, out_bf16=True, what="serving prefill o")
    q1, k1, v1 = host_qkv(3, H, d, 101, "bf16")  # one token for each of the 3 sequences
    qd, kd, vd = (to_dev(x, torch.bfloat16, dev) for x in (q1, k1, v1))
    od = la.decode_pool(qd, kd, vd, pool_dev, slots, decay)
    torch.cuda.synchronize()
    od_ref, ref = oracle.decode_pool(q1, k1, v1, ref, slots, decay)
    parity.check(to_np(od), od_ref, 1, 1e-2, out_bf16=True, what="serving decode o")
    parity.check(to_np(pool_dev)[slots], ref[slots], 1, 1e-2, what="serving states")
