"""GPU parity of la_decode_pool (decode on a state pool through a slot map)
against the fp64 oracle (needs an MI355X)."""

import numpy as np
import pytest

import oracle
from la_inputs import host_qkv, random_states
from tests import parity
from tests.gpu_util import device, say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_pool_random_slots(dev, d, dtype):
    """20 sequences on a pool of 37 states at random distinct slots, two
    successive steps with different slot sets: outputs and touched states
    against the oracle, untouched states bit for bit unchanged."""
    import torch
    import linear_attention_la_amd as la

    P, B, H = 37, 20, 3
    decay = np.array([1.0, 0.97, 0.5], np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pool = random_states(P, H, d, 61 + d)
    pool_d = to_dev(pool, torch.float32, dev)
    pool_ref = pool.astype(np.float64)
    rng = np.random.default_rng(5 + d)
    for step in range(2):
        slots = rng.choice(P, size=B, replace=False).astype(np.int32)
        say(f"decode_pool d={d} dtype={dtype} step={step} slots={slots[:6].tolist()}...")
        q, k, v = (x[:B * H].reshape(B, H, d)
                   for x in host_qkv(B * H, 1, d, 300 * step + d, dtype))
        before = pool_d.clone()
        o = la.decode_pool(to_dev(q, tdt, dev), to_dev(k, tdt, dev), to_dev(v, tdt, dev), pool_d,
                           slots, decay)
        torch.cuda.synchronize()
        o_ref, pool_ref = oracle.decode_pool(q, k, v, pool_ref, slots, decay)
        tol = 1e-5 if dtype == "fp32" else 1e-2
        parity.check(to_np(o), o_ref, 1, tol, out_bf16=(dtype == "bf16"), what="pool o")
        parity.check(to_np(pool_d[slots]), pool_ref[slots], 1, 1e-5, what="pool touched states")
        untouched = np.setdiff1d(np.arange(P), slots)
        assert torch.equal(pool_d[untouched], before[untouched]), "an untouched state changed"


def test_identity_slots_match_decode(dev):
    """Slots 0..B-1 on a pool of B states give la_decode's results bit for bit."""
    import torch
    import linear_attention_la_amd as la

    B, H, d = 16, 4, 128
    decay = np.array([0.999, 0.9, 0.7, 1.0], np.float32)
    say("decode_pool identity slots")
    kv = to_dev(random_states(B, H, d, 9), torch.float32, dev)
    kv2 = kv.clone()
    q, k, v = (to_dev(x[:B * H].reshape(B, H, d), torch.bfloat16, dev)
               for x in host_qkv(B * H, 1, d, 19))
    o1 = la.decode(q, k, v, kv, decay)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    o2 = la.decode_pool(q, k, v, kv2, slots, decay, slots_host=np.arange(B, dtype=np.int32))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(kv, kv2)
