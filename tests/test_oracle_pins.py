"""The fp64 oracle against facts fixed outside it (CPU only)."""

import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_three_way_tiny_workload():
    """The tiny workload itself (N=256, d=64, lam in {1.0, 0.9}, beta=32):
    quadratic, recurrent and blockwise agree to fp64 rounding."""
    from la_inputs import host_qkv, workload

    w = workload("tiny")
    q, k, v = host_qkv(256, w["H"], w["d"], w["seed"], dtype="fp32")
    cu = np.array([0, 256])
    o1, s1 = oracle.prefill_varlen(q, k, v, cu, w["decay"], form="quadratic")
    o2, s2 = oracle.prefill_varlen(q, k, v, cu, w["decay"], form="recurrent")
    o3, s3 = oracle.prefill_varlen(q, k, v, cu, w["decay"], form="blockwise", beta=32)
    for h in range(w["H"]):
        ref = np.linalg.norm(o1[:, h])
        assert np.linalg.norm(o2[:, h] - o1[:, h]) / ref < 1e-12
        assert np.linalg.norm(o3[:, h] - o1[:, h]) / ref < 1e-12
        assert np.linalg.norm(s3[0, h] - s1[0, h]) / np.linalg.norm(s1[0, h]) < 1e-12
        assert np.linalg.norm(s2[0, h] - s1[0, h]) / np.linalg.norm(s1[0, h]) < 1e-12


def test_bruteforce_loops_match_matrix_form():
    """The pure-Python double loop and the masked matrix form agree (N <= 64)."""
    rng = np.random.Generator(np.random.PCG64(3))
    for L, d, lam in ((1, 3, 0.5), (17, 5, 0.9), (64, 4, 1.0)):
        q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
        s0 = rng.standard_normal((d, d))
        o1, s1 = oracle.quadratic_loops(q, k, v, lam, s0)
        o2, s2 = oracle.quadratic(q, k, v, lam, s0)
        np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)


def test_blockwise_rejects_bad_beta():
    with pytest.raises(ValueError):
        oracle.blockwise(np.zeros((2, 2)), np.zeros((2, 2)), np.zeros((2, 2)), 1.0, 0)


def test_decay_mask_values():
    m = oracle.decay_mask(0.5, 3)
    assert m.tolist() == [[1.0, 0.0, 0.0], [0.5, 1.0, 0.0], [0.25, 0.5, 1.0]]
