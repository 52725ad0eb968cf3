"""The benchmark's algorithmic units and its one-GPU contract, on the CPU.

The roofline fraction the benchmark reports is its algorithmic bytes (or
flops) per launch over the measured launch time, so these units are pinned
here to the figures derived from the method's data flow: Q, K and V read and
O written once at 2 B per element plus the fp32 d x d final state per
(sequence, head); 4 d^2 + 2 d (beta + 1) flops per token and head; decode
reads and writes the fp32 state and moves q, k, v, o once.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_prefill_bytes_of_the_workloads():
    # B=1, H=64, N=8192, d=128: 8192 * 64 * 128 * 8 + 64 * 128^2 * 4
    assert bench.prefill_bytes(8192, 1) == 541_065_216
    # the 1M-token sequence
    assert bench.prefill_bytes(1 << 20, 1) == 68_723_671_040
    # per token at H=64, d=128: 65,536 B, so 8 TB/s is ~122 M tokens/s
    assert bench.prefill_bytes(1, 0) == 65_536
    assert 8.0e12 / bench.prefill_bytes(1, 0) == pytest.approx(1.2207e8, rel=1e-4)


def test_prefill_flops_at_beta_64():
    # 4 d^2 + 2 d (beta + 1) = 82,176 per token and head at d = 128, beta = 64
    assert bench.prefill_flops(1, heads=1) == 82_176
    assert bench.prefill_flops(8192) == 8192 * 64 * 82_176
    assert bench.prefill_flops(8192) == pytest.approx(4.31e10, rel=1e-3)
    # arithmetic intensity ~80 flop/B, below the ~312 flop/B ridge
    assert bench.prefill_flops(8192) / bench.prefill_bytes(8192, 1) == pytest.approx(79.6, abs=0.1)


def test_fp32_prefill_units():
    # fp32 in/out: 16 d B per token and head plus the state; beta = 32 flops
    assert bench.prefill_fp32_bytes(8192, 1) == 8192 * 64 * 128 * 16 + 64 * 128 * 128 * 4
    assert bench.prefill_fp32_bytes(8192, 1) == 2 * bench.prefill_bytes(8192, 1) - 64 * 128 * 128 * 4
    # 4 d^2 + 2 d (32 + 1) = 73,984 per token and head at d = 128
    assert bench.prefill_flops(1, heads=1, beta=32) == 73_984


def test_decode_bytes_of_the_serving_batch():
    # 256 sequences x 64 heads x (8 d^2 + 8 d) at d = 128
    assert bench.decode_bytes(256) == 2_164_260_864
    assert bench.decode_bytes(1, heads=1) == 132_096


def test_sweep_flatness():
    sweep = {"sweep1024": {"tokens_per_s": 40.0}, "sweep4096": {"tokens_per_s": 47.0},
             "n1m": {"tokens_per_s": 48.0}, "sweep65536": {"tokens_per_s": 50.0},
             "batch8_n8k": {"tokens_per_s": 99.0}}
    f = bench.sweep_flatness(sweep)
    assert f["max_over_min_1k_1m"] == 1.25 and f["max_over_min_4k_1m"] == round(50 / 47, 3)
    assert "batch8_n8k" not in f["workloads"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()
