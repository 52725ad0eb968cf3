"""Benchmark of the Lightning Attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

A timed step is one la_prefill over the workload B=1, H=64, N=8192, d=128,
bf16 Q/K/V ~ N(0,1)/sqrt(d), per-head decay exp(-U[0.001, 0.1]) (the
MiniMax-Text-01 lightning-layer shape at its 8192-token pretraining length).
Inputs are resident in HBM before timing starts; two input sets alternate
(1.08 GB together, four times the 256 MB Infinity Cache) so no step reads
inputs left in cache by the step before.  W untimed warmup steps, then K
timed steps bracketed by torch.cuda.synchronize().

One JSON line is printed with the contract fields plus:
  roofline      the prefill kernel's algorithmic HBM bytes per launch over
                its average launch time (HIP events on its stream), against
                8 TB/s; `traffic` is the counter-measured bytes per launch
                from profiles/ if it was taken on the current kernel source.
  cpu_baseline  the fp64 oracle (blockwise, beta=64) timed on the host cores
                over heads of the same workload.
  mfma          algorithmic TFLOP/s at beta=64 against 2.5 PFLOP/s bf16.
  decode        la_decode alone on 256 sequences x 64 heads: GB/s vs 8 TB/s.
  mixed         decode on one stream concurrent with a packed prefill of 8
                sequences (lengths U[1K, 32K]) on another.
  peaks         measured on the GPU: a 1 GiB read+write stream (HBM) and an 8192^3
                bf16 matmul; roofline.frac_of_measured_stream relates the
                prefill kernel to that stream.
  sweep         cold tokens/s (median, min) at N = 1K ... 1M, for eight 8K sequences in one
                call and for a packed varlen batch (the last two have enough
                (sequence, head) chains for the one-workgroup-per-chain kernel).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s + MFMA TFLOP/s (H=64,d=128,N=8K..1M); decode HBM GB/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
H, D, BETA = 64, 128, 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_bf16_n8k_hbm_traffic.txt")
KERNEL_SOURCES = ["linear_attention_la_amd/csrc/la_prefill_bf16.hip",
                  "linear_attention_la_amd/csrc/la_mfma.h",
                  "linear_attention_la_amd/csrc/la_device.h",
                  "linear_attention_la_amd/csrc/la_internal.h"]


def prefill_bytes(tokens, seqs, heads=H, d=D):
    """Algorithmic HBM bytes: Q, K, V read and O written once (2 B each), plus
    the fp32 final state."""
    return tokens * heads * d * 8 + seqs * heads * d * d * 4


def prefill_flops(tokens, heads=H, d=D, beta=BETA):
    """Algorithmic flops at block size beta: 4 d^2 (Q S and K^T V) plus
    2 d (beta + 1) (causal halves of Q K^T and P V) per token per head."""
    return tokens * heads * (4 * d * d + 2 * d * (beta + 1))


def decode_bytes(batch, heads=H, d=D):
    """fp32 state read and written, q/k/v read and o written in bf16."""
    return batch * heads * (8 * d * d + 8 * d)


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """Counter-measured HBM bytes per launch of the prefill kernel, if the
    counters were taken on the current kernel source (else None)."""
    try:
        rec = dict(line.split(":", 1) for line in open(TRAFFIC_FILE).read().splitlines()
                   if ":" in line and not line.startswith("#"))
    except (OSError, ValueError):
        return None
    rec = {k_.strip(): v_.strip() for k_, v_ in rec.items()}
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return int(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def launch_times(fn, reps, stream, flush=None):
    """Durations (s) of `reps` launches of `fn`, by HIP events on `stream`;
    `flush` runs between launches, outside the events."""
    import torch

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    with torch.cuda.stream(stream):
        for i in range(reps):
            if flush is not None:
                flush()
            starts[i].record(stream)
            fn(i)
            ends[i].record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) / 1e3 for s, e in zip(starts, ends)]


def timed_launches(fn, reps, stream, flush=None):
    """Average duration (s) of `fn` over `reps` launches (see launch_times)."""
    t = launch_times(fn, reps, stream, flush)
    return sum(t) / len(t)


def measured_peaks(dev):
    """Peaks measured on this GPU: HBM GB/s of a 1 GiB fp32 stream that reads
    and writes every element once (torch.mul with out=, the fastest of the
    torch streaming kernels here; copy_ reaches less) and bf16 TFLOP/s of an
    8192^3 torch matmul (hipBLASLt); both medians of 10 launches after
    warm-up."""
    import torch

    s = torch.cuda.current_stream()
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    t = sorted(launch_times(lambda i: torch.mul(src, 1.0, out=dst), 10, s))[5]
    stream_gbs = 2 * src.numel() * 4 / t / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.matmul(a, b)
    t = sorted(launch_times(lambda i: torch.matmul(a, b), 10, s))[5]
    gemm_tflops = 2 * n ** 3 / t / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"stream_GB_per_s": round(stream_gbs, 1), "stream_frac_of_8TBs": round(stream_gbs / HBM_PEAK_GBS, 4),
            "bf16_gemm_TFLOP_per_s": round(gemm_tflops, 1),
            "bf16_gemm_frac_of_2500": round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
            "note": "1 GiB fp32 read+write stream (torch.mul out=); 8192^3 bf16 matmul (hipBLASLt)"}


def cpu_baseline(budget_s=12.0):
    """fp64 oracle over heads of the N=8192 workload (host inputs of the same
    distribution), until budget_s of compute has been spent."""
    import oracle
    from la_inputs import decay_from_seed, host_qkv

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    N = 8192
    decay = decay_from_seed(H)
    heads_done, elapsed = 0, 0.0
    chunk = 8
    while elapsed < budget_s and heads_done < 32 * H:
        q, k, v = host_qkv(N, chunk, D, 5000 + heads_done)
        t0 = time.perf_counter()
        for j in range(chunk):
            oracle.blockwise(q[:, j], k[:, j], v[:, j], float(decay[(heads_done + j) % H]), BETA)
        elapsed += time.perf_counter() - t0
        heads_done += chunk
    tokens_equiv = N * heads_done / H
    return {"value": tokens_equiv / elapsed, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 blockwise oracle (beta={BETA}) on {heads_done} (sequence, head) "
                      f"chains of N={N}, d={D} ({heads_done / H:.2f}x the 64-head workload), "
                      f"{elapsed:.1f} s of compute on {len(os.sched_getaffinity(0))} "
                      f"visible host cores",
            "seconds": round(elapsed, 2)}


def bench_decode(dev, reps=20):
    import torch

    import linear_attention_la_amd as la
    from la_inputs import device_qkv, device_states, workload

    w = workload("mixed_decode")
    B = w["batch"]
    kv = device_states(B, H, D, w["seed"], dev, scale=0.5)
    q, k, v = (x.view(B, H, D) for x in device_qkv(B, H, D, w["seed"] + 1, dev))
    out = torch.empty_like(q)
    s = torch.cuda.current_stream()
    for _ in range(3):
        la.decode(q, k, v, kv, w["decay"], out=out)
    t = timed_launches(lambda i: la.decode(q, k, v, kv, w["decay"], out=out), reps, s)
    gbs = decode_bytes(B) / t / 1e9
    return {"batch": B, "heads": H, "head_dim": D, "us": round(t * 1e6, 2),
            "GB_per_s": round(gbs, 1), "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_launch": decode_bytes(B)}, (q, k, v, kv, out, w)


def bench_decode_pool(dev, reps=20, pool_size=1024):
    """la_decode_pool: the 256-sequence serving batch at random distinct
    slots of a pool of 1024 states (H=64, d=128); same bytes as la_decode."""
    import torch

    import linear_attention_la_amd as la
    from la_inputs import device_qkv, device_states, workload

    w = workload("mixed_decode")
    B = w["batch"]
    pool = device_states(pool_size, H, D, w["seed"] + 2, dev, scale=0.5)
    slots_h = np.random.default_rng(w["seed"]).choice(pool_size, size=B, replace=False)
    slots_h = slots_h.astype(np.int32)
    slots = torch.from_numpy(slots_h).to(dev)
    q, k, v = (x.view(B, H, D) for x in device_qkv(B, H, D, w["seed"] + 1, dev))
    out = torch.empty_like(q)
    s = torch.cuda.current_stream()
    run = lambda i: la.decode_pool(q, k, v, pool, slots, w["decay"], out=out,  # noqa: E731
                                   slots_host=slots_h)
    for _ in range(3):
        run(0)
    t = timed_launches(run, reps, s)
    gbs = decode_bytes(B) / t / 1e9
    del pool
    torch.cuda.empty_cache()
    return {"batch": B, "pool_size": pool_size, "heads": H, "head_dim": D,
            "us": round(t * 1e6, 2), "GB_per_s": round(gbs, 1),
            "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4)}


def bench_mixed(dev, dec_state, reps=10):
    import torch

    import linear_attention_la_amd as la
    from la_inputs import cu_seqlens, device_qkv, workload

    q, k, v, kv, out, wd = dec_state
    B = wd["batch"]
    wp = workload("mixed_prefill")
    cu = cu_seqlens(wp["lengths"])
    T = int(cu[-1])
    qp, kp, vp = device_qkv(T, H, D, wp["seed"], dev)
    cu_dev = torch.from_numpy(cu).to(dev)
    op = torch.empty_like(qp)
    kvp = torch.empty((len(wp["lengths"]), H, D, D), dtype=torch.float32, device=dev)
    sp, sd = torch.cuda.Stream(), torch.cuda.Stream()
    ev = {n: [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
          for n in ("p0", "p1", "d0", "d1")}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # The decode step is submitted first: it is the short, latency-bound
    # kernel of a serving step, and submitted first it takes the CUs before
    # the prefill's workgroups fill them (submitted second it waits for
    # prefill workgroups to drain and runs ~5x slower; the prefill's time is
    # the same either way).
    for i in range(reps):
        ev["d0"][i].record(sd)
        la.decode(q, k, v, kv, wd["decay"], stream=sd, out=out)
        ev["d1"][i].record(sd)
        ev["p0"][i].record(sp)
        la.prefill(qp, kp, vp, cu_dev, wp["decay"], stream=sp, out=op, kv_final=kvp,
                   cu_seqlens_host=cu)
        ev["p1"][i].record(sp)
        torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    tp = sum(a.elapsed_time(b) for a, b in zip(ev["p0"], ev["p1"])) / reps / 1e3
    td = sum(a.elapsed_time(b) for a, b in zip(ev["d0"], ev["d1"])) / reps / 1e3
    return {"prefill_seqs": len(wp["lengths"]), "prefill_tokens": T, "decode_batch": B,
            "prefill_us": round(tp * 1e6, 1), "decode_us_under_load": round(td * 1e6, 1),
            "decode_GB_per_s_under_load": round(decode_bytes(B) / td / 1e9, 1),
            "prefill_tokens_per_s_under_load": round(T / tp, 0),
            "step_wall_us": round(wall * 1e6, 1)}


SWEEP = ("sweep1024", "sweep4096", "sweep16384", "sweep65536", "sweep65536_nodecay", "n1m",
         "batch8_n8k", "varlen64")


def bench_sweep(dev, reps=20, names=SWEEP):
    import torch

    import linear_attention_la_amd as la
    from la_inputs import cu_seqlens, device_qkv, workload

    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB cache flush
    res = {}
    s = torch.cuda.current_stream()
    for name in names:
        w = workload(name)
        cu = cu_seqlens(w["lengths"])
        T = int(cu[-1])
        q, k, v = device_qkv(T, H, D, w["seed"], dev)
        cu_dev = torch.from_numpy(cu).to(dev)
        o = torch.empty_like(q)
        kvf = torch.empty((len(w["lengths"]), H, D, D), dtype=torch.float32, device=dev)
        run = lambda i: la.prefill(q, k, v, cu_dev, w["decay"], out=o, kv_final=kvf,  # noqa
                                   cu_seqlens_host=cu)
        run(0)
        n = reps if T <= 1 << 17 else 5  # >= 20 repeats, 5 for the 1M-token workloads
        ts = sorted(launch_times(run, n, s, flush=lambda: scratch.zero_()))
        t = ts[len(ts) // 2]
        by = prefill_bytes(T, len(w["lengths"]))
        res[name] = {"tokens": T, "seqs": len(w["lengths"]), "us": round(t * 1e6, 1),
                     "us_min": round(ts[0] * 1e6, 1),
                     "tokens_per_s": round(T / t, 0), "GB_per_s": round(by / t / 1e9, 1),
                     "frac_of_8TBs": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
                     "tflops_beta64": round(prefill_flops(T) / t / 1e12, 1)}
        del q, k, v, o, kvf
        torch.cuda.empty_cache()
    return res


def bench_backward(dev, reps=10, name="n8k"):
    """la_prefill_backward on the n8k workload (B=1, H=64, N=8192, d=128,
    bf16; the 32-column kernel) or on batch8_n8k (eight such sequences: the
    one-workgroup-per-chain kernel), with initial states and final-state
    gradients.  Algorithmic bytes: q, k, v, dO read and dq, dk, dv written
    (14 d B per token and head) plus kv_init and dkv_final read and dkv_init
    written."""
    import torch

    import linear_attention_la_amd as la
    from la_inputs import cu_seqlens, device_qkv, device_states, workload

    w = workload(name)
    cu = cu_seqlens(w["lengths"])
    S, N = len(w["lengths"]), int(cu[-1])
    q, k, v = device_qkv(N, H, D, w["seed"], dev)
    do = device_qkv(N, H, D, w["seed"] + 11, dev)[0]
    kv0 = device_states(S, H, D, w["seed"] + 12, dev, scale=0.1)
    g = device_states(S, H, D, w["seed"] + 13, dev, scale=0.1)
    cu_dev = torch.from_numpy(cu).to(dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dkv0 = torch.empty_like(kv0)
    ws = torch.empty(la.la_prefill_backward_workspace_size(S, H, D)[1], dtype=torch.uint8,
                     device=dev)
    run = lambda i: la.prefill_backward(q, k, v, do, cu_dev, w["decay"], kv_init=kv0,  # noqa
                                        dkv_final=g, cu_seqlens_host=cu, workspace=ws, dq=dq,
                                        dk=dk, dv=dv, dkv_init=dkv0)
    for _ in range(3):
        run(0)
    t = timed_launches(run, reps, torch.cuda.current_stream())
    by = N * H * 14 * D + 3 * S * H * D * D * 4
    del q, k, v, do, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {"workload": f"la_prefill_backward B={S} H={H} N={N // S} d={D} bf16 "
                        "(kv_init, dkv_final)",
            "us": round(t * 1e6, 1), "tokens_per_s": round(N / t, 0),
            "GB_per_s": round(by / t / 1e9, 1), "frac_of_8TBs": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": by}


SEG_H, SEG_N, SEG_LEN = 8, 1 << 20, 1 << 15


def bench_segmented(dev, reps=3):
    """Low-parallelism case: B=1, H=8, N=1,048,576, d=128 (one GPU's share
    of 64 heads split over 8 GPUs by head).  la_prefill has only 8 (sequence,
    head) chains (32 workgroups); la_prefill_segmented cuts the sequence into
    32 segments of 32,768 tokens, 256 (segment, head) chains -- enough for the
    one-workgroup-per-chain kernel -- and reads K and V a second time for the
    segment states."""
    import torch

    import linear_attention_la_amd as la
    from la_inputs import device_qkv, workload

    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB cache flush
    s = torch.cuda.current_stream()
    decay = np.asarray(workload("n1m")["decay"][:SEG_H], np.float32)
    q, k, v = device_qkv(SEG_N, SEG_H, D, 1006, dev)
    cu = np.array([0, SEG_N], np.int32)
    cu_dev = torch.from_numpy(cu).to(dev)
    o = torch.empty_like(q)
    kvf = torch.empty((1, SEG_H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(la.prefill_segmented_workspace_size(cu, SEG_H, D, SEG_LEN),
                     dtype=torch.uint8, device=dev)
    plain = lambda i: la.prefill(q, k, v, cu_dev, decay, out=o, kv_final=kvf,  # noqa: E731
                                 cu_seqlens_host=cu)
    seg = lambda i: la.prefill_segmented(q, k, v, cu_dev, decay, SEG_LEN, out=o,  # noqa: E731
                                         kv_final=kvf, cu_seqlens_host=cu, workspace=ws)
    plain(0)
    seg(0)
    tp = timed_launches(plain, reps, s, flush=lambda: scratch.zero_())
    ts = timed_launches(seg, reps, s, flush=lambda: scratch.zero_())
    by = prefill_bytes(SEG_N, 1, heads=SEG_H)
    res = {"workload": f"B=1 H={SEG_H} N={SEG_N} d={D} bf16, one sequence",
           "segment_len": SEG_LEN, "segments": SEG_N // SEG_LEN,
           "plain_us": round(tp * 1e6, 1), "segmented_us": round(ts * 1e6, 1),
           "speedup": round(tp / ts, 2),
           "plain_frac_of_8TBs": round(by / tp / 1e9 / HBM_PEAK_GBS, 4),
           "segmented_frac_of_8TBs": round(by / ts / 1e9 / HBM_PEAK_GBS, 4),
           "segmented_tokens_per_s": round(SEG_N / ts, 0),
           "extra_kv_bytes_segmented": SEG_N * SEG_H * D * 2 * 2}
    del q, k, v, o, kvf, ws, scratch
    torch.cuda.empty_cache()
    return res


def bench_backward_segmented(dev, reps=2):
    """The backward in the same low-parallelism case as bench_segmented
    (B=1, H=8, N=1,048,576, d=128, with S0 and dS_L): la_prefill_backward
    runs 3 x 8 chains, la_prefill_backward_segmented cuts each of its three
    chains into 32 segments of 32,768 tokens (256 chains a pass).
    Algorithmic bytes as in bench_backward."""
    import torch

    import linear_attention_la_amd as la
    from la_inputs import device_qkv, device_states, workload

    decay = np.asarray(workload("n1m")["decay"][:SEG_H], np.float32)
    q, k, v = device_qkv(SEG_N, SEG_H, D, 1007, dev)
    do = device_qkv(SEG_N, SEG_H, D, 1008, dev)[0]
    kv0 = device_states(1, SEG_H, D, 1009, dev, scale=0.1)
    g = device_states(1, SEG_H, D, 1010, dev, scale=0.1)
    cu = np.array([0, SEG_N], np.int32)
    cu_dev = torch.from_numpy(cu).to(dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dkv0 = torch.empty_like(kv0)
    ws = torch.empty(la.prefill_backward_segmented_workspace_size(cu, SEG_H, D, SEG_LEN),
                     dtype=torch.uint8, device=dev)
    wsp = torch.empty(la.la_prefill_backward_workspace_size(1, SEG_H, D)[1], dtype=torch.uint8,
                      device=dev)
    kw = dict(kv_init=kv0, dkv_final=g, cu_seqlens_host=cu, dq=dq, dk=dk, dv=dv, dkv_init=dkv0)
    plain = lambda i: la.prefill_backward(q, k, v, do, cu_dev, decay, workspace=wsp,  # noqa
                                          **kw)
    seg = lambda i: la.prefill_backward_segmented(q, k, v, do, cu_dev, decay, SEG_LEN,  # noqa
                                                  workspace=ws, **kw)
    plain(0)
    seg(0)
    s = torch.cuda.current_stream()
    tp = timed_launches(plain, reps, s)
    ts = timed_launches(seg, reps, s)
    by = SEG_N * SEG_H * 14 * D + 3 * SEG_H * D * D * 4
    del q, k, v, do, dq, dk, dv, ws, wsp
    torch.cuda.empty_cache()
    return {"workload": f"la_prefill_backward B=1 H={SEG_H} N={SEG_N} d={D} bf16 "
                        "(kv_init, dkv_final)",
            "segment_len": SEG_LEN, "plain_us": round(tp * 1e6, 1),
            "segmented_us": round(ts * 1e6, 1), "speedup": round(tp / ts, 2),
            "segmented_tokens_per_s": round(SEG_N / ts, 0),
            "segmented_frac_of_8TBs": round(by / ts / 1e9 / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip decode/mixed/sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (scale for HBM counters)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time la_decode on the 256 x 64-head serving batch")
    ap.add_argument("--pool-only", action="store_true",
                    help="only time la_decode_pool (256 sequences on a pool of 1024)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time la_prefill_backward on n8k and batch8_n8k")
    ap.add_argument("--sweep-only", choices=SWEEP,
                    help="only time one workload of the length / batch sweep")
    ap.add_argument("--segmented-only", action="store_true",
                    help="only time la_prefill vs la_prefill_segmented (and the two "
                         "backwards) at B=1, H=8, N=1M")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_la_amd as la
    from la_inputs import device_qkv, workload

    dev = torch.device("cuda:0")
    if args.pool_only:
        print(json.dumps({"decode_pool": bench_decode_pool(dev)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"backward": bench_backward(dev),
                          "backward_batch8": bench_backward(dev, name="batch8_n8k")}), flush=True)
        return
    if args.segmented_only:
        print(json.dumps({"segmented": bench_segmented(dev),
                          "backward_segmented": bench_backward_segmented(dev)}), flush=True)
        return
    if args.sweep_only:
        print(json.dumps({"sweep": bench_sweep(dev, names=(args.sweep_only,))}), flush=True)
        return
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": src.numel() * 4}))
        return
    if args.decode_only:
        la.lib()
        dec, _ = bench_decode(dev, reps=max(args.steps, 1))
        print(json.dumps({"decode": dec}))
        return
    la.lib()
    w = workload("n8k")
    N = w["lengths"][0]
    decay = w["decay"]
    sets = [device_qkv(N, H, D, w["seed"] + i, dev) for i in range(2)]
    cu_dev = torch.tensor([0, N], dtype=torch.int32, device=dev)
    cu_host = [0, N]
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
    kvf = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        q, k, v = sets[i & 1]
        la.prefill(q, k, v, cu_dev, decay, out=o, kv_final=kvf, cu_seqlens_host=cu_host)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev0[i].record(stream)
        step(i)
        ev1[i].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_s = sum(a.elapsed_time(b) for a, b in zip(ev0, ev1)) / args.steps / 1e3

    tokens_per_s = N * args.steps / elapsed
    by = prefill_bytes(N, 1)
    achieved = by / kern_s / 1e9
    tflops = prefill_flops(N) / kern_s / 1e12
    traffic = measured_traffic()
    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "la_prefill B=1 H=64 N=8192 d=128 bf16 in/out, fp32 state, "
                               "seeded per-head decay", "global_batch": 1, "seq_len": N,
                   "heads": H, "head_dim": D, "beta": BETA, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "prefill_bf16_kernel<128, false, false, false>",
                     "kernel_us": round(kern_s * 1e6, 2), "algorithmic_bytes": by},
        "mfma": {"tflops_algorithmic_beta64": round(tflops, 2),
                 "frac_of_2500": round(tflops / BF16_PEAK_TFLOPS, 4)},
    }
    if not args.no_extra:
        dec, dec_state = bench_decode(dev)
        line["decode"] = dec
        line["decode_pool"] = bench_decode_pool(dev)
        line["mixed"] = bench_mixed(dev, dec_state)
        del dec_state
        torch.cuda.empty_cache()
        line["sweep"] = bench_sweep(dev)
        peaks = measured_peaks(dev)
        line["peaks"] = peaks
        line["roofline"]["frac_of_measured_stream"] = round(achieved / peaks["stream_GB_per_s"], 4)
        line["segmented"] = bench_segmented(dev)
        line["backward_segmented"] = bench_backward_segmented(dev)
        line["backward"] = bench_backward(dev)
        line["backward_batch8"] = bench_backward(dev, name="batch8_n8k")
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
