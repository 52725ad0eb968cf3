"""Benchmark of the Lightning Attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

A timed step is one la_prefill over the workload B=1, H=64, N=8192, d=128,
bf16 Q/K/V ~ N(0,1)/sqrt(d), per-head decay exp(-U[0.001, 0.1]) (the
MiniMax-Text-01 lightning-layer shape at its 8192-token pretraining length).
Inputs are resident in HBM before timing starts; two input sets alternate
(1.08 GB together, four times the 256 MB Infinity Cache) so no step reads
inputs left in cache by the step before.  The step first runs untimed for
--settle-ms (200 ms: the GPU raises its clocks only after tens of ms of
sustained load), then W untimed warmup steps, then K timed steps back to
back, bracketed by torch.cuda.synchronize() and by one HIP event pair on
the launch stream.  Every other timed region below is preceded by the same
untimed settle of the operation it times.

One JSON line is printed with the contract fields plus:
  roofline      the prefill kernel's algorithmic HBM bytes per launch over
                its average launch time (one HIP event pair on its stream
                around the K timed steps), against
                8 TB/s; `traffic` is the counter-measured bytes per launch
                from profiles/ if it was taken on the current kernel source.
                config.la_ndv records the LA_NDV override of the library's
                kernel choice (null: unset, the 32-column kernel here).
  cpu_baseline  the fp64 oracle (blockwise, beta=64) timed on the host cores
                over heads of the same workload.
  mfma          algorithmic TFLOP/s at beta=64 against 2.5 PFLOP/s bf16.
  decode        la_decode alone on 256 sequences x 64 heads: GB/s vs 8 TB/s.
  fp32_prefill  la_prefill with fp32 inputs and output on the n8k shape (the
                fp32 kernel): TFLOP/s at beta=32 against the 157.3 TFLOP/s
                fp32 matrix peak, and GB/s against 8 TB/s.
  mixed         decode on one stream concurrent with a packed prefill of 8
                sequences (lengths U[1K, 32K]) on another.
  peaks         measured on the GPU: a 1 GiB read+write stream (HBM), an 8192^3
                bf16 matmul, and an MFMA-only loop on random and on zero
                operands with the shader clock it ran at;
                roofline.frac_of_measured_stream relates the prefill kernel
                to that stream.
  sweep         tokens/s at N = 1K ... 1M, for three, five and eight 8K
                sequences in one call (192, 320 and 512 chains: the
                one-workgroup-per-chain kernel, for 320 chains followed by
                the 32-column kernel on the fifth sequence) and for a packed
                varlen batch (that kernel as well): back-to-back
                launches over input sets that together exceed 1 GiB;
                sweep_flatness gives max/min tokens/s over 1K ... 1M; each entry's
                wide_seqs (la_prefill_kernel_plan) counts the sequences run one
                workgroup per chain, the rest in 32-column slices.
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
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak
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


def prefill_fp32_bytes(tokens, seqs, heads=H, d=D):
    """Algorithmic HBM bytes of an fp32-in, fp32-out prefill: Q, K, V read and
    O written once (4 B each), plus the fp32 final state."""
    return tokens * heads * d * 16 + seqs * heads * d * d * 4


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


def region_time(fn, reps, stream):
    """Average duration (s) of `fn` over `reps` launches run back to back
    inside one HIP event pair on `stream` (events between launches would
    serialise the stream and add ~20 us to each)."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps / 1e3


def timed_launches(fn, reps, stream, flush=None):
    """Average duration (s) of `fn` over `reps` launches (see launch_times)."""
    t = launch_times(fn, reps, stream, flush)
    return sum(t) / len(t)


SETTLE_S = 0.2  # set from --settle-ms


def settle(fn, seconds=None):
    """Run ``fn`` back to back, untimed, for ``seconds`` (default: the
    --settle-ms setting) and wait for it: the GPU raises its clocks only
    after tens of milliseconds of sustained load and lowers them again after
    an idle gap, so every timed region is preceded by this.  Returns the
    number of launches."""
    import torch

    seconds = SETTLE_S if seconds is None else seconds
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 8 == 0:  # keep the queue short so the host clock tracks the GPU
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


PEAK_LIB = os.path.join(ROOT, "linear_attention_la_amd", "_lib", "libla_peak.so")


def mfma_loop_peak(dev, iters=10000, reps=10):
    """bf16 MFMA rate of an MFMA-only loop (libla_peak.so: no memory traffic,
    8 independent accumulators a wave, 16 waves on every compute unit), on
    N(0,1) operands and on zero operands: TFLOP/s (region time of `reps`
    launches after a settle) and the shader clock the waves ran at (their
    shader-clock count over the 100 MHz constant clock, median over
    waves).  The operands decide how much the matrix cores switch, hence
    the power the loop draws and the clock the board's power limit allows.
    None if the library was not built."""
    import ctypes

    import torch

    if not os.path.exists(PEAK_LIB):
        return None
    L = ctypes.CDLL(PEAK_LIB)
    L.la_peak_mfma_bf16.restype = ctypes.c_int
    L.la_peak_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    threads, waves = cus * 1024, cus * 16
    s = torch.cuda.current_stream()
    sums = torch.empty(threads, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2 * waves, dtype=torch.int64, device=dev)
    flops = waves * iters * 8 * 16 * 16 * 32 * 2
    res = {}
    for name in ("random", "zeros"):
        g = torch.Generator(device=dev).manual_seed(7)
        ops = (torch.randn(threads * 128, generator=g, device=dev) if name == "random"
               else torch.zeros(threads * 128, device=dev)).to(torch.bfloat16)

        def run(i):
            st = L.la_peak_mfma_bf16(ops.data_ptr(), sums.data_ptr(), clocks.data_ptr(), cus,
                                     iters, ctypes.c_void_p(s.cuda_stream))
            if st != 0:
                raise RuntimeError(f"la_peak_mfma_bf16: HIP error {st}")
        settle(run)
        t = region_time(run, reps, s)
        c = clocks.view(waves, 2).cpu().numpy()
        ghz = float(np.median(c[:, 0] / np.maximum(c[:, 1], 1))) * 0.1
        res[name] = {"TFLOP_per_s": round(flops / t / 1e12, 1),
                     "frac_of_2500": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "clock_GHz": round(ghz, 3), "us_per_launch": round(t * 1e6, 1)}
        del ops
    del sums, clocks
    return res


def mfma_loop_peak_f32(dev, iters=2500, reps=10):
    """fp32 MFMA rate of the MFMA-only loop on v_mfma_f32_16x16x4_f32
    (libla_peak.so, as mfma_loop_peak) on N(0,1) operands: TFLOP/s against
    the 157.3 TFLOP/s fp32 matrix peak and the shader clock.  None if the
    library was not built."""
    import ctypes

    import torch

    if not os.path.exists(PEAK_LIB):
        return None
    L = ctypes.CDLL(PEAK_LIB)
    L.la_peak_mfma_f32.restype = ctypes.c_int
    L.la_peak_mfma_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    threads, waves = cus * 1024, cus * 16
    s = torch.cuda.current_stream()
    sums = torch.empty(threads, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2 * waves, dtype=torch.int64, device=dev)
    g = torch.Generator(device=dev).manual_seed(7)
    ops = torch.randn(threads * 16, generator=g, device=dev)
    flops = waves * iters * 8 * 16 * 16 * 4 * 2

    def run(i):
        st = L.la_peak_mfma_f32(ops.data_ptr(), sums.data_ptr(), clocks.data_ptr(), cus, iters,
                                ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            raise RuntimeError(f"la_peak_mfma_f32: HIP error {st}")
    settle(run)
    t = region_time(run, reps, s)
    c = clocks.view(waves, 2).cpu().numpy()
    ghz = float(np.median(c[:, 0] / np.maximum(c[:, 1], 1))) * 0.1
    del ops, sums, clocks
    return {"TFLOP_per_s": round(flops / t / 1e12, 1),
            "frac_of_157_3": round(flops / t / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
            "clock_GHz": round(ghz, 3), "us_per_launch": round(t * 1e6, 1)}


def measured_peaks(dev):
    """Peaks measured on this GPU: HBM GB/s of a 1 GiB fp32 stream that reads
    and writes every element once (torch.mul with out=, the fastest of the
    torch streaming kernels here; copy_ reaches less), bf16 TFLOP/s of an
    8192^3 torch matmul (hipBLASLt), both medians of 10 launches (the
    matmul's after a settle), and the MFMA-only loop of mfma_loop_peak."""
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
    settle(lambda i: torch.matmul(a, b))
    t = sorted(launch_times(lambda i: torch.matmul(a, b), 10, s))[5]
    gemm_tflops = 2 * n ** 3 / t / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"stream_GB_per_s": round(stream_gbs, 1), "stream_frac_of_8TBs": round(stream_gbs / HBM_PEAK_GBS, 4),
            "bf16_gemm_TFLOP_per_s": round(gemm_tflops, 1),
            "bf16_gemm_frac_of_2500": round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
            "mfma_loop_bf16": mfma_loop_peak(dev),
            "mfma_loop_f32": mfma_loop_peak_f32(dev),
            "note": "1 GiB fp32 read+write stream (torch.mul out=); 8192^3 bf16 matmul (hipBLASLt); "
                    "MFMA-only loop on N(0,1) and on zero operands (libla_peak.so)"}


def _host_info():
    """CPU model, usable host cores and the BLAS library numpy runs on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info

        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            b = libs[0]
            blas = f"{b.get('internal_api')} {b.get('version')} ({os.path.basename(b.get('filepath', ''))})"
            threads = int(b.get("num_threads", threads))
    except Exception:  # pragma: no cover
        pass
    return model, blas, threads


def cpu_baseline(budget_s=12.0, decode_budget_s=4.0):
    """The fp64 oracle on the host cores: prefill over (sequence, head)
    chains of the N=8192 workload's shape (host inputs of the same
    distribution) until budget_s of compute has been spent, reported as
    tokens/s of the 64-head workload; and the decode step over states of the
    256 x 64 serving batch until decode_budget_s, reported as GB/s of the
    decode's algorithmic bytes."""
    import oracle
    from la_inputs import decay_from_seed, host_qkv, random_states

    model, blas, threads = _host_info()
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
    # decode: one step per (sequence, head) state, in batches of 64 heads
    states_done, d_elapsed = 0, 0.0
    while d_elapsed < decode_budget_s and states_done < 256 * H:
        kv = random_states(1, H, D, 6000 + states_done)
        q, k, v = (x.reshape(1, H, D) for x in host_qkv(H, 1, D, 7000 + states_done))
        t0 = time.perf_counter()
        oracle.decode_batch(q, k, v, kv, decay)
        d_elapsed += time.perf_counter() - t0
        states_done += H
    dec_gbs = states_done * (8 * D * D + 8 * D) / d_elapsed / 1e9
    cores = len(os.sched_getaffinity(0))
    return {"value": tokens_equiv / elapsed, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 blockwise oracle (beta={BETA}) on {heads_done} (sequence, head) "
                      f"chains of N={N}, d={D} ({heads_done / H:.2f}x the 64-head workload), "
                      f"{elapsed:.1f} s of compute; decode: {states_done} (sequence, head) "
                      f"states of d={D}, {d_elapsed:.1f} s; {cores} visible host cores",
            "seconds": round(elapsed, 2),
            "decode": {"GB_per_s": round(dec_gbs, 3), "states": states_done,
                       "seconds": round(d_elapsed, 2),
                       "bytes_per_state": 8 * D * D + 8 * D},
            "cpu_model": model, "visible_cores": cores, "blas": blas,
            "blas_threads": int(threads)}


def bench_decode(dev, reps=20):
    """la_decode on the 256 x 64 serving batch (d = 128, bf16, fp32 states
    updated in place, made by a seeded prefill of 256 sequences of U[256,
    2048] tokens): settled, then `reps` launches back to back in one event
    pair.  Returns the record and the inputs (for bench_mixed)."""
    import torch

    import linear_attention_la_amd as la
    from la_inputs import cu_seqlens, device_qkv, workload

    w = workload("mixed_decode")
    B = w["batch"]
    cu_s = cu_seqlens(w["state_lengths"])
    qs, ks, vs = device_qkv(int(cu_s[-1]), H, D, w["seed"] + 7, dev)
    kv = la.prefill(qs, ks, vs, torch.from_numpy(cu_s).to(dev), w["decay"],
                    cu_seqlens_host=cu_s)[1]
    del qs, ks, vs
    torch.cuda.empty_cache()
    q, k, v = (x.view(B, H, D) for x in device_qkv(B, H, D, w["seed"] + 1, dev))
    out = torch.empty_like(q)
    s = torch.cuda.current_stream()
    for _ in range(3):
        la.decode(q, k, v, kv, w["decay"], out=out)
    settle(lambda i: la.decode(q, k, v, kv, w["decay"], out=out))
    t = region_time(lambda i: la.decode(q, k, v, kv, w["decay"], out=out), reps, s)
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
    settle(run)
    t = region_time(run, reps, s)
    gbs = decode_bytes(B) / t / 1e9
    del pool
    torch.cuda.empty_cache()
    return {"batch": B, "pool_size": pool_size, "heads": H, "head_dim": D,
            "us": round(t * 1e6, 2), "GB_per_s": round(gbs, 1),
            "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4)}


def bench_mixed(dev, dec_state, reps=10, warmup=2):
    """The mixed serving step: the 256 x 64 decode batch (la_decode) and a
    packed prefill of 8 sequences of U[1K, 32K] tokens (la_prefill, the
    one-workgroup-per-chain kernel) on two streams.  Run with either kernel
    submitted first, and with the decode arriving ~0.2 ms after the prefill
    has started (``prefill_running``), on plain streams and on streams
    restricted to disjoint compute units (decode 1/8 or 1/4 of them, prefill
    the rest).  Per variant:
    ``warmup`` untimed steps, then ``reps`` steps timed by HIP events on the
    two streams against one start event both wait for: each kernel's time
    from its submission point, and the step's time to the later of the two
    ends.  ``step_frac_of_8TBs`` is the step's algorithmic bytes (decode and
    prefill together) over its time."""
    import torch

    import linear_attention_la_amd as la
    from la_inputs import cu_seqlens, device_qkv, workload

    q, k, v, kv, out, wd = dec_state
    B = wd["batch"]
    wp = workload("mixed_prefill")
    cu = cu_seqlens(wp["lengths"])
    T = int(cu[-1])
    S = len(wp["lengths"])
    qp, kp, vp = device_qkv(T, H, D, wp["seed"], dev)
    cu_dev = torch.from_numpy(cu).to(dev)
    op = torch.empty_like(qp)
    kvp = torch.empty((S, H, D, D), dtype=torch.float32, device=dev)
    step_bytes = decode_bytes(B) + prefill_bytes(T, S)
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    full = (1 << n_cu) - 1
    dec8, dec4 = (1 << (n_cu // 8)) - 1, (1 << (n_cu // 4)) - 1
    streams = {"plain": (torch.cuda.Stream(), torch.cuda.Stream()),
               "cu_masked_8th": (la.cu_masked_stream(full & ~dec8), la.cu_masked_stream(dec8)),
               "cu_masked_4th": (la.cu_masked_stream(full & ~dec4), la.cu_masked_stream(dec4))}
    main = torch.cuda.current_stream()

    def dec(sd):
        la.decode(q, k, v, kv, wd["decay"], stream=sd, out=out)

    def pre(sp):
        la.prefill(qp, kp, vp, cu_dev, wp["decay"], stream=sp, out=op, kv_final=kvp,
                   cu_seqlens_host=cu)

    # each kernel alone, same protocol
    alone = {}
    for name, fn in (("decode", dec), ("prefill", pre)):
        for _ in range(warmup):
            fn(main)
        alone[name] = timed_launches(lambda i: fn(main), reps, main)
    res = {"prefill_seqs": S, "prefill_tokens": T, "decode_batch": B,
           "step_bytes": step_bytes, "compute_units": n_cu,
           "decode_alone_us": round(alone["decode"] * 1e6, 1),
           "prefill_alone_us": round(alone["prefill"] * 1e6, 1),
           "serial_sum_us": round((alone["decode"] + alone["prefill"]) * 1e6, 1)}
    # cycles of torch's spin kernel that hold the decode back until the
    # prefill's workgroups occupy the GPU (about 0.2 ms)
    late_cycles = 400_000
    for sname, (sp, sd) in streams.items():
        for first in ("decode", "prefill", "prefill_running"):
            if first == "decode":
                order = lambda: (dec(sd), pre(sp))  # noqa: E731
            elif first == "prefill":
                order = lambda: (pre(sp), dec(sd))  # noqa: E731
            else:
                order = None
            decode_first = first == "decode"
            ev = {n: [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
                  for n in ("s", "d0", "d1", "p0", "p1")}
            for it in range(warmup + reps):
                i = it - warmup
                if i >= 0:
                    ev["s"][i].record(main)
                    sd.wait_event(ev["s"][i])
                    sp.wait_event(ev["s"][i])
                else:
                    sd.wait_stream(main)
                    sp.wait_stream(main)
                if order is not None:
                    if i >= 0:
                        ev["d0"][i].record(sd)
                        ev["p0"][i].record(sp)
                    order()
                else:  # the decode arrives while the prefill runs
                    if i >= 0:
                        ev["p0"][i].record(sp)
                    pre(sp)
                    with torch.cuda.stream(sd):
                        torch.cuda._sleep(late_cycles)
                    if i >= 0:
                        ev["d0"][i].record(sd)
                    dec(sd)
                if i >= 0:
                    ev["d1"][i].record(sd)
                    ev["p1"][i].record(sp)
                main.wait_stream(sd)
                main.wait_stream(sp)
            torch.cuda.synchronize()
            t = {n: np.array([ev["s"][i].elapsed_time(ev[n][i]) for i in range(reps)]) * 1e3
                 for n in ("d0", "d1", "p0", "p1")}
            step = np.maximum(t["d1"], t["p1"])
            dec_us = float(np.median(t["d1"] - t["d0"]))
            del decode_first
            res[f"{sname}_{first}" + ("" if first == "prefill_running" else "_first")] = {
                "decode_us": round(dec_us, 1),
                "prefill_us": round(float(np.median(t["p1"] - t["p0"])), 1),
                "step_us": round(float(np.median(step)), 1),
                "decode_vs_alone": round(dec_us / (alone["decode"] * 1e6), 3),
                "step_frac_of_8TBs": round(step_bytes / float(np.median(step)) / 1e3 / HBM_PEAK_GBS,
                                           4)}
    # one stream, decode then prefill: the decode runs alone and the step is
    # the serial sum
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for it in range(warmup + reps):
        e = ev[it - warmup] if it >= warmup else None
        if e:
            e[0].record(main)
        dec(main)
        if e:
            e[1].record(main)
        pre(main)
        if e:
            e[2].record(main)
    torch.cuda.synchronize()
    d_us = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    st_us = float(np.median([e[0].elapsed_time(e[2]) for e in ev])) * 1e3
    res["one_stream_decode_then_prefill"] = {
        "decode_us": round(d_us, 1), "step_us": round(st_us, 1),
        "decode_vs_alone": round(d_us / (alone["decode"] * 1e6), 3),
        "step_frac_of_8TBs": round(step_bytes / st_us / 1e3 / HBM_PEAK_GBS, 4)}
    del qp, kp, vp, op, kvp, streams
    torch.cuda.empty_cache()
    return res


def bench_normed(dev, reps=10):
    """The output normalisation fused into the kernels that write O
    (la_prefill_normed, la_decode_normed; weight [H, d], eps 1e-6, a bf16
    gate) against the same result unfused: la_prefill / la_decode, then the
    normalisation and gate as torch operations on the written output.  Three
    prefill shapes: eight 8K sequences (one workgroup per chain), five (one
    wave of that kernel, then the chained scan for the fifth) and the
    headline B=1, N=8192 (fused: the chained scan; unfused: the 32-column
    kernel); and the 256 x 64 decode batch.  Algorithmic bytes of the fused
    prefill: the plain prefill's plus the gate read (2 B per element); the
    unfused path also writes O and reads it back."""
    import torch

    import linear_attention_la_amd as la
    from la_inputs import cu_seqlens, device_qkv, device_states, workload

    s = torch.cuda.current_stream()
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB cache flush
    eps = 1e-6
    w = torch.rand((H, D), dtype=torch.float32, device=dev) + 0.5

    def epilogue(o, gate):
        of = o.float()
        y = of * torch.rsqrt(of.pow(2).mean(-1, keepdim=True) + eps) * w * torch.sigmoid(gate.float())
        return y.to(o.dtype)

    res = {}
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    for name in ("batch8_n8k", "batch5_n8k", "n8k"):
        wl = workload(name)
        cu = cu_seqlens(wl["lengths"])
        T, S = int(cu[-1]), len(wl["lengths"])
        q, k, v = device_qkv(T, H, D, wl["seed"], dev)
        gate = device_qkv(T, H, D, wl["seed"] + 21, dev)[0]
        cu_dev = torch.from_numpy(cu).to(dev)
        o = torch.empty_like(q)
        kvf = torch.empty((S, H, D, D), dtype=torch.float32, device=dev)
        need = la.prefill_normed_workspace_size(cu, H, D)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        fused = lambda i: la.prefill_normed(q, k, v, cu_dev, wl["decay"], w, eps, gate, out=o,  # noqa
                                            kv_final=kvf, cu_seqlens_host=cu, workspace=ws)
        unfused = lambda i: epilogue(la.prefill(q, k, v, cu_dev, wl["decay"], out=o,  # noqa
                                                kv_final=kvf, cu_seqlens_host=cu)[0], gate)
        fused_ng = lambda i: la.prefill_normed(q, k, v, cu_dev, wl["decay"], w, eps, None,  # noqa
                                               out=o, kv_final=kvf, cu_seqlens_host=cu,
                                               workspace=ws)
        plain = lambda i: la.prefill(q, k, v, cu_dev, wl["decay"], out=o, kv_final=kvf,  # noqa
                                     cu_seqlens_host=cu)
        for fn in (fused, unfused, fused_ng, plain):
            fn(0)
        settle(fused)
        med = lambda fn: sorted(launch_times(fn, reps, s, flush=lambda: scratch.zero_()))[reps // 2]  # noqa
        tf, tu, tn, tp = med(fused), med(unfused), med(fused_ng), med(plain)
        by = prefill_bytes(T, S) + T * H * D * 2
        path = ("one workgroup per chain" if need == 0 else
                "one workgroup per chain, then the chained scan" if 2 * S * H > cus else
                "chained scan")
        res[name] = {"tokens": T, "seqs": S, "path": path, "fused_us": round(tf * 1e6, 1),
                     "fused_no_gate_us": round(tn * 1e6, 1), "plain_prefill_us": round(tp * 1e6, 1),
                     "unfused_us": round(tu * 1e6, 1), "speedup": round(tu / tf, 3),
                     "fused_frac_of_8TBs": round(by / tf / 1e9 / HBM_PEAK_GBS, 4)}
        del q, k, v, gate, o, kvf, ws
        torch.cuda.empty_cache()
    wd = workload("mixed_decode")
    B = wd["batch"]
    kv = device_states(B, H, D, wd["seed"], dev, scale=0.5)
    q, k, v = (x.view(B, H, D) for x in device_qkv(B, H, D, wd["seed"] + 1, dev))
    gate = device_qkv(B, H, D, wd["seed"] + 3, dev)[0].view(B, H, D)
    out = torch.empty_like(q)
    fused = lambda i: la.decode_normed(q, k, v, kv, wd["decay"], w, eps, gate, out=out)  # noqa
    unfused = lambda i: epilogue(la.decode(q, k, v, kv, wd["decay"], out=out), gate)  # noqa
    for fn in (fused, unfused):
        fn(0)
    settle(fused)
    tf = timed_launches(fused, 20, s)
    tu = timed_launches(unfused, 20, s)
    res["decode_b256"] = {"fused_us": round(tf * 1e6, 1), "unfused_us": round(tu * 1e6, 1),
                          "speedup": round(tu / tf, 3)}
    del scratch, kv
    torch.cuda.empty_cache()
    return res


SWEEP = ("sweep1024", "sweep4096", "sweep16384", "sweep65536", "sweep65536_nodecay", "n1m",
         "batch3_n8k", "batch5_n8k", "batch8_n8k", "varlen64")


def bench_sweep(dev, reps=20, names=SWEEP, footprint=1 << 30):
    """Tokens/s per workload of the length / batch sweep.  Several input sets
    are generated so that together they exceed ``footprint`` (1 GiB, four
    times the 256 MB Infinity Cache; one set when a set alone is larger), and
    ``reps`` launches (5 for the 1M-token workloads) run back to back over
    them in turn, so no launch finds its inputs in cache; one event pair on
    the stream around them gives the average launch time (``us``).  For
    comparison with earlier records, ``us_single`` is the median of single
    launches each bracketed by its own events after a 1 GiB cache flush
    (events between launches add ~20 us to each)."""
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
        S = len(w["lengths"])
        set_bytes = T * H * D * 2 * 3
        n_sets = 1 if set_bytes >= footprint else -(-footprint // set_bytes)
        sets = [device_qkv(T, H, D, w["seed"] + 100 * i, dev) for i in range(n_sets)]
        cu_dev = torch.from_numpy(cu).to(dev)
        o = torch.empty_like(sets[0][0])
        kvf = torch.empty((S, H, D, D), dtype=torch.float32, device=dev)

        def run(i):
            q, k, v = sets[i % n_sets]
            la.prefill(q, k, v, cu_dev, w["decay"], out=o, kv_final=kvf, cu_seqlens_host=cu)

        n = reps if T <= 1 << 17 else 5
        for i in range(min(n, 3)):
            run(i)
        settle(run)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for i in range(n):
            run(i)
        e1.record(s)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / n / 1e3
        ts = sorted(launch_times(run, n, s, flush=lambda: scratch.zero_()))
        by = prefill_bytes(T, S)
        wide_seqs = la.kernel_plan(cu, H, D)[0]  # sequences on the one-workgroup-per-chain kernel
        res[name] = {"tokens": T, "seqs": S, "us": round(t * 1e6, 1),
                     "us_single": round(ts[len(ts) // 2] * 1e6, 1), "input_sets": n_sets,
                     "tokens_per_s": round(T / t, 0), "GB_per_s": round(by / t / 1e9, 1),
                     "frac_of_8TBs": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
                     "tflops_beta64": round(prefill_flops(T) / t / 1e12, 1),
                     "wide_seqs": int(wide_seqs)}
        del sets, o, kvf
        torch.cuda.empty_cache()
    return res


def sweep_flatness(sweep):
    """max / min of tokens/s over the single-sequence length sweep (B=1,
    H=64: 1K ... 1M tokens, with and without decay), and over 4K ... 1M."""
    single = {k: v["tokens_per_s"] for k, v in sweep.items()
              if k.startswith("sweep") or k == "n1m"}
    if not single:
        return None
    no1k = {k: v for k, v in single.items() if k != "sweep1024"}
    ratio = lambda d: round(max(d.values()) / min(d.values()), 3) if d else None  # noqa: E731
    return {"max_over_min_1k_1m": ratio(single), "max_over_min_4k_1m": ratio(no1k),
            "workloads": sorted(single)}


def bench_backward(dev, reps=10, name="n8k"):
    """la_prefill_backward on the n8k workload (B=1, H=64, N=8192, d=128,
    bf16: its three chains in one launch, 192 workgroups) or on batch8_n8k
    (eight such sequences, 1536 workgroups), with initial states and
    final-state gradients; settled, then `reps` calls back to back in one
    event pair.  Algorithmic bytes: q, k, v, dO read and dq, dk, dv written
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
    settle(run)
    t = region_time(run, reps, torch.cuda.current_stream())
    by = N * H * 14 * D + 3 * S * H * D * D * 4
    del q, k, v, do, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {"workload": f"la_prefill_backward B={S} H={H} N={N // S} d={D} bf16 "
                        "(kv_init, dkv_final)",
            "us": round(t * 1e6, 1), "tokens_per_s": round(N / t, 0),
            "GB_per_s": round(by / t / 1e9, 1), "frac_of_8TBs": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": by}


def bench_prefill_fp32(dev, reps=10):
    """la_prefill with fp32 inputs and fp32 output on the n8k shape (B=1,
    H=64, N=8192, d=128): the fp32 kernel (fp32 matrix cores, beta = 32, 256
    workgroups); settled, then `reps` calls back to back in one event pair.
    Algorithmic flops at beta = 32: 4 d^2 + 2 d (beta + 1) per token and head;
    algorithmic bytes: q, k, v read and o written in fp32 plus the final
    state."""
    import torch

    import linear_attention_la_amd as la
    from la_inputs import cu_seqlens, device_qkv, workload

    w = workload("n8k")
    cu = cu_seqlens(w["lengths"])
    N = int(cu[-1])
    q, k, v = device_qkv(N, H, D, w["seed"], dev, dtype="fp32")
    cu_dev = torch.from_numpy(cu).to(dev)
    o = torch.empty_like(q)
    kv = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    run = lambda i: la.prefill(q, k, v, cu_dev, w["decay"], cu_seqlens_host=cu, out=o,  # noqa
                               kv_final=kv)
    for _ in range(3):
        run(0)
    settle(run)
    t = region_time(run, reps, torch.cuda.current_stream())
    flops = prefill_flops(N, beta=32)
    by = prefill_fp32_bytes(N, 1)
    del q, k, v, o, kv
    torch.cuda.empty_cache()
    return {"workload": f"la_prefill B=1 H={H} N={N} d={D} fp32 in/out, fp32 state",
            "kernel": "prefill_f32_kernel<128, float>",
            "us": round(t * 1e6, 1), "tokens_per_s": round(N / t, 0),
            "TFLOP_per_s": round(flops / t / 1e12, 2),
            "frac_of_fp32_mfma_peak": round(flops / t / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
            "GB_per_s": round(by / t / 1e9, 1),
            "frac_of_8TBs": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_flops": flops, "algorithmic_bytes": by}


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
    settle(plain)
    tp = timed_launches(plain, reps, s, flush=lambda: scratch.zero_())
    settle(seg)
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
    settle(plain)
    tp = timed_launches(plain, reps, s)
    settle(seg)
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
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps for this long before the warm-up steps (clock ramp)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (scale for HBM counters)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time la_decode on the 256 x 64-head serving batch")
    ap.add_argument("--peaks-only", action="store_true",
                    help="only the measured HBM stream, GEMM and MFMA-loop peaks")
    ap.add_argument("--normed-only", action="store_true",
                    help="only time the fused output normalisation against the unfused one")
    ap.add_argument("--mixed-only", action="store_true",
                    help="only time the mixed serving step (decode beside a packed prefill)")
    ap.add_argument("--pool-only", action="store_true",
                    help="only time la_decode_pool (256 sequences on a pool of 1024)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time la_prefill_backward on n8k and batch8_n8k")
    ap.add_argument("--fp32-only", action="store_true",
                    help="only time la_prefill with fp32 inputs on the n8k shape")
    ap.add_argument("--sweep-only", choices=SWEEP,
                    help="only time one workload of the length / batch sweep")
    ap.add_argument("--segmented-only", action="store_true",
                    help="only time la_prefill vs la_prefill_segmented (and the two "
                         "backwards) at B=1, H=8, N=1M")
    args = ap.parse_args()
    global SETTLE_S
    SETTLE_S = args.settle_ms / 1e3
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
    if args.fp32_only:
        print(json.dumps({"fp32_prefill": bench_prefill_fp32(dev),
                          "mfma_loop_f32": mfma_loop_peak_f32(dev)}), flush=True)
        return
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": src.numel() * 4}))
        return
    if args.peaks_only:
        print(json.dumps({"peaks": measured_peaks(dev)}), flush=True)
        return
    if args.normed_only:
        la.lib()
        print(json.dumps({"normed": bench_normed(dev)}), flush=True)
        return
    if args.mixed_only:
        la.lib()
        _, dec_state = bench_decode(dev, reps=3)
        print(json.dumps({"mixed": bench_mixed(dev, dec_state)}), flush=True)
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

    # Settle: the GPU raises its clocks only after tens of milliseconds of
    # sustained load (measured on this workload: 201 us a launch after 5
    # launches, 172-174 us after 150, and 206 us again after 0.5 s idle), so
    # the step runs untimed for --settle-ms before the W warm-up steps.
    settle_steps = settle(step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # One event pair around the K back-to-back steps (events between steps
    # would serialise the stream and add ~20 us to every launch): the
    # kernel's average launch duration over the timed region.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_s = ev0.elapsed_time(ev1) / args.steps / 1e3

    tokens_per_s = N * args.steps / elapsed
    by = prefill_bytes(N, 1)
    achieved = by / kern_s / 1e9
    tflops = prefill_flops(N) / kern_s / 1e12
    # LA_NDV (sweep override of the library's kernel choice) is recorded;
    # unset, this workload (64 chains) runs the 32-column kernel
    ndv = os.environ.get("LA_NDV") or None
    kernel = ("prefill_wide_kernel<false, false, false>" if ndv == "1"
              else "prefill_bf16_kernel<128, false, false, false>")
    traffic = measured_traffic() if ndv in (None, "4") else None
    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "la_prefill B=1 H=64 N=8192 d=128 bf16 in/out, fp32 state, "
                               "seeded per-head decay", "global_batch": 1, "seq_len": N,
                   "heads": H, "head_dim": D, "beta": BETA, "parallelism": "single GPU",
                   "la_ndv": ndv},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kernel,
                     "kernel_us": round(kern_s * 1e6, 2), "algorithmic_bytes": by},
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "mfma": {"tflops_algorithmic_beta64": round(tflops, 2),
                 "frac_of_2500": round(tflops / BF16_PEAK_TFLOPS, 4)},
    }
    if not args.no_extra:
        dec, dec_state = bench_decode(dev)
        line["decode"] = dec
        line["decode_pool"] = bench_decode_pool(dev)
        line["mixed"] = bench_mixed(dev, dec_state)
        line["normed"] = bench_normed(dev)
        del dec_state
        torch.cuda.empty_cache()
        line["sweep"] = bench_sweep(dev)
        line["sweep_flatness"] = sweep_flatness(line["sweep"])
        peaks = measured_peaks(dev)
        line["peaks"] = peaks
        line["roofline"]["frac_of_measured_stream"] = round(achieved / peaks["stream_GB_per_s"], 4)
        line["segmented"] = bench_segmented(dev)
        line["backward_segmented"] = bench_backward_segmented(dev)
        line["backward"] = bench_backward(dev)
        line["backward_batch8"] = bench_backward(dev, name="batch8_n8k")
        line["fp32_prefill"] = bench_prefill_fp32(dev)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
