"""Seeded synthetic inputs for Lightning Attention prefill and decode.

This module is the only code that both the oracle-side checks and the HIP
path's callers (tests, bench, smoke) use.  It draws random numbers and
packs them; it holds none of the attention arithmetic.

Workloads (sizes of the MiniMax-Text-01 lightning layers: 64 heads of
width 128, mizuki blog "MiniMax-01：4M 上下文破局" §二 架构总览; 8192-token
pretraining length, CSDN translation §3.1; 1M-token context, emonzhong.com
summary 关键结论; 1K-64K length sweep, mizuki blog §三; packed varlen
batches, CSDN §3.2; separate decode and prefill on two streams, jvyan.cn
二、计算优化):

* ``tiny``      1 x 256 tokens, 2 heads, d=64, fp32, decay {1.0, 0.9}.
* ``n8k``       1 x 8192 tokens, 64 heads, d=128, bf16.
* ``sweep``     1 x {1K, 4K, 16K, 64K} tokens, plus a no-decay 64K run.
* ``n1m``       1 x 1,048,576 tokens.
* ``batch8_n8k`` 8 x 8192 tokens (the n8k shape, batched).
* ``varlen64``  64 sequences, lengths log-uniform in [512, 131072].
* ``mixed``     256 decode tokens (1 per sequence) beside a prefill of 8
                sequences with lengths uniform in [1K, 32K].

Q, K, V are N(0, 1)/sqrt(d), drawn in fp32 and rounded to nearest-even
bf16 for bf16 workloads.  The per-head decay is lambda_h = fp32(exp(-s_h))
with s_h uniform in [0.001, 0.1] from one seed shared by every workload.
"""

import math

import numpy as np

DECAY_SEED = 2025
SEEDS = {"tiny": 1001, "n8k": 1002, "sweep": 1003, "n1m": 1004, "varlen64": 1004,
         "mixed": 1005, "batch8_n8k": 1006}


def rne_bf16(x):
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def decay_from_seed(num_heads, seed=DECAY_SEED, lo=0.001, hi=0.1):
    """Per-head decay lambda_h = fp32(exp(-s_h)), s_h ~ U[lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = rng.uniform(lo, hi, size=num_heads)
    return np.exp(-s).astype(np.float32)


def host_qkv(num_tokens, num_heads, head_dim, seed, dtype="bf16"):
    """Q, K, V as fp32 arrays [T, H, d]; bf16-representable when dtype='bf16'."""
    rng = np.random.Generator(np.random.PCG64(seed))
    scale = np.float32(1.0 / math.sqrt(head_dim))
    out = []
    for _ in range(3):
        x = rng.standard_normal((num_tokens, num_heads, head_dim), dtype=np.float32) * scale
        out.append(rne_bf16(x) if dtype == "bf16" else x)
    return tuple(out)


def host_int_qkv(num_tokens, num_heads, head_dim, seed, values=(-1.0, 0.0, 1.0)):
    """Q, K, V with entries drawn from a small set of integers (exact in bf16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    vals = np.asarray(values, dtype=np.float32)
    return tuple(vals[rng.integers(0, len(vals), size=(num_tokens, num_heads, head_dim))]
                 for _ in range(3))


def loguniform_lengths(n, lo, hi, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n)))
    return np.clip(x, lo, hi).astype(np.int64)


def uniform_lengths(n, lo, hi, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=n).astype(np.int64)


def cu_seqlens(lengths):
    """Packed boundaries: int32 [S+1] with cu[0] = 0 and cu[S] = sum(lengths)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] >= 2 ** 31:
        raise ValueError("total tokens exceed int32 cu_seqlens")
    return cu.astype(np.int32)


def random_states(num, num_heads, head_dim, seed, scale=1.0):
    """fp32 states [num, H, d, d] with N(0, scale^2) entries (for decode inputs)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((num, num_heads, head_dim, head_dim), dtype=np.float32)
            * np.float32(scale))


def device_qkv(num_tokens, num_heads, head_dim, seed, device, dtype="bf16",
               chunk_tokens=1 << 16):
    """Q, K, V drawn on the device with torch's seeded generator.

    Used where host generation would be too slow (1M tokens x 64 heads).
    Tokens are drawn in chunks so the fp32 temporaries stay small; the
    result is a deterministic function of (seed, shape, chunk_tokens).
    Returns three tensors [T, H, d] of torch.bfloat16 or torch.float32.
    """
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    scale = 1.0 / math.sqrt(head_dim)
    out = []
    for _ in range(3):
        t = torch.empty((num_tokens, num_heads, head_dim), dtype=tdt, device=device)
        for a in range(0, num_tokens, chunk_tokens):
            b = min(num_tokens, a + chunk_tokens)
            x = torch.randn((b - a, num_heads, head_dim), generator=gen,
                            dtype=torch.float32, device=device)
            t[a:b] = (x * scale).to(tdt)
        out.append(t)
    return tuple(out)


def device_states(num, num_heads, head_dim, seed, device, scale=1.0):
    """fp32 states [num, H, d, d] drawn on the device with torch's generator."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return torch.randn((num, num_heads, head_dim, head_dim), generator=gen,
                       dtype=torch.float32, device=device) * scale


def workload(name):
    """Shape description of a named workload (no tensors)."""
    if name == "tiny":
        return dict(name=name, lengths=[256], H=2, d=64, dtype="fp32",
                    decay=np.array([1.0, 0.9], dtype=np.float32), seed=SEEDS[name])
    if name == "n8k":
        return dict(name=name, lengths=[8192], H=64, d=128, dtype="bf16",
                    decay=decay_from_seed(64), seed=SEEDS[name])
    if name.startswith("sweep"):
        nodecay = name.endswith("_nodecay")
        n = int(name[len("sweep"):].removesuffix("_nodecay"))
        dec = np.ones(64, np.float32) if nodecay else decay_from_seed(64)
        return dict(name=name, lengths=[n], H=64, d=128, dtype="bf16", decay=dec,
                    seed=SEEDS["sweep"])
    if name == "batch8_n8k":
        # the n8k sequence shape, eight sequences in one call (512 chains)
        return dict(name=name, lengths=[8192] * 8, H=64, d=128, dtype="bf16",
                    decay=decay_from_seed(64), seed=SEEDS[name])
    if name in ("batch3_n8k", "batch5_n8k"):
        # the same shape three or five times (192 or 320 chains)
        b = int(name[5])
        return dict(name=name, lengths=[8192] * b, H=64, d=128, dtype="bf16",
                    decay=decay_from_seed(64), seed=SEEDS["batch8_n8k"] + 10 * b)
    if name == "n1m":
        return dict(name=name, lengths=[1 << 20], H=64, d=128, dtype="bf16",
                    decay=decay_from_seed(64), seed=SEEDS[name])
    if name == "varlen64":
        return dict(name=name, lengths=loguniform_lengths(64, 512, 131072, SEEDS[name]).tolist(),
                    H=64, d=128, dtype="bf16", decay=decay_from_seed(64), seed=SEEDS[name])
    if name == "mixed_prefill":
        return dict(name=name, lengths=uniform_lengths(8, 1024, 32768, SEEDS["mixed"]).tolist(),
                    H=64, d=128, dtype="bf16", decay=decay_from_seed(64), seed=SEEDS["mixed"])
    if name == "mixed_decode":
        return dict(name=name, batch=256, H=64, d=128, dtype="bf16",
                    decay=decay_from_seed(64), seed=SEEDS["mixed"] + 1,
                    state_lengths=uniform_lengths(256, 256, 2048, SEEDS["mixed"] + 2).tolist())
    raise KeyError(name)
