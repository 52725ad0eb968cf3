"""Parity metrics between the HIP path and the fp64 oracle.

Bars (per head h):
  * relative L2:  ||X_gpu[h] - X_ref[h]||_2 / ||X_ref[h]||_2 <= rel_tol
    (1e-2 for bf16 inputs, 1e-5 for fp32 inputs);
  * elementwise:  |X_gpu - X_ref| <= 2e-2 * rms_h(X_ref), with rms taken per
    head.  When the output itself is bf16, an element over that bound is
    accepted only if it is within one bf16 ulp of the correctly rounded
    reference (the output format alone explains it); such elements are
    counted and reported.
"""

import numpy as np

from la_inputs import rne_bf16


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (fp64 array)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return np.exp2(e - 7)


def check(gpu, ref, head_axis, rel_tol, elem_tol=2e-2, out_bf16=False, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    g = np.moveaxis(gpu, head_axis, 0).reshape(gpu.shape[head_axis], -1)
    r = np.moveaxis(ref, head_axis, 0).reshape(ref.shape[head_axis], -1)
    stats = {"max_rel_l2": 0.0, "max_elem_over_rms": 0.0, "format_explained": 0}
    for h in range(g.shape[0]):
        if r.shape[1] == 0:
            continue
        nr = np.linalg.norm(r[h])
        diff = g[h] - r[h]
        if nr == 0.0:
            assert np.all(diff == 0.0), f"{what}: head {h} reference is zero but output is not"
            continue
        rel = np.linalg.norm(diff) / nr
        rms = nr / np.sqrt(r.shape[1])
        worst = float(np.max(np.abs(diff)) / rms)
        stats["max_rel_l2"] = max(stats["max_rel_l2"], float(rel))
        stats["max_elem_over_rms"] = max(stats["max_elem_over_rms"], worst)
        assert np.isfinite(rel) and rel <= rel_tol, \
            f"{what}: head {h} relative L2 {rel:.3e} > {rel_tol:.1e}"
        over = np.abs(diff) > elem_tol * rms
        if np.any(over):
            assert out_bf16, (f"{what}: head {h}: {int(over.sum())} elements over "
                              f"{elem_tol} * rms (worst {worst:.3e} * rms)")
            rounded = rne_bf16(r[h][over].astype(np.float32)).astype(np.float64)
            off = np.abs(g[h][over] - rounded)
            ok = off <= bf16_ulp(r[h][over])
            assert np.all(ok), (f"{what}: head {h}: {int((~ok).sum())} elements over "
                                f"{elem_tol} * rms not explained by bf16 output rounding")
            stats["format_explained"] += int(over.sum())
    return stats
