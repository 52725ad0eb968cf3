"""Build libla.so (gfx950 only) in-tree with hipcc.

    python -m linear_attention_la_amd.build

compiles every source under csrc/ for --offload-arch=gfx950 and links
linear_attention_la_amd/_lib/libla.so.  It always recompiles.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libla.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror", "-Wno-unused-function",
    # only the C ABI is exported (la_host.cpp gives the declarations of la.h
    # default visibility)
    "-fvisibility=hidden",
    # packed fp32 VALU ops stay off (v_pk_{add,mul,fma}_f32 are not emitted)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SOURCES = ["la_host.cpp", "la_prefill_bf16.hip", "la_prefill_wide.hip", "la_prefill_f32.hip",
           "la_decode.hip", "la_segment.hip", "la_state.hip"]
# A separate library with the MFMA-only loop that the benchmark uses to
# measure the GPU's matrix-core peak (not part of la.h, not linked into
# libla.so).
PEAK_SOURCE = os.path.join("probe", "la_peak.hip")
PEAK_LIB = os.path.join(OUT_DIR, "libla_peak.so")


def _compile(src):
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *[f for f in FLAGS if not f.startswith("--offload-arch")], "-x", "hip",
               "--offload-arch=" + ARCH, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj, errs


def _link(objs, lib):
    tmp = lib + ".tmp"
    # --no-undefined: a kernel whose host stub was not emitted (clang can drop
    # it without a diagnostic) fails here instead of at load time.
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + \
        list(objs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_compile, SOURCES + [PEAK_SOURCE]))
    for obj, msgs in results:
        if msgs.strip() and verbose:
            print(msgs, file=sys.stderr)
    _link([o for o, _ in results[:len(SOURCES)]], LIB)
    _link([results[-1][0]], PEAK_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
