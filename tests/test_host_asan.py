"""libla's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

Every source is built with both sanitizers on its host code alone (each flag
follows -Xarch_host, so no GPU code is instrumented), linked into a small C
driver (tests/host_asan/driver.c) that runs each entry point's host paths --
validation, workspace sizes, long-batch dispatch order, argument packing --
with fake device addresses.  Any out-of-bounds access, use after free,
signed overflow, misaligned access or other undefined behaviour in that code
aborts the driver."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from linear_attention_la_amd import build as labuild  # noqa: E402

OUT = os.path.join(ROOT, "_build", "host_asan")
ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    flags = [f for f in labuild.FLAGS if f != "-Werror"]
    if src.endswith(".cpp"):
        cmd = [labuild.HIPCC, *[f for f in flags if not f.startswith("--offload-arch")], "-x",
               "hip", "--offload-arch=" + labuild.ARCH, *ASAN, "-c", src, "-o", obj]
    else:
        cmd = [labuild.HIPCC, *flags, *ASAN, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return obj


@pytest.mark.skipif(not os.path.exists(labuild.HIPCC), reason="hipcc not found")
def test_host_code_under_address_sanitizer():
    os.makedirs(OUT, exist_ok=True)
    srcs = [os.path.join(labuild.CSRC, s) for s in labuild.SOURCES]
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, srcs))
    exe = os.path.join(OUT, "driver")
    drv = os.path.join(ROOT, "tests", "host_asan", "driver.c")
    cmd = [labuild.HIPCC, "--offload-arch=" + labuild.ARCH, *ASAN, f"-I{labuild.INCLUDE}",
           "-x", "c", drv, "-x", "none", *objs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]  # UndefinedBehaviorSanitizer
    assert r.returncode == 0 and "OK: 0 failure(s)" in out, out[-4000:]
