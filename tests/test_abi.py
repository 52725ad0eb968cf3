"""C ABI checks that need no GPU: the library loads, exports every entry point
the public header declares, and rejects bad arguments on the host (before
any HIP call) with the documented status codes."""

import ctypes
import os
import re

import numpy as np
import pytest

import linear_attention_la_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            src = open(os.path.join(inc, fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(la_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_entry_points():
    names = _declared_functions()
    for n in ("la_prefill", "la_prefill_segmented", "la_prefill_segmented_workspace_size",
              "la_prefill_segmented_noalloc", "la_prefill_normed",
              "la_prefill_normed_workspace_size", "la_decode_normed",
              "la_prefill_backward", "la_prefill_backward_workspace_size",
              "la_prefill_backward_segmented", "la_prefill_backward_segmented_workspace_size",
              "la_prefill_pool", "la_prefill_kernel_plan", "la_decode", "la_decode_pool",
              "la_status_str", "la_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = la.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), f"libla.so does not export {name}"


def test_library_exports_only_the_c_abi():
    """Every exported la_* symbol is declared in the header, and no internal
    helper (kernel launchers, host checks) is exported."""
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", la.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert {n for n in names if n.startswith("la_")} == set(_declared_functions())
    assert not [n for n in names if "launch_" in n or "segmented_chain" in n or "check_" in n]


def test_peak_probe_library_is_separate():
    """The benchmark's MFMA-loop probe is its own library: it exports only its
    entry points (the bf16 and fp32 loops), and libla.so contains neither."""
    import subprocess

    path = os.path.join(os.path.dirname(la.lib_path()), "libla_peak.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert {n for n in names if n.startswith("la_")} == {"la_peak_mfma_bf16", "la_peak_mfma_f32"}
    assert not hasattr(la.lib(), "la_peak_mfma_bf16")
    assert not hasattr(la.lib(), "la_peak_mfma_f32")


def test_status_strings():
    assert la.la_status_str(la.LA_OK) == "LA_OK"
    assert la.la_status_str(la.LA_ERR_INVALID_ARG) == "LA_ERR_INVALID_ARG"
    assert la.la_status_str(la.LA_ERR_UNSUPPORTED) == "LA_ERR_UNSUPPORTED"
    assert la.la_status_str(la.LA_ERR_HIP) == "LA_ERR_HIP"
    assert la.la_status_str(77) == "LA_STATUS_UNKNOWN"


# Fake, never-dereferenced device addresses: validation runs on the host only
# and must reject every case below before touching them.
Q, K, V, O, KVF, KVI, CUD = (0x10000000 * (i + 1) for i in range(7))
T, H, D = 100, 4, 128
BIG = T * H * D * 4  # bytes of one fp32 [T,H,d] tensor


def _prefill(**kw):
    args = dict(q=Q, k=K, v=V, cu_dev=CUD, cu_host=np.array([0, 40, 100], np.int32), S=2, T=T,
                H=H, d=D, in_dt=la.LA_BF16, out_dt=la.LA_BF16,
                decay=np.full(H, 0.9, np.float32), kv_init=None, o=O, kv_final=KVF)
    args.update(kw)
    cu = args["cu_host"]
    dec = args["decay"]
    st = la.la_prefill(args["q"], args["k"], args["v"], args["cu_dev"],
                       None if cu is None else cu.ctypes.data, args["S"], args["T"], args["H"],
                       args["d"], args["in_dt"], args["out_dt"],
                       None if dec is None else dec.ctypes.data, args["kv_init"], args["o"],
                       args["kv_final"], None)
    return st, la.la_last_error()


BAD_PREFILL = [
    ("negative_seqs", dict(S=-1), la.LA_ERR_INVALID_ARG),
    ("negative_tokens", dict(T=-5), la.LA_ERR_INVALID_ARG),
    ("tokens_over_int32", dict(T=1 << 31), la.LA_ERR_INVALID_ARG),
    ("zero_heads", dict(H=0), la.LA_ERR_INVALID_ARG),
    ("too_many_heads", dict(H=257, decay=np.full(257, 0.9, np.float32)), la.LA_ERR_UNSUPPORTED),
    ("head_dim_96", dict(d=96), la.LA_ERR_UNSUPPORTED),
    ("head_dim_zero", dict(d=0), la.LA_ERR_INVALID_ARG),
    ("bad_in_dtype", dict(in_dt=7), la.LA_ERR_INVALID_ARG),
    ("bad_out_dtype", dict(out_dt=-1), la.LA_ERR_INVALID_ARG),
    ("fp32_in_bf16_out", dict(in_dt=la.LA_FP32, out_dt=la.LA_BF16), la.LA_ERR_UNSUPPORTED),
    ("decay_null", dict(decay=None), la.LA_ERR_INVALID_ARG),
    ("decay_zero", dict(decay=np.array([0.9, 0.0, 0.9, 0.9], np.float32)), la.LA_ERR_INVALID_ARG),
    ("decay_above_one", dict(decay=np.array([0.9, 1.0001, 0.9, 0.9], np.float32)),
     la.LA_ERR_INVALID_ARG),
    ("decay_nan", dict(decay=np.array([0.9, np.nan, 0.9, 0.9], np.float32)), la.LA_ERR_INVALID_ARG),
    ("decay_negative", dict(decay=np.array([-0.5, 0.9, 0.9, 0.9], np.float32)),
     la.LA_ERR_INVALID_ARG),
    ("cu_host_null", dict(cu_host=None), la.LA_ERR_INVALID_ARG),
    ("cu_first_nonzero", dict(cu_host=np.array([1, 40, 100], np.int32)), la.LA_ERR_INVALID_ARG),
    ("cu_decreasing", dict(cu_host=np.array([0, 60, 50], np.int32), T=50), la.LA_ERR_INVALID_ARG),
    ("cu_last_mismatch", dict(cu_host=np.array([0, 40, 99], np.int32)), la.LA_ERR_INVALID_ARG),
    ("cu_dev_null", dict(cu_dev=None), la.LA_ERR_INVALID_ARG),
    ("q_null", dict(q=None), la.LA_ERR_INVALID_ARG),
    ("o_null", dict(o=None), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_q", dict(o=Q + 64), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_v", dict(o=V - 64), la.LA_ERR_INVALID_ARG),
    ("kv_final_overlaps_k", dict(kv_final=K + 2), la.LA_ERR_INVALID_ARG),
    ("kv_final_overlaps_o", dict(kv_final=O + 2), la.LA_ERR_INVALID_ARG),
    ("kv_final_overlaps_kv_init_partially", dict(kv_init=KVI, kv_final=KVI + 4),
     la.LA_ERR_INVALID_ARG),
    ("o_overlaps_kv_init", dict(kv_init=KVI, o=KVI + 16), la.LA_ERR_INVALID_ARG),
    ("q_misaligned", dict(q=Q + 2), la.LA_ERR_INVALID_ARG),
    ("o_misaligned", dict(o=O + 8), la.LA_ERR_INVALID_ARG),
    ("kv_final_misaligned", dict(kv_final=KVF + 4), la.LA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", BAD_PREFILL, ids=[b[0] for b in BAD_PREFILL])
def test_prefill_rejects(name, kw, code):
    st, msg = _prefill(**kw)
    assert st == code, (st, msg)
    assert msg, "la_last_error must describe the failure"


def test_prefill_zero_sequences_is_noop():
    st, msg = _prefill(S=0, T=0, cu_host=np.array([0], np.int32), q=None, k=None, v=None, o=None,
                       kv_final=None, cu_dev=None)
    assert st == la.LA_OK, msg
    assert msg == ""


def _decode(**kw):
    args = dict(q=Q, k=K, v=V, kv=KVF, decay=np.full(H, 0.9, np.float32), B=3, H=H, d=D,
                dt=la.LA_BF16, o=O)
    args.update(kw)
    dec = args["decay"]
    st = la.la_decode(args["q"], args["k"], args["v"], args["kv"],
                      None if dec is None else dec.ctypes.data, args["B"], args["H"], args["d"],
                      args["dt"], args["o"], None)
    return st, la.la_last_error()


BAD_DECODE = [
    ("negative_batch", dict(B=-1), la.LA_ERR_INVALID_ARG),
    ("zero_heads", dict(H=0), la.LA_ERR_INVALID_ARG),
    ("head_dim_32", dict(d=32), la.LA_ERR_UNSUPPORTED),
    ("bad_dtype", dict(dt=3), la.LA_ERR_INVALID_ARG),
    ("decay_null", dict(decay=None), la.LA_ERR_INVALID_ARG),
    ("decay_zero", dict(decay=np.array([0.9, 0.9, 0.0, 0.9], np.float32)), la.LA_ERR_INVALID_ARG),
    ("kv_null", dict(kv=None), la.LA_ERR_INVALID_ARG),
    ("o_null", dict(o=None), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_kv", dict(o=KVF + 8), la.LA_ERR_INVALID_ARG),
    ("kv_overlaps_q", dict(kv=Q - 16), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_k", dict(o=K + 2), la.LA_ERR_INVALID_ARG),
    ("kv_misaligned", dict(kv=KVF + 8), la.LA_ERR_INVALID_ARG),
    ("v_misaligned", dict(v=V + 2), la.LA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", BAD_DECODE, ids=[b[0] for b in BAD_DECODE])
def test_decode_rejects(name, kw, code):
    st, msg = _decode(**kw)
    assert st == code, (st, msg)
    assert msg


def test_decode_zero_batch_is_noop():
    st, msg = _decode(B=0, q=None, k=None, v=None, kv=None, o=None)
    assert st == la.LA_OK, msg


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """No CPU fallback: a missing library is an error, not a silent path."""
    from linear_attention_la_amd import _binding

    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setenv("LA_LIB", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not found"):
        _binding.lib()
    monkeypatch.setattr(_binding, "_lib", None)


# ---- segmented prefill (host-side checks only) ----

def _ws_size(cu, H=4, d=128, seg=64):
    cu = np.asarray(cu, np.int32)
    return la.la_prefill_segmented_workspace_size(cu.shape[0] - 1, cu.ctypes.data, H, d, seg)


def test_segmented_workspace_size_layout():
    """8 segments (lengths 100, 0, 300 at 64 tokens each: 2 + 1 + 5): 4
    sections of int32 and the control words (2 + 2 S H) padded to 256 B,
    then fp32 states: d = 128 runs the chained scan, whose exchange ring holds
    2 states per (sequence, head) (2 x 3 x 4 of 128^2); d = 64 runs the
    four-kernel path with (8 + 3) states per head."""
    st, n = _ws_size([0, 100, 100, 400])
    assert st == la.LA_OK
    assert n == 5 * 256 + 2 * 3 * 4 * 128 * 128 * 4
    st, n = _ws_size([0, 100, 100, 400], d=64)
    assert st == la.LA_OK
    assert n == 5 * 256 + 11 * 4 * 64 * 64 * 4
    st, n = _ws_size([0, 64], seg=64)       # exactly one segment
    assert st == la.LA_OK and n == 5 * 256 + 2 * 4 * 128 * 128 * 4
    st, n = _ws_size([0], seg=64)           # no sequences: the empty slot sections take no space
    assert st == la.LA_OK and n == 3 * 256
    # 64 sequences of one segment x 64 heads: cu_seg and seq_first (65 words)
    # take 512 B each, the slot maps 256 B, 8194 control words 33,024 B
    cu = np.arange(0, 65 * 64, 64, dtype=np.int32)
    st, n = _ws_size(cu, H=64, seg=64)
    assert st == la.LA_OK
    assert n == 2 * 512 + 2 * 256 + 33024 + 2 * 64 * 64 * 128 * 128 * 4


def test_segmented_auto_segment_len():
    """segment_len 0 lets the library pick about one (segment, head) item per
    compute unit (256 without a device), in multiples of 64 tokens: 1M
    tokens x 8 heads -> 32768, 8192 x 64 -> 2048, 100 x 4 -> 64."""
    for cu, H, seg in (([0, 1 << 20], 8, 32768), ([0, 8192], 64, 2048), ([0, 100], 4, 64),
                       ([0, 5000, 5000, 9000], 16, 576)):
        for d in (64, 128):
            assert _ws_size(cu, H=H, d=d, seg=0) == _ws_size(cu, H=H, d=d, seg=seg)
            c = np.asarray(cu, np.int32)
            assert la.la_prefill_backward_segmented_workspace_size(c.shape[0] - 1, c.ctypes.data,
                                                                   H, d, 0) == \
                la.la_prefill_backward_segmented_workspace_size(c.shape[0] - 1, c.ctypes.data,
                                                                H, d, seg)


@pytest.mark.parametrize("seg", [-64, 100, 63, -1])
def test_segmented_workspace_size_rejects_segment_len(seg):
    st, n = _ws_size([0, 100], seg=seg)
    assert st == la.LA_ERR_INVALID_ARG and n == 0
    assert la.la_last_error()


def test_segmented_workspace_size_rejects_bad_cu():
    assert _ws_size([1, 100])[0] == la.LA_ERR_INVALID_ARG
    assert _ws_size([0, 100, 50])[0] == la.LA_ERR_INVALID_ARG
    assert _ws_size([0, 100], d=96)[0] == la.LA_ERR_UNSUPPORTED


WS = 0x90000000


def _seg(**kw):
    args = dict(q=Q, k=K, v=V, cu_dev=CUD, cu_host=np.array([0, 40, 100], np.int32), S=2, T=T,
                H=H, d=D, in_dt=la.LA_BF16, out_dt=la.LA_BF16,
                decay=np.full(H, 0.9, np.float32), kv_init=None, o=O, kv_final=KVF, seg=64,
                ws=WS, ws_bytes=1 << 30)
    args.update(kw)
    cu = args["cu_host"]
    st = la.la_prefill_segmented(args["q"], args["k"], args["v"], args["cu_dev"],
                                 None if cu is None else cu.ctypes.data, args["S"], args["T"],
                                 args["H"], args["d"], args["in_dt"], args["out_dt"],
                                 args["decay"].ctypes.data, args["kv_init"], args["o"],
                                 args["kv_final"], args["seg"], args["ws"], args["ws_bytes"], None)
    return st, la.la_last_error()


BAD_SEGMENTED = [
    ("segment_len_negative", dict(seg=-64), la.LA_ERR_INVALID_ARG),
    ("segment_len_not_multiple", dict(seg=96), la.LA_ERR_INVALID_ARG),
    ("fp32_input", dict(in_dt=la.LA_FP32, out_dt=la.LA_FP32), la.LA_ERR_UNSUPPORTED),
    ("workspace_null", dict(ws=None), la.LA_ERR_INVALID_ARG),
    ("workspace_misaligned", dict(ws=WS + 8), la.LA_ERR_INVALID_ARG),
    ("workspace_too_small", dict(ws_bytes=4096), la.LA_ERR_INVALID_ARG),
    ("workspace_overlaps_q", dict(ws=Q + 256), la.LA_ERR_INVALID_ARG),
    ("workspace_overlaps_kv_final", dict(ws=KVF - 4096), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_k", dict(o=K + 64), la.LA_ERR_INVALID_ARG),
    ("cu_last_mismatch", dict(cu_host=np.array([0, 40, 99], np.int32)), la.LA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", BAD_SEGMENTED, ids=[b[0] for b in BAD_SEGMENTED])
def test_segmented_rejects(name, kw, code):
    st, msg = _seg(**kw)
    assert st == code, (st, msg)
    assert msg


# ---- segmented prefill without allocation (host-side checks only) ----

def _seg_noalloc(**kw):
    args = dict(q=Q, k=K, v=V, cu_dev=CUD, cu_host=np.array([0, 40, 100], np.int32), S=2, T=T,
                H=H, d=D, in_dt=la.LA_BF16, out_dt=la.LA_BF16,
                decay=np.full(H, 0.9, np.float32), kv_init=None, o=O, kv_final=KVF, seg=64)
    args.update(kw)
    cu = args["cu_host"]
    st = la.la_prefill_segmented_noalloc(args["q"], args["k"], args["v"], args["cu_dev"],
                                         None if cu is None else cu.ctypes.data, args["S"],
                                         args["T"], args["H"], args["d"], args["in_dt"],
                                         args["out_dt"], args["decay"].ctypes.data,
                                         args["kv_init"], args["o"], args["kv_final"],
                                         args["seg"], None)
    return st, la.la_last_error()


BAD_SEGMENTED_NOALLOC = [b for b in BAD_SEGMENTED if not b[0].startswith("workspace")] + [
    # d = 128 (the chained scan): 9 sequences x 64 heads need 2 exchange
    # states per (sequence, head), 72 MiB, above the 64 MiB scratch
    ("scratch_too_small", dict(H=64, decay=np.full(64, 0.9, np.float32), T=9, S=9,
                               cu_host=np.arange(10, dtype=np.int32)), la.LA_ERR_UNSUPPORTED),
    # d = 64 (four-kernel path): 16,384 tokens in segments of 64 need
    # (256 + 1) x 64 states of 16 KiB, 257 MiB
    ("scratch_too_small_d64", dict(H=64, d=64, decay=np.full(64, 0.9, np.float32), T=16384,
                                   S=1, cu_host=np.array([0, 16384], np.int32)),
     la.LA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,kw,code", BAD_SEGMENTED_NOALLOC,
                         ids=[b[0] for b in BAD_SEGMENTED_NOALLOC])
def test_segmented_noalloc_rejects(name, kw, code):
    st, msg = _seg_noalloc(**kw)
    assert st == code, (st, msg)
    assert msg
    if name.startswith("scratch_too_small"):
        assert "scratch" in msg


def test_segmented_noalloc_no_sequences():
    st, _ = _seg_noalloc(S=0, T=0, cu_host=np.array([0], np.int32))
    assert st == la.LA_OK


# ---- output normalisation (host-side checks only) ----

NW, GT = 0xB0000000, 0xC0000000


def _prefill_normed(norm="default", **kw):
    args = dict(q=Q, k=K, v=V, cu_dev=CUD, cu_host=np.array([0, 40, 100], np.int32), S=2, T=T,
                H=H, d=D, in_dt=la.LA_BF16, out_dt=la.LA_BF16,
                decay=np.full(H, 0.9, np.float32), kv_init=None, o=O, kv_final=KVF, ws=WS,
                ws_bytes=1 << 30)
    args.update(kw)
    nm = la.LaNorm(NW, 1e-6, GT) if norm == "default" else norm
    cu = args["cu_host"]
    st = la.la_prefill_normed(args["q"], args["k"], args["v"], args["cu_dev"], cu.ctypes.data,
                              args["S"], args["T"], args["H"], args["d"], args["in_dt"],
                              args["out_dt"], args["decay"].ctypes.data, args["kv_init"], nm,
                              args["o"], args["kv_final"], args["ws"], args["ws_bytes"], None)
    return st, la.la_last_error()


BAD_NORMED = [
    ("norm_null", dict(norm=None), la.LA_ERR_INVALID_ARG),
    ("weight_null", dict(norm=la.LaNorm(None, 1e-6, GT)), la.LA_ERR_INVALID_ARG),
    ("eps_zero", dict(norm=la.LaNorm(NW, 0.0, None)), la.LA_ERR_INVALID_ARG),
    ("eps_negative", dict(norm=la.LaNorm(NW, -1.0, None)), la.LA_ERR_INVALID_ARG),
    ("eps_nan", dict(norm=la.LaNorm(NW, float("nan"), None)), la.LA_ERR_INVALID_ARG),
    ("eps_inf", dict(norm=la.LaNorm(NW, float("inf"), None)), la.LA_ERR_INVALID_ARG),
    ("weight_misaligned", dict(norm=la.LaNorm(NW + 4, 1e-6, None)), la.LA_ERR_INVALID_ARG),
    ("gate_misaligned", dict(norm=la.LaNorm(NW, 1e-6, GT + 8)), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_gate", dict(o=GT + 256), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_weight", dict(o=NW - 256), la.LA_ERR_INVALID_ARG),
    ("fp32_input", dict(in_dt=la.LA_FP32, out_dt=la.LA_FP32), la.LA_ERR_UNSUPPORTED),
    ("head_dim_64", dict(d=64), la.LA_ERR_UNSUPPORTED),
    ("workspace_null", dict(ws=None), la.LA_ERR_INVALID_ARG),
    ("workspace_short", dict(ws_bytes=256), la.LA_ERR_INVALID_ARG),
    ("workspace_overlaps_gate", dict(ws=GT - 4096), la.LA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", BAD_NORMED, ids=[b[0] for b in BAD_NORMED])
def test_prefill_normed_rejects(name, kw, code):
    st, msg = _prefill_normed(**kw)
    assert st == code, (st, msg)
    assert msg


def test_prefill_normed_workspace_size():
    """Without a GPU the compute-unit count is taken as 256: 2 sequences x 4
    heads use the chained scan, whose ring holds 2 states per pair; 64
    sequences x 4 heads (256 pairs) need no workspace."""
    cu = np.array([0, 40, 100], np.int32)
    st, n = la.la_prefill_normed_workspace_size(2, cu.ctypes.data, 4, 128)
    assert st == la.LA_OK and n >= 2 * 2 * 4 * 128 * 128 * 4
    cu64 = np.arange(0, 65 * 10, 10, dtype=np.int32)
    st, n = la.la_prefill_normed_workspace_size(64, cu64.ctypes.data, 4, 128)
    assert st == la.LA_OK and n == 0
    assert la.la_prefill_normed_workspace_size(2, cu.ctypes.data, 4, 64)[0] == la.LA_ERR_UNSUPPORTED
    assert la.la_prefill_normed_workspace_size(2, None, 4, 128)[0] == la.LA_ERR_INVALID_ARG


def _decode_normed(norm="default", **kw):
    args = dict(q=Q, k=K, v=V, kv=KVF, decay=np.full(H, 0.9, np.float32), B=3, H=H, d=D,
                dt=la.LA_BF16, o=O)
    args.update(kw)
    nm = la.LaNorm(NW, 1e-6, GT) if norm == "default" else norm
    st = la.la_decode_normed(args["q"], args["k"], args["v"], args["kv"],
                             args["decay"].ctypes.data, args["B"], args["H"], args["d"],
                             args["dt"], nm, args["o"], None)
    return st, la.la_last_error()


BAD_DECODE_NORMED = [
    ("norm_null", dict(norm=None), la.LA_ERR_INVALID_ARG),
    ("eps_zero", dict(norm=la.LaNorm(NW, 0.0, None)), la.LA_ERR_INVALID_ARG),
    ("gate_misaligned", dict(norm=la.LaNorm(NW, 1e-6, GT + 2)), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_gate", dict(o=GT), la.LA_ERR_INVALID_ARG),
    ("kv_overlaps_weight", dict(kv=NW - 64), la.LA_ERR_INVALID_ARG),
    ("negative_batch", dict(B=-1), la.LA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", BAD_DECODE_NORMED, ids=[b[0] for b in BAD_DECODE_NORMED])
def test_decode_normed_rejects(name, kw, code):
    st, msg = _decode_normed(**kw)
    assert st == code, (st, msg)
    assert msg


# ---- decode on a state pool (host-side checks only) ----

POOL = 0xA0000000


def _pool(**kw):
    args = dict(q=Q, k=K, v=V, pool=POOL, P=10, slots=np.array([3, 0, 7], np.int32),
                slots_dev=CUD, decay=np.full(H, 0.9, np.float32), B=3, H=H, d=D,
                dt=la.LA_BF16, o=O)
    args.update(kw)
    sl = args["slots"]
    st = la.la_decode_pool(args["q"], args["k"], args["v"], args["pool"], args["P"],
                           args["slots_dev"], None if sl is None else sl.ctypes.data,
                           args["decay"].ctypes.data, args["B"], args["H"], args["d"], args["dt"],
                           args["o"], None)
    return st, la.la_last_error()


BAD_POOL = [
    ("slot_out_of_range", dict(slots=np.array([3, 0, 10], np.int32)), la.LA_ERR_INVALID_ARG),
    ("slot_negative", dict(slots=np.array([3, -1, 7], np.int32)), la.LA_ERR_INVALID_ARG),
    ("slot_repeated", dict(slots=np.array([3, 0, 3], np.int32)), la.LA_ERR_INVALID_ARG),
    ("slots_host_null", dict(slots=None), la.LA_ERR_INVALID_ARG),
    ("slots_dev_null", dict(slots_dev=None), la.LA_ERR_INVALID_ARG),
    ("pool_size_negative", dict(P=-1), la.LA_ERR_INVALID_ARG),
    ("pool_empty", dict(P=0), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_pool", dict(o=POOL + 10 * 4 * 128 * 128 * 4 - 64), la.LA_ERR_INVALID_ARG),
    ("pool_overlaps_q", dict(pool=Q - 64), la.LA_ERR_INVALID_ARG),
    ("head_dim_32", dict(d=32), la.LA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,kw,code", BAD_POOL, ids=[b[0] for b in BAD_POOL])
def test_decode_pool_rejects(name, kw, code):
    st, msg = _pool(**kw)
    assert st == code, (st, msg)
    assert msg


def test_pool_slot_checks_scale_with_the_slots():
    # A repeated slot in a pool of 2^31 - 1 states is found by sorting the
    # slots, not by a table of the pool's size (that would take 2 GiB).
    big = 2**31 - 1
    st, msg = _pool(P=big, slots=np.array([5, big - 1, 5], np.int32))
    assert st == la.LA_ERR_INVALID_ARG and "slot 5 is used twice" in msg, msg
    st, msg = _prefill_pool(P=big, slots=np.array([big - 1, big - 1], np.int32))
    assert st == la.LA_ERR_INVALID_ARG and "used twice" in msg, msg
    st, msg = _pool(slots=np.array([3, 9, 10], np.int32))
    assert st == la.LA_ERR_INVALID_ARG and "slots[2] = 10" in msg, msg


def test_decode_pool_zero_batch_is_noop():
    st, msg = _pool(B=0, slots=None, slots_dev=None, q=None, k=None, v=None, o=None)
    assert st == la.LA_OK, msg


def _prefill_pool(**kw):
    args = dict(q=Q, k=K, v=V, cu_dev=CUD, cu_host=np.array([0, 40, 100], np.int32), S=2, T=T,
                H=H, d=D, in_dt=la.LA_BF16, out_dt=la.LA_BF16,
                decay=np.full(H, 0.9, np.float32), pool=POOL, P=10,
                slots=np.array([7, 2], np.int32), slots_dev=KVI, o=O)
    args.update(kw)
    cu, sl, dec = args["cu_host"], args["slots"], args["decay"]
    st = la.la_prefill_pool(args["q"], args["k"], args["v"], args["cu_dev"],
                            None if cu is None else cu.ctypes.data, args["S"], args["T"],
                            args["H"], args["d"], args["in_dt"], args["out_dt"],
                            None if dec is None else dec.ctypes.data, args["pool"], args["P"],
                            args["slots_dev"], None if sl is None else sl.ctypes.data, args["o"],
                            None)
    return st, la.la_last_error()


BAD_PREFILL_POOL = [
    ("slot_out_of_range", dict(slots=np.array([7, 10], np.int32)), la.LA_ERR_INVALID_ARG),
    ("slot_negative", dict(slots=np.array([-1, 2], np.int32)), la.LA_ERR_INVALID_ARG),
    ("slot_repeated", dict(slots=np.array([2, 2], np.int32)), la.LA_ERR_INVALID_ARG),
    ("slots_host_null", dict(slots=None), la.LA_ERR_INVALID_ARG),
    ("slots_dev_null", dict(slots_dev=None), la.LA_ERR_INVALID_ARG),
    ("pool_null", dict(pool=None), la.LA_ERR_INVALID_ARG),
    ("pool_misaligned", dict(pool=POOL + 4), la.LA_ERR_INVALID_ARG),
    ("pool_size_negative", dict(P=-1), la.LA_ERR_INVALID_ARG),
    ("pool_empty", dict(P=0), la.LA_ERR_INVALID_ARG),
    ("o_overlaps_pool", dict(o=POOL + 10 * 4 * 128 * 128 * 4 - 64), la.LA_ERR_INVALID_ARG),
    ("pool_overlaps_k", dict(pool=K - 64), la.LA_ERR_INVALID_ARG),
    ("fp32_inputs", dict(in_dt=la.LA_FP32, out_dt=la.LA_FP32), la.LA_ERR_UNSUPPORTED),
    ("decay_null", dict(decay=None), la.LA_ERR_INVALID_ARG),
    ("cu_last_mismatch", dict(cu_host=np.array([0, 40, 99], np.int32)), la.LA_ERR_INVALID_ARG),
    ("head_dim_96", dict(d=96), la.LA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,kw,code", BAD_PREFILL_POOL, ids=[b[0] for b in BAD_PREFILL_POOL])
def test_prefill_pool_rejects(name, kw, code):
    st, msg = _prefill_pool(**kw)
    assert st == code, (st, msg)
    assert msg


def test_prefill_pool_zero_sequences_is_noop():
    st, msg = _prefill_pool(S=0, T=0, cu_host=np.array([0], np.int32), slots=None,
                            slots_dev=None, q=None, k=None, v=None, o=None, pool=None)
    assert st == la.LA_OK, msg


# LA_NDV: the sweep override of the kernel choice (1 or d/32 workgroups per
# chain).  Only rejected values are tried here: an accepted one would launch.
BAD_NDV = [("2", 128), ("8", 128), ("0", 128), ("1", 64), ("4", 64), ("four", 128),
           ("4 ", 128), ("-4", 128)]


@pytest.mark.parametrize("value,d", BAD_NDV, ids=[f"{v!r}-d{d}" for v, d in BAD_NDV])
def test_ndv_override_rejects(monkeypatch, value, d):
    monkeypatch.setenv("LA_NDV", value)
    st, msg = _prefill(d=d)
    assert st == la.LA_ERR_UNSUPPORTED and "LA_NDV" in msg, (st, msg)
    st, msg = _prefill_pool(d=d)
    assert st == la.LA_ERR_UNSUPPORTED and "LA_NDV" in msg, (st, msg)


def test_ndv_override_checked_after_arguments(monkeypatch):
    """An argument error is still reported as such with LA_NDV set."""
    monkeypatch.setenv("LA_NDV", "2")
    st, msg = _prefill(decay=None)
    assert st == la.LA_ERR_INVALID_ARG, (st, msg)


# ---- backward (host-side checks only) ----

DO_, DQ, DK, DV, DKV0, BWS = (0xB0000000 + 0x10000000 * i for i in range(6))


def _bwd(**kw):
    args = dict(q=Q, k=K, v=V, do=DO_, cu_dev=CUD, cu_host=np.array([0, 40, 100], np.int32), S=2,
                T=T, H=H, d=D, in_dt=la.LA_BF16, g_dt=la.LA_BF16,
                decay=np.full(H, 0.9, np.float32), kv_init=KVI, dkv_final=KVF, dq=DQ, dk=DK,
                dv=DV, dkv_init=DKV0, ws=BWS, ws_bytes=1 << 30)
    args.update(kw)
    cu = args["cu_host"]
    st = la.la_prefill_backward(args["q"], args["k"], args["v"], args["do"], args["cu_dev"],
                                None if cu is None else cu.ctypes.data, args["S"], args["T"],
                                args["H"], args["d"], args["in_dt"], args["g_dt"],
                                args["decay"].ctypes.data, args["kv_init"], args["dkv_final"],
                                args["dq"], args["dk"], args["dv"], args["dkv_init"], args["ws"],
                                args["ws_bytes"], None)
    return st, la.la_last_error()


def test_backward_workspace_size():
    st, n = la.la_prefill_backward_workspace_size(2, 4, 128)
    assert st == la.LA_OK and n == 2 * 4 * 128 * 128 * 4
    assert la.la_prefill_backward_workspace_size(-1, 4, 128)[0] == la.LA_ERR_INVALID_ARG
    assert la.la_prefill_backward_workspace_size(1, 4, 96)[0] == la.LA_ERR_UNSUPPORTED


BAD_BACKWARD = [
    ("fp32_inputs", dict(in_dt=la.LA_FP32), la.LA_ERR_UNSUPPORTED),
    ("bad_grad_dtype", dict(g_dt=5), la.LA_ERR_INVALID_ARG),
    ("tiny_decay_with_final_grad", dict(decay=np.array([0.9, 1e-30, 0.9, 0.9], np.float32)),
     la.LA_ERR_UNSUPPORTED),
    ("d_o_null", dict(do=None), la.LA_ERR_INVALID_ARG),
    ("dk_null", dict(dk=None), la.LA_ERR_INVALID_ARG),
    ("workspace_null", dict(ws=None), la.LA_ERR_INVALID_ARG),
    ("workspace_short", dict(ws_bytes=1024), la.LA_ERR_INVALID_ARG),
    ("dq_overlaps_d_o", dict(dq=DO_ + 64), la.LA_ERR_INVALID_ARG),
    ("dk_overlaps_dv", dict(dk=DV - 64), la.LA_ERR_INVALID_ARG),
    ("dkv_init_overlaps_workspace", dict(dkv_init=BWS + 64), la.LA_ERR_INVALID_ARG),
    ("dkv_init_overlaps_dkv_final", dict(dkv_init=KVF), la.LA_ERR_INVALID_ARG),
    ("dv_misaligned", dict(dv=DV + 4), la.LA_ERR_INVALID_ARG),
    ("cu_decreasing", dict(cu_host=np.array([0, 60, 50], np.int32), T=50), la.LA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", BAD_BACKWARD, ids=[b[0] for b in BAD_BACKWARD])
def test_backward_rejects(name, kw, code):
    st, msg = _bwd(**kw)
    assert st == code, (st, msg)
    assert msg


def test_backward_no_states_needs_no_workspace():
    """Without kv_init and dkv_final the workspace may be NULL (host check
    passes; nothing is launched because there are no sequences)."""
    st, msg = _bwd(S=0, T=0, cu_host=np.array([0], np.int32), kv_init=None, dkv_final=None,
                   ws=None, ws_bytes=0)
    assert st == la.LA_OK, msg


# ---- segmented backward (host-side checks only) ----

def _bwd_seg(seg=64, **kw):
    args = dict(q=Q, k=K, v=V, do=DO_, cu_dev=CUD, cu_host=np.array([0, 40, 100], np.int32), S=2,
                T=T, H=H, d=D, in_dt=la.LA_BF16, g_dt=la.LA_BF16,
                decay=np.full(H, 0.9, np.float32), kv_init=KVI, dkv_final=KVF, dq=DQ, dk=DK,
                dv=DV, dkv_init=DKV0, ws=BWS, ws_bytes=1 << 26)
    args.update(kw)
    cu = args["cu_host"]
    st = la.la_prefill_backward_segmented(
        args["q"], args["k"], args["v"], args["do"], args["cu_dev"],
        None if cu is None else cu.ctypes.data, args["S"], args["T"], args["H"], args["d"],
        args["in_dt"], args["g_dt"], args["decay"].ctypes.data, args["kv_init"],
        args["dkv_final"], args["dq"], args["dk"], args["dv"], args["dkv_init"], seg, args["ws"],
        args["ws_bytes"], None)
    return st, la.la_last_error()


def test_backward_segmented_workspace_size():
    """The segmented forward's layout plus one set of S x H x d x d states
    (256-byte aligned after it)."""
    cu = np.array([0, 40, 100, 100], np.int32)
    st, fwd = la.la_prefill_segmented_workspace_size(3, cu.ctypes.data, 4, 128, 64)
    assert st == la.LA_OK
    st, n = la.la_prefill_backward_segmented_workspace_size(3, cu.ctypes.data, 4, 128, 64)
    assert st == la.LA_OK
    assert n == ((fwd + 255) // 256) * 256 + 3 * 4 * 128 * 128 * 4
    assert la.la_prefill_backward_segmented_workspace_size(3, cu.ctypes.data, 4, 128, 100)[0] == \
        la.LA_ERR_INVALID_ARG
    assert la.la_prefill_backward_segmented_workspace_size(3, None, 4, 128, 64)[0] == \
        la.LA_ERR_INVALID_ARG
    assert la.prefill_backward_segmented_workspace_size(cu, 4, 128, 64) == n


BAD_BACKWARD_SEGMENTED = [
    ("segment_len_not_multiple", dict(seg=96), la.LA_ERR_INVALID_ARG),
    ("segment_len_negative", dict(seg=-128), la.LA_ERR_INVALID_ARG),
    ("fp32_inputs", dict(in_dt=la.LA_FP32), la.LA_ERR_UNSUPPORTED),
    ("tiny_decay_with_final_grad", dict(decay=np.array([0.9, 1e-30, 0.9, 0.9], np.float32)),
     la.LA_ERR_UNSUPPORTED),
    ("workspace_null_without_states", dict(ws=None, kv_init=None, dkv_final=None),
     la.LA_ERR_INVALID_ARG),
    ("workspace_short", dict(ws_bytes=4096), la.LA_ERR_INVALID_ARG),
    ("workspace_misaligned", dict(ws=BWS + 8), la.LA_ERR_INVALID_ARG),
    ("workspace_overlaps_dk", dict(ws=DK - 4096), la.LA_ERR_INVALID_ARG),
    ("dq_overlaps_q", dict(dq=Q + 64), la.LA_ERR_INVALID_ARG),
    ("cu_decreasing", dict(cu_host=np.array([0, 60, 50], np.int32), T=50), la.LA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", BAD_BACKWARD_SEGMENTED,
                         ids=[b[0] for b in BAD_BACKWARD_SEGMENTED])
def test_backward_segmented_rejects(name, kw, code):
    st, msg = _bwd_seg(**kw)
    assert st == code, (st, msg)
    assert msg


def test_backward_segmented_no_sequences():
    st, msg = _bwd_seg(S=0, T=0, cu_host=np.array([0], np.int32), ws=None, ws_bytes=0)
    assert st == la.LA_OK, msg


# ---- la_prefill_kernel_plan: the kernel choice of la_prefill on the host ----

VARLEN40 = [8335, 8420, 3054, 1378, 617, 1933, 2109, 598, 606, 16337, 4911, 1154, 2311, 14981,
            11492, 9549, 1994, 2827, 5343, 632, 3511, 1311, 10796, 639, 5389, 10444, 1125, 11403,
            10520, 545, 5945, 514, 2930, 2325, 1035, 1578, 8370, 1533, 858, 5762]

# (lengths, heads, head_dim, expected wide_seqs) on 256 compute units
PLANS = [
    ([8192], 64, 128, 0),                   # 64 chains: one wave of slices
    ([8192] * 2, 64, 128, 0),               # 128: two waves of slices beat one wide wave
    ([8192] * 3, 64, 128, 3),               # 192: one wave of the wide kernel
    ([8192] * 4, 64, 128, 4),               # 256
    ([8192] * 5, 64, 128, 4),               # 320: a wide wave, the fifth in slices
    ([576, 640, 640, 640, 640], 64, 128, 4),  # the same, the short one dispatched last
    ([8192] * 33, 8, 128, 32),              # 264: 32 sequences wide, one in slices
    ([8192] * 8, 64, 128, 8),               # 512: two whole waves
    ([8192] * 17, 64, 128, 16),             # 1088
    ([10356, 8478, 4478, 13501, 13513], 64, 128, 5),  # leftover chains fit the idle CUs
    (VARLEN40, 8, 128, 40),                 # likewise
    ([8192] * 200, 8, 128, 200),            # more sequences than the model plans for
    ([8192] * 5, 64, 64, 0),                # d = 64: slices only
    ([], 64, 128, 0),                       # no sequences
]


@pytest.mark.parametrize("lengths,H,d,expected", PLANS,
                         ids=[f"{len(p[0])}x{p[1]}h-d{p[2]}-{i}" for i, p in enumerate(PLANS)])
def test_kernel_plan(monkeypatch, lengths, H, d, expected):
    from la_inputs import cu_seqlens

    monkeypatch.delenv("LA_NDV", raising=False)
    n, order = la.kernel_plan(cu_seqlens(lengths), H, d, compute_units=256)
    assert n == expected
    # the dispatch order is longest first (stable) for 2 to 512 sequences
    if 2 <= len(lengths) <= 512:
        assert order.tolist() == sorted(range(len(lengths)), key=lambda i: -lengths[i])
    else:
        assert order.tolist() == list(range(len(lengths)))


def test_kernel_plan_override_and_errors(monkeypatch):
    from la_inputs import cu_seqlens

    cu = cu_seqlens([8192] * 5)
    monkeypatch.setenv("LA_NDV", "1")
    assert la.kernel_plan(cu, 64, compute_units=256)[0] == 5
    monkeypatch.setenv("LA_NDV", "4")
    assert la.kernel_plan(cu, 64, compute_units=256)[0] == 0
    monkeypatch.setenv("LA_NDV", "3")
    with pytest.raises(la.LAError, match="LA_NDV"):
        la.kernel_plan(cu, 64, compute_units=256)
    monkeypatch.delenv("LA_NDV")
    for args, code in (((5, cu.ctypes.data, 64, 128, -1), la.LA_ERR_INVALID_ARG),
                       ((-1, cu.ctypes.data, 64, 128, 256), la.LA_ERR_INVALID_ARG),
                       ((5, None, 64, 128, 256), la.LA_ERR_INVALID_ARG),
                       ((5, cu.ctypes.data, 0, 128, 256), la.LA_ERR_INVALID_ARG),
                       ((5, cu.ctypes.data, 64, 96, 256), la.LA_ERR_UNSUPPORTED)):
        st, _ = la.la_prefill_kernel_plan(*args, None)
        assert st == code, (args, st, la.la_last_error())
    bad = np.array([0, 10, 5], np.int32)
    st, _ = la.la_prefill_kernel_plan(2, bad.ctypes.data, 64, 128, 256, None)
    assert st == la.LA_ERR_INVALID_ARG
