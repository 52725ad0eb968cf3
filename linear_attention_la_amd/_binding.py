"""ctypes binding of libla's C ABI (include/la.h).

Two layers:

* ``la_prefill`` / ``la_decode`` / ``la_status_str`` / ``la_last_error``:
  the C entry points with the same names and plain integer pointers.
* ``prefill`` / ``decode``: torch-facing wrappers that check shapes, allocate
  outputs with torch on the inputs' device and pass ``data_ptr()`` and the
  current (or given) stream handle.
"""

import contextlib
import ctypes
import os

import numpy as np

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP = 0, 1, 2, 3
LA_BF16, LA_FP32 = 0, 1
LA_MAX_HEADS = 256

_HERE = os.path.dirname(os.path.abspath(__file__))
_DEFAULT_LIB = os.path.join(_HERE, "_lib", "libla.so")
_lib = None


class LaNorm(ctypes.Structure):
    """struct la_norm of la.h: the output normalisation's weight (device fp32
    [H, d]), epsilon and optional gate (device, layout and dtype of q)."""
    _fields_ = [("weight", ctypes.c_void_p), ("eps", ctypes.c_float), ("gate", ctypes.c_void_p)]


class LAError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


def _status_name(s):
    return {0: "LA_OK", 1: "LA_ERR_INVALID_ARG", 2: "LA_ERR_UNSUPPORTED", 3: "LA_ERR_HIP"}.get(
        s, f"status {s}")


def lib_path():
    """The in-tree libla.so, or the build that the environment variable
    LA_LIB names (to compare two builds of the library)."""
    return os.environ.get("LA_LIB", _DEFAULT_LIB)


def lib():
    """Load libla.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"libla.so not found at {path}; build it with "
            "`python -m linear_attention_la_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.la_prefill.restype = ctypes.c_int
    L.la_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_int, ctypes.c_int,
                             vp, vp, vp, vp, vp]
    L.la_prefill_pool.restype = ctypes.c_int
    L.la_prefill_pool.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_int,
                                  ctypes.c_int, vp, vp, i32, vp, vp, vp, vp]
    L.la_prefill_kernel_plan.restype = ctypes.c_int
    L.la_prefill_kernel_plan.argtypes = [i32, vp, i32, i32, i32, ctypes.POINTER(i32), vp]
    L.la_prefill_segmented.restype = ctypes.c_int
    L.la_prefill_segmented.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_int,
                                       ctypes.c_int, vp, vp, vp, vp, i32, vp, ctypes.c_size_t, vp]
    L.la_prefill_segmented_noalloc.restype = ctypes.c_int
    L.la_prefill_segmented_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                               ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i32,
                                               vp]
    L.la_prefill_segmented_workspace_size.restype = ctypes.c_int
    L.la_prefill_segmented_workspace_size.argtypes = [i32, vp, i32, i32, i32,
                                                      ctypes.POINTER(ctypes.c_size_t)]
    L.la_prefill_backward.restype = ctypes.c_int
    L.la_prefill_backward.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_int,
                                      ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    L.la_prefill_backward_workspace_size.restype = ctypes.c_int
    L.la_prefill_backward_workspace_size.argtypes = [i32, i32, i32,
                                                     ctypes.POINTER(ctypes.c_size_t)]
    L.la_prefill_backward_segmented.restype = ctypes.c_int
    L.la_prefill_backward_segmented.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                                ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp,
                                                vp, vp, i32, vp, ctypes.c_size_t, vp]
    L.la_prefill_backward_segmented_workspace_size.restype = ctypes.c_int
    L.la_prefill_backward_segmented_workspace_size.argtypes = [i32, vp, i32, i32, i32,
                                                               ctypes.POINTER(ctypes.c_size_t)]
    L.la_prefill_normed.restype = ctypes.c_int
    L.la_prefill_normed.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_int,
                                    ctypes.c_int, vp, vp, ctypes.POINTER(LaNorm), vp, vp, vp,
                                    ctypes.c_size_t, vp]
    L.la_prefill_normed_workspace_size.restype = ctypes.c_int
    L.la_prefill_normed_workspace_size.argtypes = [i32, vp, i32, i32,
                                                   ctypes.POINTER(ctypes.c_size_t)]
    L.la_decode_normed.restype = ctypes.c_int
    L.la_decode_normed.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_int,
                                   ctypes.POINTER(LaNorm), vp, vp]
    L.la_decode.restype = ctypes.c_int
    L.la_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_int, vp, vp]
    L.la_decode_pool.restype = ctypes.c_int
    L.la_decode_pool.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, ctypes.c_int,
                                 vp, vp]
    L.la_status_str.restype = ctypes.c_char_p
    L.la_status_str.argtypes = [ctypes.c_int]
    L.la_last_error.restype = ctypes.c_char_p
    L.la_last_error.argtypes = []
    _lib = L
    return L


# ---- raw C entry points (plain integer pointers) ----

def la_prefill(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens, num_heads,
               head_dim, in_dtype, out_dtype, decay, kv_init, o, kv_final, stream):
    return lib().la_prefill(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                            num_heads, head_dim, in_dtype, out_dtype, decay, kv_init, o,
                            kv_final, stream)


def la_prefill_segmented(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                         num_heads, head_dim, in_dtype, out_dtype, decay, kv_init, o, kv_final,
                         segment_len, workspace, workspace_bytes, stream):
    return lib().la_prefill_segmented(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                      total_tokens, num_heads, head_dim, in_dtype, out_dtype,
                                      decay, kv_init, o, kv_final, segment_len, workspace,
                                      workspace_bytes, stream)


def la_prefill_segmented_noalloc(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                 total_tokens, num_heads, head_dim, in_dtype, out_dtype, decay,
                                 kv_init, o, kv_final, segment_len, stream):
    return lib().la_prefill_segmented_noalloc(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                              total_tokens, num_heads, head_dim, in_dtype,
                                              out_dtype, decay, kv_init, o, kv_final,
                                              segment_len, stream)


def la_prefill_kernel_plan(num_seqs, cu_seqlens_host, num_heads, head_dim, compute_units,
                           order):
    """Returns (status, wide_seqs); ``order`` is a host int32 pointer or None."""
    n = ctypes.c_int32(0)
    st = lib().la_prefill_kernel_plan(num_seqs, cu_seqlens_host, num_heads, head_dim,
                                      compute_units, ctypes.byref(n), order)
    return st, n.value


def la_prefill_segmented_workspace_size(num_seqs, cu_seqlens_host, num_heads, head_dim,
                                        segment_len):
    """Returns (status, bytes)."""
    n = ctypes.c_size_t(0)
    st = lib().la_prefill_segmented_workspace_size(num_seqs, cu_seqlens_host, num_heads, head_dim,
                                                   segment_len, ctypes.byref(n))
    return st, n.value


def la_prefill_pool(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens, num_heads,
                    head_dim, in_dtype, out_dtype, decay, kv_pool, pool_size, slots_dev,
                    slots_host, o, stream):
    return lib().la_prefill_pool(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                 total_tokens, num_heads, head_dim, in_dtype, out_dtype, decay,
                                 kv_pool, pool_size, slots_dev, slots_host, o, stream)


def la_prefill_normed(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                      num_heads, head_dim, in_dtype, out_dtype, decay, kv_init, norm, o, kv_final,
                      workspace, workspace_bytes, stream):
    """``norm``: a LaNorm (or None for a NULL pointer)."""
    return lib().la_prefill_normed(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                   total_tokens, num_heads, head_dim, in_dtype, out_dtype, decay,
                                   kv_init, None if norm is None else ctypes.byref(norm), o,
                                   kv_final, workspace, workspace_bytes, stream)


def la_prefill_normed_workspace_size(num_seqs, cu_seqlens_host, num_heads, head_dim):
    """Returns (status, bytes)."""
    n = ctypes.c_size_t(0)
    st = lib().la_prefill_normed_workspace_size(num_seqs, cu_seqlens_host, num_heads, head_dim,
                                                ctypes.byref(n))
    return st, n.value


def la_decode_normed(q, k, v, kv, decay, batch, num_heads, head_dim, in_dtype, norm, o, stream):
    return lib().la_decode_normed(q, k, v, kv, decay, batch, num_heads, head_dim, in_dtype,
                                  None if norm is None else ctypes.byref(norm), o, stream)


def la_decode(q, k, v, kv, decay, batch, num_heads, head_dim, in_dtype, o, stream):
    return lib().la_decode(q, k, v, kv, decay, batch, num_heads, head_dim, in_dtype, o, stream)


def la_prefill_backward(q, k, v, d_o, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                        num_heads, head_dim, in_dtype, grad_dtype, decay, kv_init, dkv_final, dq,
                        dk, dv, dkv_init, workspace, workspace_bytes, stream):
    return lib().la_prefill_backward(q, k, v, d_o, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                     total_tokens, num_heads, head_dim, in_dtype, grad_dtype,
                                     decay, kv_init, dkv_final, dq, dk, dv, dkv_init, workspace,
                                     workspace_bytes, stream)


def la_prefill_backward_workspace_size(num_seqs, num_heads, head_dim):
    """Returns (status, bytes)."""
    n = ctypes.c_size_t(0)
    st = lib().la_prefill_backward_workspace_size(num_seqs, num_heads, head_dim, ctypes.byref(n))
    return st, n.value


def la_prefill_backward_segmented(q, k, v, d_o, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                  total_tokens, num_heads, head_dim, in_dtype, grad_dtype, decay,
                                  kv_init, dkv_final, dq, dk, dv, dkv_init, segment_len, workspace,
                                  workspace_bytes, stream):
    return lib().la_prefill_backward_segmented(q, k, v, d_o, cu_seqlens_dev, cu_seqlens_host,
                                               num_seqs, total_tokens, num_heads, head_dim,
                                               in_dtype, grad_dtype, decay, kv_init, dkv_final,
                                               dq, dk, dv, dkv_init, segment_len, workspace,
                                               workspace_bytes, stream)


def la_prefill_backward_segmented_workspace_size(num_seqs, cu_seqlens_host, num_heads, head_dim,
                                                 segment_len):
    """Returns (status, bytes); cu_seqlens_host: host address of int32 [S+1]."""
    n = ctypes.c_size_t(0)
    st = lib().la_prefill_backward_segmented_workspace_size(num_seqs, cu_seqlens_host, num_heads,
                                                            head_dim, segment_len,
                                                            ctypes.byref(n))
    return st, n.value


def la_decode_pool(q, k, v, kv_pool, pool_size, slots_dev, slots_host, decay, batch, num_heads,
                   head_dim, in_dtype, o, stream):
    return lib().la_decode_pool(q, k, v, kv_pool, pool_size, slots_dev, slots_host, decay, batch,
                                num_heads, head_dim, in_dtype, o, stream)


def la_status_str(s):
    return lib().la_status_str(s).decode()


def la_last_error():
    return lib().la_last_error().decode()


def _check(status):
    if status != LA_OK:
        raise LAError(status, la_last_error())


# ---- torch-facing wrappers ----

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


_SAME_DEVICE = contextlib.nullcontext()


def _on(device):
    """Context in which ``device`` is the calling thread's current HIP device:
    the library takes the device that owns a call's buffers to be the current
    one (its compute units, its static scratch), so every wrapper calls it
    inside this.  Switches only when another device is current."""
    torch = _torch()
    if device.index is None or device.index == torch.cuda.current_device():
        return _SAME_DEVICE
    return torch.cuda.device(device)


_hip = None


def _hip_runtime():
    """The HIP runtime already loaded in this process (torch's, which libla
    uses too: both name it by its soname)."""
    global _hip
    if _hip is None:
        _torch()
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipExtStreamCreateWithCUMask.restype = ctypes.c_int
        _hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint32,
                                                     ctypes.POINTER(ctypes.c_uint32)]
    return _hip


_masked_streams = {}


def cu_masked_stream(cu_mask, device=None):
    """A HIP stream (default priority) whose kernels run only on the compute
    units set in ``cu_mask`` (an int, bit i = compute unit i as the HIP
    runtime numbers them), wrapped as a torch ExternalStream usable as
    ``stream=`` of every call here.  Serving can give the latency-bound decode
    and the prefill disjoint sets of compute units, so that neither waits for
    the other's workgroups to drain.  One stream is created per (device,
    mask) and reused; it lives until the process ends (it is never destroyed:
    destroying it from a finaliser at interpreter exit would race the HIP
    runtime's own teardown)."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    m = int(cu_mask)
    if m <= 0:
        raise ValueError("cu_mask must select at least one compute unit")
    key = (dev.index, m)
    if key in _masked_streams:
        return _masked_streams[key]
    words = []
    while m:
        words.append(m & 0xFFFFFFFF)
        m >>= 32
    arr = (ctypes.c_uint32 * len(words))(*words)
    handle = ctypes.c_void_p()
    with torch.cuda.device(dev):
        st = _hip_runtime().hipExtStreamCreateWithCUMask(ctypes.byref(handle), len(words), arr)
    if st != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with HIP error {st}")
    stream = torch.cuda.ExternalStream(handle.value, device=dev)
    _masked_streams[key] = stream
    return stream


def _check_out(name, t, shape, dtype, device):
    """A caller-supplied output or workspace-like buffer: the library writes
    exactly ``shape`` elements of ``dtype`` through its pointer and cannot
    see the tensor's size, so anything else is rejected here."""
    torch = _torch()
    if not (isinstance(t, torch.Tensor) and t.device == device and t.dtype == dtype
            and tuple(t.shape) == tuple(shape) and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}")
    return t


def _check_device_buffer(name, t, device):
    """A caller-supplied workspace: a contiguous tensor on ``device`` (its
    size in bytes is passed to the library, which checks it)."""
    torch = _torch()
    if not (isinstance(t, torch.Tensor) and t.device == device and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    return t


def _host_decay(decay, num_heads):
    torch = _torch()
    if isinstance(decay, torch.Tensor):
        decay = decay.detach().cpu().numpy()
    d = np.ascontiguousarray(np.asarray(decay, dtype=np.float32).reshape(-1))
    if d.shape[0] != num_heads:
        raise ValueError(f"decay has {d.shape[0]} entries, expected {num_heads}")
    return d


class _Prefill:
    """Marshalled arguments of a prefill call."""


def _marshal_prefill(q, k, v, cu_seqlens, decay, kv_init, out_dtype, stream, final_state, out,
                     kv_final, cu_seqlens_host):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a device tensor")
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [T, H, d] tensor")
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype \
            or q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must share shape, dtype and device")
    T, H, d = q.shape
    dev = q.device
    in_code = _dtype_code(q)
    if out_dtype is None:
        out_dtype = q.dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported out_dtype {out_dtype} (bfloat16 or float32)")
    out_code = LA_BF16 if out_dtype == torch.bfloat16 else LA_FP32
    if cu_seqlens_host is not None:
        cu_host = torch.as_tensor(np.ascontiguousarray(
            cu_seqlens_host.cpu().numpy() if isinstance(cu_seqlens_host, torch.Tensor)
            else cu_seqlens_host, dtype=np.int32))
        if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda
                and cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous()):
            raise ValueError("cu_seqlens_host needs cu_seqlens as a contiguous int32 device tensor")
        cu_dev = cu_seqlens
    elif isinstance(cu_seqlens, torch.Tensor):
        cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
        cu_dev = cu_seqlens if (cu_seqlens.is_cuda and cu_seqlens.dtype == torch.int32
                                and cu_seqlens.is_contiguous()) else cu_host.to(dev)
    else:
        cu_host = torch.from_numpy(np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32)))
        cu_dev = cu_host.to(dev)
    if stream is not None and cu_dev is not cu_seqlens:
        cu_dev.record_stream(stream)  # temporary read by a kernel on another stream
    S = cu_host.numel() - 1
    if S < 0:
        raise ValueError("cu_seqlens must have at least one entry")
    if cu_dev.numel() != cu_host.numel() or cu_dev.device != dev:
        raise ValueError("cu_seqlens and cu_seqlens_host must have the same length, "
                         "cu_seqlens on q's device")
    dec = _host_decay(decay, H)
    if kv_init is not None:
        _check_out("kv_init", kv_init, (S, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty((T, H, d), dtype=out_dtype, device=dev)
    else:
        _check_out("out", out, (T, H, d), out_dtype, dev)
    if not final_state:
        kv_final = None
    elif kv_final is None:
        kv_final = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
    else:
        _check_out("kv_final", kv_final, (S, H, d, d), torch.float32, dev)
    m = _Prefill()
    m.T, m.H, m.d, m.S, m.dev = T, H, d, S, dev
    m.in_code, m.out_code = in_code, out_code
    m.cu_dev, m.cu_host, m.dec = cu_dev, cu_host, dec
    m.out, m.kv_final = out, kv_final
    m.args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_dev.data_ptr(), cu_host.data_ptr(), S,
              T, H, d, in_code, out_code, dec.ctypes.data,
              None if kv_init is None else kv_init.data_ptr(), out.data_ptr(),
              None if kv_final is None else kv_final.data_ptr())
    m.stream = _stream_handle(stream, dev)
    return m


def prefill(q, k, v, cu_seqlens, decay, kv_init=None, out_dtype=None, stream=None,
            final_state=True, out=None, kv_final=None, cu_seqlens_host=None):
    """Packed varlen prefill.  q, k, v: device [T, H, d] (bf16 or fp32, same
    dtype, contiguous).  cu_seqlens: [S+1] int (host or device).  decay: host
    [H] floats in (0, 1].  kv_init: device fp32 [S, H, d, d] or None.

    Returns (o [T, H, d], kv_final [S, H, d, d] or None).  ``out`` and
    ``kv_final`` may supply preallocated outputs; ``kv_final`` may be
    ``kv_init`` itself (in-place continuation).  When cu_seqlens is a device
    tensor, passing its host copy as ``cu_seqlens_host`` (a CPU int32 tensor or
    array with the same contents) avoids a device-to-host copy, which would
    synchronise the stream on every call."""
    m = _marshal_prefill(q, k, v, cu_seqlens, decay, kv_init, out_dtype, stream, final_state,
                         out, kv_final, cu_seqlens_host)
    with _on(m.dev):
        _check(la_prefill(*m.args, m.stream))
    return m.out, m.kv_final


def kernel_plan(cu_seqlens_host, num_heads, head_dim=128, compute_units=0):
    """The kernels prefill() and prefill_pool() would run for bf16 inputs with
    these sequences (la_prefill_kernel_plan): (wide_seqs, order) -- the first
    ``wide_seqs`` sequences of ``order`` run one workgroup per (sequence,
    head), the others in 32-column slices.  ``compute_units`` 0 plans for the
    current device."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32).reshape(-1))
    order = np.zeros(max(cu.shape[0] - 1, 0), dtype=np.int32)
    st, n = la_prefill_kernel_plan(cu.shape[0] - 1, cu.ctypes.data, num_heads, head_dim,
                                   compute_units, order.ctypes.data if order.size else None)
    _check(st)
    return n, order


def prefill_segmented_workspace_size(cu_seqlens_host, num_heads, head_dim, segment_len):
    """Bytes of workspace that prefill_segmented needs (host computation)."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32).reshape(-1))
    st, n = la_prefill_segmented_workspace_size(cu.shape[0] - 1, cu.ctypes.data, num_heads,
                                                head_dim, segment_len)
    _check(st)
    return n


def prefill_segmented(q, k, v, cu_seqlens, decay, segment_len, kv_init=None, out_dtype=None,
                      stream=None, final_state=True, out=None, kv_final=None,
                      cu_seqlens_host=None, workspace=None):
    """prefill() with every sequence cut into segments of ``segment_len``
    tokens (a multiple of 64, or 0 for the library's choice) processed as
    parallel chains.  ``workspace``: a device tensor of at least
    prefill_segmented_workspace_size() bytes, or None to allocate one.  Same
    returns as prefill()."""
    torch = _torch()
    m = _marshal_prefill(q, k, v, cu_seqlens, decay, kv_init, out_dtype, stream, final_state,
                         out, kv_final, cu_seqlens_host)
    with _on(m.dev):
        st, need = la_prefill_segmented_workspace_size(m.S, m.cu_host.data_ptr(), m.H, m.d,
                                                       segment_len)
        _check(st)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=m.dev)
            if stream is not None:
                workspace.record_stream(stream)
        else:
            _check_device_buffer("workspace", workspace, m.dev)
        nbytes = workspace.numel() * workspace.element_size()
        _check(la_prefill_segmented(*m.args, segment_len, workspace.data_ptr(), nbytes,
                                    m.stream))
    return m.out, m.kv_final


def prefill_segmented_noalloc(q, k, v, cu_seqlens, decay, segment_len, kv_init=None,
                              out_dtype=None, stream=None, final_state=True, out=None,
                              kv_final=None, cu_seqlens_host=None):
    """prefill_segmented() whose workspace is the library's static device
    scratch (la_prefill_segmented_noalloc): the library allocates nothing.
    Pass ``out`` (and ``kv_final``) to allocate nothing on the Python side
    either.  Calls that overlap in time on one device race on the scratch.
    Same returns as prefill()."""
    m = _marshal_prefill(q, k, v, cu_seqlens, decay, kv_init, out_dtype, stream, final_state,
                         out, kv_final, cu_seqlens_host)
    with _on(m.dev):
        _check(la_prefill_segmented_noalloc(*m.args, segment_len, m.stream))
    return m.out, m.kv_final


def _marshal_norm(weight, eps, gate, H, d, dev, like):
    """LaNorm for a weight [H, d] (device fp32 tensor, or host values copied
    to the device) and an optional gate tensor shaped and typed as ``like``.
    Returns (LaNorm, tensors to keep alive)."""
    torch = _torch()
    if not isinstance(weight, torch.Tensor):
        weight = torch.as_tensor(np.asarray(weight, dtype=np.float32)).to(dev)
    if (weight.device != dev or weight.dtype != torch.float32 or not weight.is_contiguous()
            or tuple(weight.shape) != (H, d)):
        raise ValueError("norm weight must be a contiguous fp32 device tensor [H, d]")
    if gate is not None:
        if (not isinstance(gate, torch.Tensor) or gate.device != dev or gate.dtype != like.dtype
                or not gate.is_contiguous() or gate.shape != like.shape):
            raise ValueError("gate must be a contiguous device tensor shaped and typed as q")
    nm = LaNorm(weight.data_ptr(), float(eps), None if gate is None else gate.data_ptr())
    return nm, (weight, gate)


def prefill_normed(q, k, v, cu_seqlens, decay, weight, eps=1e-6, gate=None, kv_init=None,
                   out_dtype=None, stream=None, final_state=True, out=None, kv_final=None,
                   cu_seqlens_host=None, workspace=None):
    """prefill() whose output rows are normalised before they are written:
    out = weight[h] * o / sqrt(mean(o^2) + eps) (* sigmoid(gate)), o being
    prefill()'s output (la_prefill_normed).  q, k, v bf16 [T, H, 128];
    weight fp32 [H, 128]; gate None or like q.  ``workspace``: device bytes
    of at least prefill_normed_workspace_size() (allocated here if None and
    needed).  Returns (out, kv_final)."""
    torch = _torch()
    m = _marshal_prefill(q, k, v, cu_seqlens, decay, kv_init, out_dtype, stream, final_state,
                         out, kv_final, cu_seqlens_host)
    nm, keep = _marshal_norm(weight, eps, gate, m.H, m.d, m.dev, q)
    with _on(m.dev):
        st, need = la_prefill_normed_workspace_size(m.S, m.cu_host.data_ptr(), m.H, m.d)
        _check(st)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=m.dev)
            if stream is not None:
                workspace.record_stream(stream)
        elif workspace is not None:
            _check_device_buffer("workspace", workspace, m.dev)
        wp = 0 if workspace is None else workspace.data_ptr()
        nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        a = m.args
        _check(la_prefill_normed(*a[:13], nm, a[13], a[14], wp or None, nbytes, m.stream))
    del keep
    return m.out, m.kv_final


def prefill_normed_workspace_size(cu_seqlens_host, num_heads, head_dim):
    """Bytes of device workspace prefill_normed needs on the current device."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32).reshape(-1))
    st, n = la_prefill_normed_workspace_size(cu.shape[0] - 1, cu.ctypes.data, num_heads,
                                             head_dim)
    _check(st)
    return n


def _marshal_slots(slots, slots_host, n, dev, stream):
    """Pool slots as (device int32 tensor, host int32 array) of shape [n]."""
    torch = _torch()
    if slots_host is not None:
        sl_host = np.ascontiguousarray(
            slots_host.cpu().numpy() if isinstance(slots_host, torch.Tensor) else slots_host,
            dtype=np.int32)
        if not (isinstance(slots, torch.Tensor) and slots.is_cuda and slots.dtype == torch.int32
                and slots.is_contiguous()):
            raise ValueError("slots_host needs slots as a contiguous int32 device tensor")
        sl_dev = slots
    elif isinstance(slots, torch.Tensor):
        sl_host = slots.detach().to("cpu", torch.int32).contiguous().numpy()
        sl_dev = slots if (slots.is_cuda and slots.dtype == torch.int32
                           and slots.is_contiguous()) else torch.from_numpy(sl_host).to(dev)
    else:
        sl_host = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
        sl_dev = torch.from_numpy(sl_host).to(dev)
    if stream is not None and sl_dev is not slots:
        sl_dev.record_stream(stream)  # temporary read by a kernel on another stream
    if sl_host.shape != (n,) or sl_dev.numel() != n or sl_dev.device != dev:
        raise ValueError(f"slots has shape {sl_host.shape} (device copy: {sl_dev.numel()} on "
                         f"{sl_dev.device}), expected ({n},) on {dev}")
    return sl_dev, sl_host


def prefill_pool(q, k, v, cu_seqlens, decay, kv_pool, slots, out_dtype=None, stream=None,
                 out=None, cu_seqlens_host=None, slots_host=None):
    """Packed varlen prefill on a state pool: sequence s continues from
    kv_pool[slots[s]] and writes its final state back to that slot (in
    place).  q, k, v: device bf16 [T, H, d]; kv_pool: device fp32
    [P, H, d, d]; slots: [S] int (host or device), distinct, in [0, P).
    Passing host copies (``cu_seqlens_host``, ``slots_host``) with device
    int32 ``cu_seqlens`` and ``slots`` avoids device-to-host copies.
    Returns o [T, H, d]."""
    torch = _torch()
    m = _marshal_prefill(q, k, v, cu_seqlens, decay, None, out_dtype, stream, False, out, None,
                         cu_seqlens_host)
    if (not isinstance(kv_pool, torch.Tensor) or kv_pool.device != m.dev
            or kv_pool.dtype != torch.float32 or not kv_pool.is_contiguous()
            or kv_pool.dim() != 4 or tuple(kv_pool.shape[1:]) != (m.H, m.d, m.d)):
        raise ValueError("kv_pool must be a contiguous fp32 device tensor [P, H, d, d]")
    sl_dev, sl_host = _marshal_slots(slots, slots_host, m.S, m.dev, stream)
    with _on(m.dev):
        _check(la_prefill_pool(q.data_ptr(), k.data_ptr(), v.data_ptr(), m.cu_dev.data_ptr(),
                               m.cu_host.data_ptr(), m.S, m.T, m.H, m.d, m.in_code, m.out_code,
                               m.dec.ctypes.data, kv_pool.data_ptr(), kv_pool.shape[0],
                               sl_dev.data_ptr(), sl_host.ctypes.data, m.out.data_ptr(),
                               m.stream))
    return m.out


def decode(q, k, v, kv, decay, stream=None, out=None):
    """One decode token per sequence.  q, k, v: device [B, H, d]; kv: device
    fp32 [B, H, d, d], updated in place.  Returns o [B, H, d] (q's dtype)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("kv", kv)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dim() != 3 or q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype \
            or q.dtype != v.dtype or q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must share shape [B, H, d], dtype and device")
    B, H, d = q.shape
    _dtype_code(q)
    _check_out("kv", kv, (B, H, d, d), torch.float32, q.device)
    dec = _host_decay(decay, H)
    out = torch.empty_like(q) if out is None else _check_out("out", out, q.shape, q.dtype, q.device)
    with _on(q.device):
        _check(la_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), kv.data_ptr(),
                         dec.ctypes.data, B, H, d, _dtype_code(q), out.data_ptr(),
                         _stream_handle(stream, q.device)))
    return out


def decode_normed(q, k, v, kv, decay, weight, eps=1e-6, gate=None, stream=None, out=None):
    """decode() whose output is normalised before it is written (la_decode_normed):
    out = weight[h] * o / sqrt(mean(o^2) + eps) (* sigmoid(gate)).  weight:
    fp32 [H, d]; gate None or like q.  kv is updated in place as by decode()."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("kv", kv)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dim() != 3 or q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype \
            or q.dtype != v.dtype or q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must share shape [B, H, d], dtype and device")
    B, H, d = q.shape
    _dtype_code(q)
    _check_out("kv", kv, (B, H, d, d), torch.float32, q.device)
    dec = _host_decay(decay, H)
    nm, keep = _marshal_norm(weight, eps, gate, H, d, q.device, q)
    out = torch.empty_like(q) if out is None else _check_out("out", out, q.shape, q.dtype, q.device)
    with _on(q.device):
        _check(la_decode_normed(q.data_ptr(), k.data_ptr(), v.data_ptr(), kv.data_ptr(),
                                dec.ctypes.data, B, H, d, _dtype_code(q), nm, out.data_ptr(),
                                _stream_handle(stream, q.device)))
    del keep
    return out


def decode_pool(q, k, v, kv_pool, slots, decay, stream=None, out=None, slots_host=None):
    """One decode token per sequence on a state pool.  q, k, v: device
    [B, H, d]; kv_pool: device fp32 [P, H, d, d] updated in place at the
    slots; slots: [B] int (host or device), distinct, in [0, P).  Passing the
    host copy as ``slots_host`` with a device int32 ``slots`` avoids a
    device-to-host copy.  Returns o [B, H, d]."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 3 \
                or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, d] device tensor")
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype \
            or q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must share shape [B, H, d], dtype and device")
    B, H, d = q.shape
    _dtype_code(q)
    if (not isinstance(kv_pool, torch.Tensor) or kv_pool.device != q.device
            or kv_pool.dtype != torch.float32 or not kv_pool.is_contiguous()
            or kv_pool.dim() != 4 or tuple(kv_pool.shape[1:]) != (H, d, d)):
        raise ValueError("kv_pool must be a contiguous fp32 device tensor [P, H, d, d]")
    P = kv_pool.shape[0]
    dev = q.device
    sl_dev, sl_host = _marshal_slots(slots, slots_host, B, dev, stream)
    dec = _host_decay(decay, H)
    out = torch.empty_like(q) if out is None else _check_out("out", out, q.shape, q.dtype, dev)
    with _on(dev):
        _check(la_decode_pool(q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_pool.data_ptr(), P,
                              sl_dev.data_ptr(), sl_host.ctypes.data, dec.ctypes.data, B, H, d,
                              _dtype_code(q), out.data_ptr(), _stream_handle(stream, dev)))
    return out


def _backward(q, k, v, d_o, cu_seqlens, decay, kv_init, dkv_final, grad_dtype, stream, init_grad,
              cu_seqlens_host, workspace, dq, dk, dv, dkv_init, segment_len):
    torch = _torch()
    m = _marshal_prefill(q, k, v, cu_seqlens, decay, kv_init, grad_dtype, stream, False, dq,
                         None, cu_seqlens_host)
    _check_out("d_o", d_o, q.shape, q.dtype, m.dev)
    if dkv_final is not None:
        _check_out("dkv_final", dkv_final, (m.S, m.H, m.d, m.d), torch.float32, m.dev)
    gdt = m.out.dtype  # grad_dtype (default: q's), as checked for dq
    dk = torch.empty(q.shape, dtype=gdt, device=m.dev) if dk is None else \
        _check_out("dk", dk, q.shape, gdt, m.dev)
    dv = torch.empty(q.shape, dtype=gdt, device=m.dev) if dv is None else \
        _check_out("dv", dv, q.shape, gdt, m.dev)
    if not init_grad:
        dkv_init = None
    elif dkv_init is None:
        dkv_init = torch.empty((m.S, m.H, m.d, m.d), dtype=torch.float32, device=m.dev)
    else:
        _check_out("dkv_init", dkv_init, (m.S, m.H, m.d, m.d), torch.float32, m.dev)
    with _on(m.dev):
        return _backward_call(m, d_o, kv_init, dkv_final, stream, workspace, dk, dv, dkv_init,
                              segment_len)


def _backward_call(m, d_o, kv_init, dkv_final, stream, workspace, dk, dv, dkv_init,
                   segment_len):
    torch = _torch()
    if segment_len is None:
        st, need = la_prefill_backward_workspace_size(m.S, m.H, m.d)
        needed = kv_init is not None or dkv_final is not None
    else:
        st, need = la_prefill_backward_segmented_workspace_size(m.S, m.cu_host.data_ptr(), m.H,
                                                                m.d, segment_len)
        needed = True
    _check(st)
    if workspace is None and needed:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=m.dev)
        if stream is not None:
            workspace.record_stream(stream)
    elif workspace is not None:
        _check_device_buffer("workspace", workspace, m.dev)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    (qp, kp, vp_, cud, cuh, S, T, H, d, in_code, out_code, decp, kvip, dqp, _) = m.args
    common = (qp, kp, vp_, d_o.data_ptr(), cud, cuh, S, T, H, d, in_code, out_code, decp, kvip,
              None if dkv_final is None else dkv_final.data_ptr(), dqp, dk.data_ptr(),
              dv.data_ptr(), None if dkv_init is None else dkv_init.data_ptr())
    ws = None if workspace is None else workspace.data_ptr()
    if segment_len is None:
        _check(la_prefill_backward(*common, ws, nbytes, m.stream))
    else:
        _check(la_prefill_backward_segmented(*common, segment_len, ws, nbytes, m.stream))
    return m.out, dk, dv, dkv_init


def prefill_backward(q, k, v, d_o, cu_seqlens, decay, kv_init=None, dkv_final=None,
                     grad_dtype=None, stream=None, init_grad=True, cu_seqlens_host=None,
                     workspace=None, dq=None, dk=None, dv=None, dkv_init=None):
    """Gradients of prefill().  q, k, v, d_o: device bf16 [T, H, d];
    kv_init / dkv_final: device fp32 [S, H, d, d] or None.  Returns
    (dq, dk, dv, dkv_init or None); grad_dtype defaults to the input dtype."""
    return _backward(q, k, v, d_o, cu_seqlens, decay, kv_init, dkv_final, grad_dtype, stream,
                     init_grad, cu_seqlens_host, workspace, dq, dk, dv, dkv_init, None)


def prefill_backward_segmented(q, k, v, d_o, cu_seqlens, decay, segment_len, kv_init=None,
                               dkv_final=None, grad_dtype=None, stream=None, init_grad=True,
                               cu_seqlens_host=None, workspace=None, dq=None, dk=None, dv=None,
                               dkv_init=None):
    """prefill_backward() with every sequence cut into segments of
    ``segment_len`` tokens (a multiple of 64, or 0 for the library's choice)
    processed as parallel chains.
    ``workspace``: a device tensor of at least
    prefill_backward_segmented_workspace_size() bytes, or None to allocate
    one.  Same returns as prefill_backward()."""
    return _backward(q, k, v, d_o, cu_seqlens, decay, kv_init, dkv_final, grad_dtype, stream,
                     init_grad, cu_seqlens_host, workspace, dq, dk, dv, dkv_init, segment_len)


def prefill_backward_segmented_workspace_size(cu_seqlens_host, num_heads, head_dim, segment_len):
    """Bytes of workspace that prefill_backward_segmented needs (host computation)."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32).reshape(-1))
    st, n = la_prefill_backward_segmented_workspace_size(cu.shape[0] - 1, cu.ctypes.data,
                                                         num_heads, head_dim, segment_len)
    _check(st)
    return n


# ---- autograd ----

_attention_fn = None


def _attention_function():
    """The torch.autograd.Function behind attention(), defined on first use
    (torch is imported lazily by this module)."""
    global _attention_fn
    if _attention_fn is not None:
        return _attention_fn
    torch = _torch()

    class LightningAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, kv_init, cu_dev, cu_host, decay, segment_len):
            ctx.set_materialize_grads(False)
            if segment_len is None:
                o, kv = prefill(q, k, v, cu_dev, decay, kv_init=kv_init,
                                cu_seqlens_host=cu_host)
            else:
                o, kv = prefill_segmented(q, k, v, cu_dev, decay, segment_len, kv_init=kv_init,
                                          cu_seqlens_host=cu_host)
            ctx.save_for_backward(q, k, v, kv_init)
            ctx.cu = (cu_dev, cu_host)
            ctx.decay, ctx.segment_len = decay, segment_len
            return o, kv

        @staticmethod
        def backward(ctx, d_o, dkv_final):
            q, k, v, kv_init = ctx.saved_tensors
            needs = ctx.needs_input_grad
            if d_o is None and dkv_final is None:
                return (None,) * 8
            # an unused output's gradient is zero (the library needs d_o)
            d_o = torch.zeros_like(q) if d_o is None else d_o.contiguous()
            if dkv_final is not None:
                dkv_final = dkv_final.contiguous()
            cu_dev, cu_host = ctx.cu
            init_grad = kv_init is not None and needs[3]
            common = dict(kv_init=kv_init, dkv_final=dkv_final, init_grad=init_grad,
                          cu_seqlens_host=cu_host)
            if ctx.segment_len is None:
                dq, dk, dv, dkv0 = prefill_backward(q, k, v, d_o, cu_dev, ctx.decay, **common)
            else:
                dq, dk, dv, dkv0 = prefill_backward_segmented(q, k, v, d_o, cu_dev, ctx.decay,
                                                              ctx.segment_len, **common)
            return (dq if needs[0] else None, dk if needs[1] else None,
                    dv if needs[2] else None, dkv0 if init_grad else None,
                    None, None, None, None)

    _attention_fn = LightningAttention
    return _attention_fn


def attention(q, k, v, cu_seqlens, decay, kv_init=None, segment_len=None):
    """Differentiable prefill: (o, kv_final) = prefill(...) with gradients for
    q, k, v and kv_init through prefill_backward (segment_len given: through
    prefill_segmented and prefill_backward_segmented).  q, k, v: device bf16
    [T, H, d]; decay: host [H], not differentiated; kv_init: device fp32
    [S, H, d, d] or None.  Gradients have the dtype of their input.
    cu_seqlens is copied to the host once, here, and both copies are reused
    by the backward."""
    torch = _torch()
    if not isinstance(q, torch.Tensor) or not q.is_cuda:
        raise TypeError("q must be a device tensor")
    if q.dtype != torch.bfloat16:
        raise TypeError("attention() takes bf16 q, k, v (the backward is bf16-only)")
    if q.dim() != 3:
        raise ValueError("q must be a [T, H, d] tensor")
    dev = q.device
    if isinstance(cu_seqlens, torch.Tensor):
        cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
        cu_dev = cu_seqlens if (cu_seqlens.device == dev and cu_seqlens.dtype == torch.int32
                                and cu_seqlens.is_contiguous()) else cu_host.to(dev)
    else:
        cu_host = torch.from_numpy(np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32)))
        cu_dev = cu_host.to(dev)
    decay = _host_decay(decay, q.shape[1])
    return _attention_function().apply(q, k, v, kv_init, cu_dev, cu_host, decay, segment_len)
