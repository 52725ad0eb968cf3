"""ctypes binding of libla's C ABI (include/la.h).

Two layers:

* ``la_prefill`` / ``la_decode`` / ``la_status_str`` / ``la_last_error``:
  the C entry points with the same names and plain integer pointers.
* ``prefill`` / ``decode``: torch-facing wrappers that check shapes, allocate
  outputs with torch on the inputs' device and pass ``data_ptr()`` and the
  current (or given) stream handle.
"""

import ctypes
import os

import numpy as np

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP = 0, 1, 2, 3
LA_BF16, LA_FP32 = 0, 1
LA_MAX_HEADS = 256

_HERE = os.path.dirname(os.path.abspath(__file__))
_DEFAULT_LIB = os.path.join(_HERE, "_lib", "libla.so")
_lib = None


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
    L.la_prefill_segmented.restype = ctypes.c_int
    L.la_prefill_segmented.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_int,
                                       ctypes.c_int, vp, vp, vp, vp, i32, vp, ctypes.c_size_t, vp]
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
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    T, H, d = q.shape
    dev = q.device
    in_code = _dtype_code(q)
    if out_dtype is None:
        out_dtype = q.dtype
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
    dec = _host_decay(decay, H)
    if kv_init is not None:
        if (not kv_init.is_cuda or kv_init.dtype != torch.float32 or not kv_init.is_contiguous()
                or tuple(kv_init.shape) != (S, H, d, d)):
            raise ValueError("kv_init must be a contiguous fp32 device tensor [S, H, d, d]")
    if out is None:
        out = torch.empty((T, H, d), dtype=out_dtype, device=dev)
    if final_state and kv_final is None:
        kv_final = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
    if not final_state:
        kv_final = None
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
    _check(la_prefill(*m.args, m.stream))
    return m.out, m.kv_final


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
    tokens (a multiple of 64) processed as parallel chains.  ``workspace``: a
    device tensor of at least prefill_segmented_workspace_size() bytes, or
    None to allocate one.  Same returns as prefill()."""
    torch = _torch()
    m = _marshal_prefill(q, k, v, cu_seqlens, decay, kv_init, out_dtype, stream, final_state,
                         out, kv_final, cu_seqlens_host)
    st, need = la_prefill_segmented_workspace_size(m.S, m.cu_host.data_ptr(), m.H, m.d,
                                                   segment_len)
    _check(st)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=m.dev)
        if stream is not None:
            workspace.record_stream(stream)
    elif not (isinstance(workspace, torch.Tensor) and workspace.is_cuda
              and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(la_prefill_segmented(*m.args, segment_len, workspace.data_ptr(), nbytes, m.stream))
    return m.out, m.kv_final


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
    if sl_host.shape != (n,):
        raise ValueError(f"slots has shape {sl_host.shape}, expected ({n},)")
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
    if (not isinstance(kv_pool, torch.Tensor) or not kv_pool.is_cuda
            or kv_pool.dtype != torch.float32 or not kv_pool.is_contiguous()
            or kv_pool.dim() != 4 or tuple(kv_pool.shape[1:]) != (m.H, m.d, m.d)):
        raise ValueError("kv_pool must be a contiguous fp32 device tensor [P, H, d, d]")
    sl_dev, sl_host = _marshal_slots(slots, slots_host, m.S, m.dev, stream)
    _check(la_prefill_pool(q.data_ptr(), k.data_ptr(), v.data_ptr(), m.cu_dev.data_ptr(),
                           m.cu_host.data_ptr(), m.S, m.T, m.H, m.d, m.in_code, m.out_code,
                           m.dec.ctypes.data, kv_pool.data_ptr(), kv_pool.shape[0],
                           sl_dev.data_ptr(), sl_host.ctypes.data, m.out.data_ptr(), m.stream))
    return m.out


def decode(q, k, v, kv, decay, stream=None, out=None):
    """One decode token per sequence.  q, k, v: device [B, H, d]; kv: device
    fp32 [B, H, d, d], updated in place.  Returns o [B, H, d] (q's dtype)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("kv", kv)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dim() != 3 or q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype \
            or q.dtype != v.dtype:
        raise ValueError("q, k, v must share shape [B, H, d] and dtype")
    B, H, d = q.shape
    if kv.dtype != torch.float32 or tuple(kv.shape) != (B, H, d, d):
        raise ValueError("kv must be fp32 [B, H, d, d]")
    dec = _host_decay(decay, H)
    if out is None:
        out = torch.empty_like(q)
    st = la_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), kv.data_ptr(), dec.ctypes.data,
                   B, H, d, _dtype_code(q), out.data_ptr(), _stream_handle(stream, q.device))
    _check(st)
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
    B, H, d = q.shape
    if (not kv_pool.is_cuda or kv_pool.dtype != torch.float32 or not kv_pool.is_contiguous()
            or kv_pool.dim() != 4 or tuple(kv_pool.shape[1:]) != (H, d, d)):
        raise ValueError("kv_pool must be a contiguous fp32 device tensor [P, H, d, d]")
    P = kv_pool.shape[0]
    dev = q.device
    sl_dev, sl_host = _marshal_slots(slots, slots_host, B, dev, stream)
    dec = _host_decay(decay, H)
    if out is None:
        out = torch.empty_like(q)
    st = la_decode_pool(q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_pool.data_ptr(), P,
                        sl_dev.data_ptr(), sl_host.ctypes.data, dec.ctypes.data, B, H, d,
                        _dtype_code(q), out.data_ptr(), _stream_handle(stream, dev))
    _check(st)
    return out


def _backward(q, k, v, d_o, cu_seqlens, decay, kv_init, dkv_final, grad_dtype, stream, init_grad,
              cu_seqlens_host, workspace, dq, dk, dv, dkv_init, segment_len):
    torch = _torch()
    m = _marshal_prefill(q, k, v, cu_seqlens, decay, kv_init, grad_dtype, stream, False, dq,
                         None, cu_seqlens_host)
    if not (isinstance(d_o, torch.Tensor) and d_o.is_cuda and d_o.shape == q.shape
            and d_o.dtype == q.dtype and d_o.is_contiguous()):
        raise ValueError("d_o must be a contiguous device tensor like q")
    if dkv_final is not None and (not dkv_final.is_cuda or dkv_final.dtype != torch.float32
                                  or not dkv_final.is_contiguous()
                                  or tuple(dkv_final.shape) != (m.S, m.H, m.d, m.d)):
        raise ValueError("dkv_final must be a contiguous fp32 device tensor [S, H, d, d]")
    gdt = q.dtype if grad_dtype is None else grad_dtype
    dk = torch.empty(q.shape, dtype=gdt, device=m.dev) if dk is None else dk
    dv = torch.empty(q.shape, dtype=gdt, device=m.dev) if dv is None else dv
    if init_grad and dkv_init is None:
        dkv_init = torch.empty((m.S, m.H, m.d, m.d), dtype=torch.float32, device=m.dev)
    if not init_grad:
        dkv_init = None
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
    elif workspace is not None and not (isinstance(workspace, torch.Tensor) and workspace.is_cuda
                                        and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
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
    ``segment_len`` tokens (a multiple of 64) processed as parallel chains.
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
