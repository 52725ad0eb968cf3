"""Lightning Attention prefill and decode for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libla.so`` (include/la.h).  It only
marshals arguments: torch supplies device memory and streams, every step of
the computation runs in the HIP kernels.  There is no CPU fallback: if the
library is missing, every call raises.

    o, kv = prefill(q, k, v, cu_seqlens, decay, kv_init=None, out_dtype=None)
    o, kv = prefill_segmented(q, k, v, cu_seqlens, decay, segment_len)
    o, kv = prefill_segmented_noalloc(q, k, v, cu_seqlens, decay, segment_len)  # static scratch
    dq, dk, dv, dkv0 = prefill_backward(q, k, v, do, cu_seqlens, decay, kv_init, dkv_final)
    o = decode(q, k, v, kv, decay)          # kv updated in place
    y, kv = prefill_normed(q, k, v, cu_seqlens, decay, weight, eps, gate)  # fused output norm
    y = decode_normed(q, k, v, kv, decay, weight, eps, gate)
    o = decode_pool(q, k, v, pool, slots, decay)   # pool[slots] updated in place
    o = prefill_pool(q, k, v, cu_seqlens, decay, pool, slots)   # continues from pool[slots]
    s = cu_masked_stream(mask)   # a stream restricted to some compute units (two-stream serving)
    n, order = kernel_plan(cu_seqlens, num_heads)   # which prefill kernels a call would run
    o, kv = attention(q, k, v, cu_seqlens, decay, kv_init)   # differentiable (torch autograd)
"""

from ._binding import (  # noqa: F401
    LAError,
    LaNorm,
    LA_OK,
    LA_ERR_INVALID_ARG,
    LA_ERR_UNSUPPORTED,
    LA_ERR_HIP,
    LA_BF16,
    LA_FP32,
    LA_MAX_HEADS,
    lib,
    lib_path,
    cu_masked_stream,
    la_prefill,
    la_prefill_kernel_plan,
    la_prefill_segmented,
    la_prefill_segmented_noalloc,
    la_prefill_segmented_workspace_size,
    la_prefill_backward,
    la_prefill_backward_workspace_size,
    la_prefill_backward_segmented,
    la_prefill_backward_segmented_workspace_size,
    la_decode,
    la_decode_normed,
    la_prefill_normed,
    la_prefill_normed_workspace_size,
    la_decode_pool,
    la_prefill_pool,
    la_status_str,
    la_last_error,
    prefill,
    kernel_plan,
    prefill_segmented,
    prefill_segmented_noalloc,
    prefill_segmented_workspace_size,
    prefill_backward,
    prefill_backward_segmented,
    prefill_backward_segmented_workspace_size,
    decode,
    decode_normed,
    prefill_normed,
    prefill_normed_workspace_size,
    decode_pool,
    prefill_pool,
    attention,
)
