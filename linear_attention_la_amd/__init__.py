"""Lightning Attention prefill and decode for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libla.so`` (include/la.h).  It only
marshals arguments: torch supplies device memory and streams, every step of
the computation runs in the HIP kernels.  There is no CPU fallback: if the
library is missing, every call raises.

    o, kv = prefill(q, k, v, cu_seqlens, decay, kv_init=None, out_dtype=None)
    o, kv = prefill_segmented(q, k, v, cu_seqlens, decay, segment_len)
    dq, dk, dv, dkv0 = prefill_backward(q, k, v, do, cu_seqlens, decay, kv_init, dkv_final)
    o = decode(q, k, v, kv, decay)          # kv updated in place
    o = decode_pool(q, k, v, pool, slots, decay)   # pool[slots] updated in place
    o = prefill_pool(q, k, v, cu_seqlens, decay, pool, slots)   # continues from pool[slots]
"""

from ._binding import (  # noqa: F401
    LAError,
    LA_OK,
    LA_ERR_INVALID_ARG,
    LA_ERR_UNSUPPORTED,
    LA_ERR_HIP,
    LA_BF16,
    LA_FP32,
    LA_MAX_HEADS,
    lib,
    lib_path,
    la_prefill,
    la_prefill_segmented,
    la_prefill_segmented_workspace_size,
    la_prefill_backward,
    la_prefill_backward_workspace_size,
    la_prefill_backward_segmented,
    la_prefill_backward_segmented_workspace_size,
    la_decode,
    la_decode_pool,
    la_prefill_pool,
    la_status_str,
    la_last_error,
    prefill,
    prefill_segmented,
    prefill_segmented_workspace_size,
    prefill_backward,
    prefill_backward_segmented,
    prefill_backward_segmented_workspace_size,
    decode,
    decode_pool,
    prefill_pool,
)
