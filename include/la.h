/*
 * la.h -- C ABI of libla: Lightning Attention prefill and decode for AMD
 * MI355X (gfx950).
 *
 * What is computed.  Lightning Attention is causal linear attention in which
 * an element-wise product takes the place of softmax (emonzhong.com,
 * "MiniMax-01: Scaling Foundation Models with Lightning Attention", section
 * 方法要点), evaluated with the right-product kernel trick and split into
 * intra-block and inter-block work so that the cumsum of causal linear
 * attention is avoided (CSDN, "【AI论文】MiniMax-01:利用闪电注意力机制扩展基础
 * 模型", §2.1; jvyan.cn news article, 一、模型架构; mizuki blog,
 * "MiniMax-01：4M 上下文破局", 关键概念清单).  The pages print no formula.
 * This library reads the element-wise product as a causal decay mask: for
 * one sequence and one head h with decay lambda = decay[h],
 *
 *     S_t = lambda * S_{t-1} + k_t^T v_t,     o_t = q_t S_t,
 *
 * i.e. O = [(Q K^T) .* M] V + diag(lambda^(t+1)) Q S_init with
 * M[t][j] = lambda^(t-j) for t >= j and 0 otherwise, and the final state
 * S_L = lambda^L S_init + sum_j lambda^(L-1-j) k_j^T v_j.  There is no
 * softmax, no 1/sqrt(d) scale and no normaliser in this core.  The state
 * S is d x d, rows indexed by the key dimension r and columns by the value
 * dimension c.
 *
 * Layouts.  q, k, v, o are contiguous [T, H, d] (token-major): element
 * (t, h, c) sits at ((int64)t * H + h) * d + c.  Sequences are packed along
 * the token axis (data packing, CSDN §3.2; jvyan.cn 二、计算优化) and
 * delimited by cu_seqlens[S+1] (cu[0] = 0, cu[S] = T, non-decreasing).
 * States are contiguous fp32 [S, H, d, d]; element (s, h, r, c) sits at
 * (((int64)s * H + h) * d + r) * d + c.
 *
 * Ownership.  The caller allocates and owns every buffer.  The library
 * allocates no device memory, keeps no pointer after a call returns and
 * holds no global state (apart from the static device scratch of
 * la_prefill_segmented_noalloc and per-device caches of the compute-unit
 * count and that scratch's address); calls on different streams with
 * disjoint outputs may run concurrently (la_prefill_segmented_noalloc
 * excepted).  Which kernels run -- and so the last bits of the results, all
 * within the same tolerance -- depends on the arguments, the device's
 * compute-unit count and the LA_NDV sweep override (see la_prefill); given
 * those, every call is deterministic.  Work is enqueued on `stream` (a
 * hipStream_t passed as void*, NULL = the default stream) and is
 * asynchronous: device buffers must stay valid until the stream has passed
 * the kernel.  Host arrays
 * (decay, cu_seqlens_host) are read only during the call.  The device that
 * owns the buffers must be the calling thread's current HIP device.
 *
 * Alignment.  Every device pointer must be 16-byte aligned (the kernels use
 * 16 B vector accesses); a misaligned pointer is LA_ERR_INVALID_ARG.
 *
 * Errors.  Every entry point returns la_status and never aborts or prints.
 * Argument errors are detected on the host before anything is enqueued:
 * LA_ERR_INVALID_ARG, nothing runs, outputs are untouched.  Valid but
 * unsupported shapes or dtypes: LA_ERR_UNSUPPORTED.  A failed kernel launch:
 * LA_ERR_HIP.  A fault inside a kernel surfaces at the caller's next
 * synchronisation; the library never synchronises.  la_last_error() gives a
 * thread-local description of the last non-OK return.
 */
#ifndef LA_H_
#define LA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are int-sized.  A C caller may pass any int where one is
 * expected (unknown values are rejected); in C++ the enums take int32_t as
 * their underlying type, so that every such value is a valid value of the
 * type and the library's checks of it are well defined. */
#ifdef __cplusplus
#define LA_ENUM_BASE : int32_t
#else
#define LA_ENUM_BASE
#endif

typedef enum la_status LA_ENUM_BASE {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = 1,
  LA_ERR_UNSUPPORTED = 2,
  LA_ERR_HIP = 3
} la_status;

typedef enum la_dtype LA_ENUM_BASE { LA_BF16 = 0, LA_FP32 = 1 } la_dtype;

/* Largest number of heads one call accepts (per-head decay travels in the
 * kernel arguments). */
#define LA_MAX_HEADS 256

/*
 * la_prefill -- blockwise causal linear attention with per-head decay over
 * packed variable-length sequences; writes O and the final state.
 *
 * Follows the intra-block / inter-block split (emonzhong.com 方法要点;
 * mizuki blog 关键概念清单: intra-block left product, inter-block right
 * product) over packed sequences (CSDN §3.2).  Blocks never straddle two
 * sequences; each (sequence, head) pair is an independent chain.
 *
 *   q, k, v          device, [T, H, d] of in_dtype (not written).
 *   cu_seqlens_dev   device int32 [S+1]; same contents as cu_seqlens_host.
 *   cu_seqlens_host  host int32 [S+1]; validated (cu[0] = 0, non-decreasing,
 *                    cu[S] = T) and used for scheduling.
 *   num_seqs         S >= 0.  S = 0 is a no-op returning LA_OK.
 *   total_tokens     T >= 0, < 2^31.
 *   num_heads        H in [1, LA_MAX_HEADS].
 *   head_dim         d: 64 or 128 (d_k = d_v = d).
 *   in_dtype         LA_BF16 or LA_FP32.
 *   out_dtype        dtype of o: LA_BF16 or LA_FP32 (bf16 output needs bf16
 *                    input).  fp32 results are rounded to bf16 with
 *                    round-to-nearest-even.
 *   decay            host float [H], 0 < decay[h] <= 1 (1 = no decay).
 *   kv_init          device fp32 [S, H, d, d] initial states, or NULL for
 *                    zero states.
 *   o                device [T, H, d] of out_dtype (written); must not
 *                    overlap q, k, v, kv_init or kv_final.
 *   kv_final         device fp32 [S, H, d, d] final states (written), or
 *                    NULL to skip.  May be exactly kv_init (in-place
 *                    continuation); any other overlap with an input is an
 *                    error.
 *   stream           hipStream_t or NULL.
 *
 * Zero-length sequences produce no rows; their final state is kv_init's (or
 * zero).
 *
 * Kernels: bf16 inputs with d = 128 and more (sequence, head) pairs than
 * half the compute units of the current device run one workgroup per pair
 * (each input row is read once); otherwise each pair is split by value
 * columns over d / 32 workgroups (with at most half as many pairs as
 * compute units these fill the GPU in two waves of workgroups, the faster
 * choice there).  When the pairs fill whole waves of the first kind plus a
 * remainder of at most half the compute units, and a model of the two plans
 * finds it faster, the sequences of the remainder run in 32-column slices
 * in a second launch on the stream instead of an extra wave.  Both kernels
 * give results within the same tolerance, not bitwise equal to each other;
 * each sequence's results come from one kernel, and a given call is
 * deterministic.
 * A one-workgroup-per-pair launch occupies whole compute units, so work on
 * another stream gets fewer of them while it runs.  Calls of 2 to 512
 * sequences hand the sequences to the grid longest first (read from
 * cu_seqlens_host), so that when the grid runs in several waves of
 * workgroups the longest chains start in the first.  With fewer than about
 * a quarter as many (sequence, head) pairs as compute units (e.g. a few
 * heads of one long sequence), most compute units stay idle: there
 * la_prefill_segmented, which cuts the sequences into parallel segments, is
 * several times faster (it needs a workspace, which la_prefill does not).
 *
 * Sweep override (bf16 inputs): the environment variable LA_NDV, read on
 * every call that has sequences, forces one kernel for every pair -- "1"
 * one workgroup per pair (d = 128 only), "4" (d = 128) or "2" (d = 64) the
 * 32-column slices.  Unset or empty: the choice above.  Any other value is
 * LA_ERR_UNSUPPORTED (after the argument checks, before anything is
 * enqueued).  The block length is not an option: both kernels tile by 64
 * tokens.
 */
la_status la_prefill(const void* q, const void* k, const void* v,
                     const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                     int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                     int32_t head_dim, la_dtype in_dtype, la_dtype out_dtype,
                     const float* decay, const float* kv_init, void* o, float* kv_final,
                     void* stream);

/*
 * la_prefill_pool -- la_prefill whose states live in a state pool: sequence
 * s starts from kv_pool[slots[s]] and its final state is written back to the
 * same slot.  A server keeps the states of all live sequences in one pool,
 * prefills new chunks of any of them (continuing from the pooled state) and
 * decodes them with la_decode_pool, with no copy between the two (the
 * serving engine's length > 1 path beside its length-1 path, jvyan.cn
 * 二、计算优化; CSDN §3.2).
 *
 *   kv_pool      device fp32 [pool_size, H, d, d], read and written in place;
 *                entries no slot names are not touched.  A sequence that
 *                starts from scratch needs its slot zeroed first.
 *   pool_size    number of states in the pool (>= 0).
 *   slots_dev    device int32 [S]: pool index of sequence s.
 *   slots_host   host int32 [S], same contents; validated before any launch:
 *                every slot in [0, pool_size) and no slot twice.
 *   q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
 *   num_heads, head_dim, out_dtype, decay, o, stream: as in la_prefill;
 *                in_dtype must be LA_BF16; o must not overlap the pool and
 *                the pool must not overlap q, k or v.
 *
 * A zero-length sequence leaves its slot unchanged.  Kernels, and the
 * LA_NDV override, as in la_prefill.  Errors as la_prefill, plus
 * LA_ERR_INVALID_ARG for a NULL pool or slot array, a slot out of range or a
 * repeated slot, and LA_ERR_UNSUPPORTED for fp32 inputs.  Repeated slots are
 * found on a sorted host copy of slots_host (S entries, whatever pool_size);
 * if it cannot be allocated the call returns LA_ERR_UNSUPPORTED.
 */
la_status la_prefill_pool(const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                          int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                          int32_t head_dim, la_dtype in_dtype, la_dtype out_dtype,
                          const float* decay, float* kv_pool, int32_t pool_size,
                          const int32_t* slots_dev, const int32_t* slots_host, void* o,
                          void* stream);

/*
 * la_prefill_kernel_plan -- the kernels la_prefill and la_prefill_pool would
 * run for a call with bf16 inputs and these sequences and heads (see
 * "Kernels" at la_prefill).  Host only: nothing is enqueued and no device
 * memory is touched.
 *
 *   num_seqs, cu_seqlens_host, num_heads, head_dim: as in la_prefill.
 *   compute_units  compute units of the device to plan for (e.g. 256 for
 *                  MI355X), or 0 for the current device.
 *   wide_seqs      host int32, receives the number of leading sequences, in
 *                  dispatch order, that run one workgroup per (sequence,
 *                  head); the others run in 32-column slices (in a second
 *                  launch when both kinds occur).  0: every sequence in
 *                  slices; num_seqs: every sequence one workgroup per pair.
 *   order          NULL, or host int32 [num_seqs], receives the dispatch
 *                  order (longest first for 2 to 512 sequences, else the
 *                  index order).
 *
 * LA_NDV is applied as in la_prefill.  Errors: LA_ERR_INVALID_ARG (NULL
 * wide_seqs or cu_seqlens_host, num_seqs or compute_units < 0, bad
 * cu_seqlens), LA_ERR_UNSUPPORTED (num_heads or head_dim as in la_prefill, an
 * LA_NDV value la_prefill rejects, or compute_units 0 with no device).
 */
la_status la_prefill_kernel_plan(int32_t num_seqs, const int32_t* cu_seqlens_host,
                                 int32_t num_heads, int32_t head_dim, int32_t compute_units,
                                 int32_t* wide_seqs, int32_t* order);

/*
 * la_prefill_segmented -- la_prefill with every sequence cut into segments of
 * segment_len tokens that run as parallel chains; same results (up to the
 * order of fp32 sums) and the same arguments, plus:
 *
 *   segment_len      tokens per segment, a positive multiple of 64; the last
 *                    segment of a sequence may be shorter.  A sequence of L
 *                    tokens gives max(1, ceil(L / segment_len)) segments.
 *                    0: the library's choice, about one (segment, head) item
 *                    per compute unit of the current device (256 without
 *                    one): ceil(T x num_heads / CUs) rounded up to a
 *                    multiple of 64 -- the length that first fills the
 *                    compute units, which measured fastest.
 *   workspace        device scratch of at least the size that
 *                    la_prefill_segmented_workspace_size reports for the same
 *                    num_seqs, cu_seqlens_host, num_heads, head_dim and
 *                    segment_len; 16-byte aligned; overlaps no other buffer;
 *                    contents on entry are ignored and on return undefined.
 *   workspace_bytes  its size.
 *
 * It raises the number of workgroups when few (sequence, head) pairs exist.
 * The segment states are found without any exchange beyond the device: the
 * local decayed state of each segment (a state-only pass over K and V) is
 * chained in order, S_(i+1) = lambda^(len_i) S_i + Shat_i, which is the
 * local-prefix-sum step of the LASP+ sequence split (mizuki blog
 * "MiniMax-01：4M 上下文破局", 五) done on one device; then each segment runs
 * the prefill from its start state.  K and V are read twice.  in_dtype must
 * be LA_BF16 (LA_FP32 is LA_ERR_UNSUPPORTED).  Errors as la_prefill, plus
 * LA_ERR_INVALID_ARG for a bad segment_len or a NULL, misaligned, short or
 * overlapping workspace.  Nothing synchronises.
 *
 * d = 128: two kernels are enqueued on `stream` -- a one-workgroup plan, then
 * one launch in which every (segment, head) item computes its segment's local
 * state, receives the state entering the segment from the item of the
 * previous segment of its sequence (through the workspace, at device scope),
 * passes the state entering the next segment on, and writes its outputs.
 * An item only ever waits for an item that has already started, so the
 * launch always completes.  Each wait is also bounded (a poll count that
 * grows with the segment length and the segment count, far beyond what a
 * correct run needs); a wait that reached it would end the remaining waits
 * at once and leave the outputs undefined -- it exists so that a fault
 * cannot hang the GPU, and no correct call reaches it.  The workspace holds
 * 2 states per (sequence, head) whatever the segment count.  d = 64: four
 * kernels (plan, a state-only pass over all segments, the prefix over them,
 * the output pass); the workspace holds one state per segment and per
 * sequence.
 */
la_status la_prefill_segmented(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                               int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                               int32_t head_dim, la_dtype in_dtype, la_dtype out_dtype,
                               const float* decay, const float* kv_init, void* o,
                               float* kv_final, int32_t segment_len, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Size in bytes of the static device scratch of
 * la_prefill_segmented_noalloc (each device the library runs on holds one
 * such array until the process ends). */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * la_prefill_segmented_noalloc -- la_prefill_segmented without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * calls no hipMalloc, hipFree or allocating library routine: the workspace
 * is a static device array of LA_NOALLOC_SCRATCH_BYTES bytes (64 MiB) that
 * the library holds on every device it runs on; its device address is
 * looked up once per device (hipGetSymbolAddress) on the first call there.
 *
 * Arguments, results and errors as la_prefill_segmented, without workspace
 * and workspace_bytes.  A call whose workspace
 * (la_prefill_segmented_workspace_size) would exceed the scratch returns
 * LA_ERR_UNSUPPORTED before anything is enqueued; with d = 128 the scratch
 * holds up to 511 (sequence, head) pairs whatever the segment count (e.g.
 * 7 sequences of 64 heads), with d = 64 up to about 4000 (segment or
 * sequence, head) pairs.  Failing to look up the scratch address is
 * LA_ERR_HIP.
 *
 * Every call on one device shares that device's scratch, which keeps the
 * last call's contents (nothing in it needs to start at zero).  Calls that
 * overlap in time on one device -- on different streams, or from different
 * host threads -- race on the scratch and give undefined results; calls on
 * one stream are ordered by the stream and are safe.
 */
la_status la_prefill_segmented_noalloc(const void* q, const void* k, const void* v,
                                       const int32_t* cu_seqlens_dev,
                                       const int32_t* cu_seqlens_host, int32_t num_seqs,
                                       int64_t total_tokens, int32_t num_heads,
                                       int32_t head_dim, la_dtype in_dtype, la_dtype out_dtype,
                                       const float* decay, const float* kv_init, void* o,
                                       float* kv_final, int32_t segment_len, void* stream);

/*
 * la_prefill_segmented_workspace_size -- bytes of workspace that
 * la_prefill_segmented needs for these arguments (host only, no device
 * call apart from reading the current device's compute-unit count when
 * segment_len is 0).  *bytes is 0 on error.  Errors: LA_ERR_INVALID_ARG
 * (NULL bytes or cu_seqlens_host, bad cu_seqlens, num_seqs < 0, bad
 * segment_len),
 * LA_ERR_UNSUPPORTED (heads or head_dim as la_prefill, too many segments).
 */
la_status la_prefill_segmented_workspace_size(int32_t num_seqs, const int32_t* cu_seqlens_host,
                                              int32_t num_heads, int32_t head_dim,
                                              int32_t segment_len, size_t* bytes);

/*
 * la_prefill_backward -- gradients of la_prefill with respect to q, k, v and
 * the initial state, for upstream gradients d_o of the output and dkv_final
 * of the final state.
 *
 * The pages give only the forward; differentiating the causal decayed form
 * (see the top of this header) gives, per sequence and head, with
 * M[t][j] = lambda^(t-j) for t >= j and 0 otherwise:
 *     dQ  = [(dO V^T) .* M] K   + diag(lambda^(t+1)) dO S_init^T
 *     dK  = [(dO V^T) .* M]^T Q + diag(lambda^(L-1-j)) V dS_L^T
 *     dV  = [(Q K^T) .* M]^T dO + diag(lambda^(L-1-j)) K dS_L
 *     dS_init = Q^T diag(lambda^(t+1)) dO + lambda^L dS_L
 * dQ is the blockwise forward chain with dO, V, K in the roles of Q, K, V;
 * dK and dV are the same chain run backwards in time (a reverse-direction
 * state), in the intra-block / inter-block split of the forward (emonzhong.com
 * 方法要点; mizuki blog 关键概念清单).
 *
 *   q, k, v, d_o     device [T, H, d], bf16 (in_dtype must be LA_BF16).
 *   cu_seqlens_dev/host, num_seqs, total_tokens, num_heads, head_dim, decay:
 *                    as in la_prefill (the forward's arguments).
 *   grad_dtype       dtype of dq, dk, dv: LA_BF16 (RNE) or LA_FP32.
 *   kv_init          device fp32 [S, H, d, d] initial states of the forward,
 *                    or NULL (zero).
 *   dkv_final        device fp32 [S, H, d, d] gradient of the final states,
 *                    or NULL (zero).  Needs every decay >= 2^-64
 *                    (else LA_ERR_UNSUPPORTED).
 *   dq, dk, dv       device [T, H, d] of grad_dtype (written).
 *   dkv_init         device fp32 [S, H, d, d] gradient of the initial states
 *                    (written), or NULL to skip.
 *   workspace        device scratch of la_prefill_backward_workspace_size
 *                    bytes, needed when kv_init or dkv_final is given (may be
 *                    NULL otherwise); 16-byte aligned.  Only d = 64 writes
 *                    it; the size contract is the same for both d.
 *
 * The outputs and the workspace may overlap nothing else.  Errors as
 * la_prefill.  Nothing synchronises.  d = 128: one kernel is enqueued on
 * `stream`, running the three chains side by side (one workgroup per
 * (chain, sequence, head)) and reading kv_init and dkv_final directly.
 * d = 64: up to seven kernels -- the three chains one after the other, each
 * on the kernel la_prefill would choose, with the states transposed and
 * scaled into the workspace between them.
 */
la_status la_prefill_backward(const void* q, const void* k, const void* v, const void* d_o,
                              const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                              int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                              int32_t head_dim, la_dtype in_dtype, la_dtype grad_dtype,
                              const float* decay, const float* kv_init, const float* dkv_final,
                              void* dq, void* dk, void* dv, float* dkv_init, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of workspace for la_prefill_backward: num_seqs x num_heads x d x d
 * fp32 (host only).  Errors: LA_ERR_INVALID_ARG (NULL bytes, num_seqs < 0),
 * LA_ERR_UNSUPPORTED (heads or head_dim as la_prefill). */
la_status la_prefill_backward_workspace_size(int32_t num_seqs, int32_t num_heads,
                                             int32_t head_dim, size_t* bytes);

/*
 * la_prefill_backward_segmented -- la_prefill_backward with every sequence
 * cut into segments of segment_len tokens, for few long sequences (few
 * (sequence, head) chains to spread over the GPU).
 *
 * Each of the backward's three chains (dQ forwards in time, dK and dV
 * backwards) runs as la_prefill_segmented runs its chain: every segment's
 * local state from a zero state, a prefix over the segments -- for the two
 * reverse-time chains from the last segment to the first -- then every
 * segment's outputs from the state at its start.  The one-exchange sequence
 * split of LASP+ (mizuki blog "MiniMax-01：4M 上下文破局", 五) applied to
 * the gradient chains.  The dV chain's states are the transposes of the dK
 * chain's, so only its output pass runs, from the dK chain's segment start
 * states read transposed; at d = 128, with more (segment, head) pairs than
 * half the compute units, the dK and dV output passes run side by side in
 * one launch.  The same result as la_prefill_backward up to the order of
 * fp32 sums.
 *
 * Arguments as la_prefill_backward, except:
 *   segment_len      tokens per segment, a positive multiple of 64, or 0
 *                    for the library's choice (as in la_prefill_segmented).
 *   workspace        device scratch of at least
 *                    la_prefill_backward_segmented_workspace_size bytes
 *                    (always needed), 16-byte aligned, overlapping no other
 *                    argument.
 * Errors as la_prefill_backward (LA_ERR_INVALID_ARG also for a bad
 * segment_len).  Up to sixteen kernels are enqueued on `stream`; nothing
 * synchronises.
 */
la_status la_prefill_backward_segmented(
    const void* q, const void* k, const void* v, const void* d_o, const int32_t* cu_seqlens_dev,
    const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
    int32_t head_dim, la_dtype in_dtype, la_dtype grad_dtype, const float* decay,
    const float* kv_init, const float* dkv_final, void* dq, void* dk, void* dv, float* dkv_init,
    int32_t segment_len, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace for la_prefill_backward_segmented (host only): the
 * segment plan and states of la_prefill_segmented_workspace_size plus one
 * set of S x H x d x d fp32 states.  Errors as
 * la_prefill_segmented_workspace_size. */
la_status la_prefill_backward_segmented_workspace_size(int32_t num_seqs,
                                                       const int32_t* cu_seqlens_host,
                                                       int32_t num_heads, int32_t head_dim,
                                                       int32_t segment_len, size_t* bytes);

/*
 * la_decode -- one decode token per sequence, updating fp32 states in place.
 *
 * The length-1 step that serving runs in its own kernel, apart from the
 * length > 1 prefill, so that both can run on two streams in parallel
 * (jvyan.cn 二、计算优化; CSDN §3.2).  For every (b, h):
 *     kv[b,h] <- decay[h] * kv[b,h] + k[b,h]^T v[b,h]      (update first)
 *     o[b,h]  <- q[b,h] kv[b,h]                            (then read out)
 *
 *   q, k, v    device [B, H, d] of in_dtype (not written).
 *   kv         device fp32 [B, H, d, d], read and written in place.
 *   decay      host float [H], 0 < decay[h] <= 1.
 *   batch      B >= 0 (0 is a no-op).
 *   num_heads  H in [1, LA_MAX_HEADS].
 *   head_dim   d: 64 or 128.
 *   in_dtype   LA_BF16 or LA_FP32; o has the same dtype (bf16 rounded to
 *              nearest-even).
 *   o          device [B, H, d] (written); must not overlap q, k, v or kv.
 *   stream     hipStream_t or NULL.
 */
la_status la_decode(const void* q, const void* k, const void* v, float* kv,
                    const float* decay, int32_t batch, int32_t num_heads, int32_t head_dim,
                    la_dtype in_dtype, void* o, void* stream);

/*
 * la_decode_pool -- la_decode on a state pool: sequence b reads and updates
 * state kv_pool[slots[b]], so a server can keep the states of all live
 * sequences in one pool and decode any subset of them in one launch (the
 * serving engine's length-1 path, jvyan.cn 二、计算优化; CSDN §3.2).
 *
 *   kv_pool     device fp32 [pool_size, H, d, d], read and written in place;
 *               entries no slot names are not touched.
 *   pool_size   number of states in the pool (>= 0).
 *   slots_dev   device int32 [batch]: pool index of sequence b.
 *   slots_host  host int32 [batch], same contents; validated before any
 *               launch: every slot in [0, pool_size) and no slot twice.
 *   q, k, v, o, decay, batch, num_heads, head_dim, in_dtype, stream: as in
 *               la_decode; o must not overlap the pool.
 *
 * Errors as la_decode, plus LA_ERR_INVALID_ARG for a NULL slot array, a slot
 * out of range or a repeated slot.  Repeated slots are found on a sorted host
 * copy of slots_host (batch entries, whatever pool_size); if it cannot be
 * allocated the call returns LA_ERR_UNSUPPORTED.
 */
la_status la_decode_pool(const void* q, const void* k, const void* v, float* kv_pool,
                         int32_t pool_size, const int32_t* slots_dev, const int32_t* slots_host,
                         const float* decay, int32_t batch, int32_t num_heads, int32_t head_dim,
                         la_dtype in_dtype, void* o, void* stream);

/*
 * la_norm -- the output normalisation that la_prefill_normed and
 * la_decode_normed fuse into the kernels that write O.
 *
 * The pages say the model uses TransNormer's NormAttention, a normalisation
 * of the linear-attention output (CSDN §2.1), and that the memory-bound
 * kernels around lightning attention are fused so that intermediate results
 * are not stored (jvyan.cn 二、计算优化; CSDN §3.2: batched kernel fusion).
 * They do not define the normalisation; this library reads it as an RMS
 * normalisation of each head's output row over its d features:
 *
 *     y[t,h,:] = weight[h,:] * o[t,h,:] / sqrt(mean_c(o[t,h,c]^2) + eps)
 *                * sigmoid(gate[t,h,:])            (if gate is given)
 *
 * where o is the attention output of la_prefill / la_decode, computed in
 * fp32 and normalised before its only rounding to the output dtype.  The
 * gate is not on the pages; it is an option for a caller whose layer gates
 * the attention output.
 *
 *   weight   device fp32 [H, d] (16-byte aligned).
 *   eps      added to each row's mean square; finite and > 0.
 *   gate     device [T, H, d] (prefill) or [B, H, d] (decode), the layout and
 *            dtype of q, 16-byte aligned; or NULL (no gate).
 */
typedef struct la_norm {
  const float* weight;
  float eps;
  const void* gate;
} la_norm;

/*
 * la_prefill_normed -- la_prefill with the output normalisation of *norm
 * applied to every output row before it is written: o receives y (see
 * la_norm), the final states are those of la_prefill.  One pass; the
 * unnormalised O never reaches memory.
 *
 * Arguments as la_prefill, plus norm, workspace and workspace_bytes.
 * in_dtype must be LA_BF16 and head_dim 128 (else LA_ERR_UNSUPPORTED).
 * With more (sequence, head) pairs than half the compute units of the
 * current device, one workgroup per pair runs the chain (as la_prefill).
 * With fewer, the sequences are cut into segments (as la_prefill_segmented's
 * chained scan, with a segment length the library chooses so that segments
 * x heads reaches the compute units).  When the pairs past whole waves of
 * the first kind fill at most half the compute units and their sequences
 * are consecutive, those sequences may run through the chained scan after
 * the wave (as la_prefill's split, decided by a model of both plans).  The
 * scan needs a workspace of la_prefill_normed_workspace_size bytes (16-byte
 * aligned, overlapping no other buffer; contents ignored and left
 * undefined); when that size is 0 the workspace is unused (may be NULL).
 * o must not overlap the weight or the gate.  Errors as la_prefill, plus
 * LA_ERR_INVALID_ARG for a NULL norm or weight, a bad eps,
 * a misaligned or overlapping weight or gate, or a missing or short
 * workspace.  Nothing synchronises.
 */
la_status la_prefill_normed(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                            int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                            int32_t head_dim, la_dtype in_dtype, la_dtype out_dtype,
                            const float* decay, const float* kv_init, const la_norm* norm,
                            void* o, float* kv_final, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Bytes of workspace la_prefill_normed needs for these sequences and heads
 * on the current device: 0 when every (sequence, head) pair runs one
 * workgroup each, else the chained scan's workspace for the sequences it
 * takes.  The plan is the call's own, so the size is exact for it.  Host
 * only apart from reading the device's compute-unit count.  Errors as
 * la_prefill_segmented_workspace_size. */
la_status la_prefill_normed_workspace_size(int32_t num_seqs, const int32_t* cu_seqlens_host,
                                           int32_t num_heads, int32_t head_dim, size_t* bytes);

/*
 * la_decode_normed -- la_decode with the output normalisation of *norm
 * (la_norm) applied to o before it is written; the states are updated as
 * by la_decode.  Arguments as la_decode plus norm (gate: [B, H, d] of
 * in_dtype, or NULL).  Errors as la_decode, plus LA_ERR_INVALID_ARG for a
 * NULL norm or weight, a bad eps, or a misaligned or overlapping weight or
 * gate.
 */
la_status la_decode_normed(const void* q, const void* k, const void* v, float* kv,
                           const float* decay, int32_t batch, int32_t num_heads, int32_t head_dim,
                           la_dtype in_dtype, const la_norm* norm, void* o, void* stream);

/* Static, never-NULL name of a status code. */
const char* la_status_str(la_status s);

/* Thread-local description of the last non-OK return on this thread
 * ("" if none).  Valid until the next library call on the same thread. */
const char* la_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_H_ */
