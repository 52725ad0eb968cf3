// Host side of the libla C ABI: argument validation, per-head decay
// preprocessing and kernel dispatch.  Every argument error is found here,
// before anything is enqueued; the library never synchronises and allocates
// no device memory.

#include <math.h>
#include <algorithm>
#include <atomic>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "la.h"
#include "la_backward.h"
#include "la_internal.h"

namespace {

thread_local char g_err[512] = "";

la_status fail(la_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

la_status ok() {
  g_err[0] = '\0';
  return LA_OK;
}

bool valid_dtype(la_dtype d) { return d == LA_BF16 || d == LA_FP32; }
// Kernels use 16 B vector loads and stores at row granularity.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t dtype_size(la_dtype d) { return d == LA_BF16 ? 2 : 4; }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

Range range(const char* name, const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + bytes : lo};
}

la_status check_decay(const float* decay, int32_t num_heads) {
  if (!decay) return fail(LA_ERR_INVALID_ARG, "decay is NULL");
  for (int32_t h = 0; h < num_heads; ++h) {
    const float x = decay[h];
    if (!(x > 0.0f && x <= 1.0f))
      return fail(LA_ERR_INVALID_ARG, "decay[%d] = %g is outside (0, 1]", h, (double)x);
  }
  return LA_OK;
}

la_status check_heads_dim(int32_t num_heads, int32_t head_dim) {
  if (num_heads < 1) return fail(LA_ERR_INVALID_ARG, "num_heads = %d < 1", num_heads);
  if (num_heads > LA_MAX_HEADS)
    return fail(LA_ERR_UNSUPPORTED, "num_heads = %d exceeds %d", num_heads, LA_MAX_HEADS);
  if (head_dim < 1) return fail(LA_ERR_INVALID_ARG, "head_dim = %d < 1", head_dim);
  if (head_dim != 64 && head_dim != 128)
    return fail(LA_ERR_UNSUPPORTED, "head_dim = %d (supported: 64, 128)", head_dim);
  return LA_OK;
}

la_status check_cu(const int32_t* cu, int32_t num_seqs) {
  if (cu[0] != 0) return fail(LA_ERR_INVALID_ARG, "cu_seqlens[0] = %d, expected 0", cu[0]);
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (cu[s + 1] < cu[s])
      return fail(LA_ERR_INVALID_ARG, "cu_seqlens decreases at %d (%d -> %d)", s, cu[s], cu[s + 1]);
  }
  return LA_OK;
}

// Validation shared by la_prefill and la_prefill_segmented (everything
// except the workspace).  Returns LA_OK for num_seqs == 0 after checking the
// scalar arguments.
la_status check_prefill(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                        int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                        int32_t head_dim, la_dtype in_dtype, la_dtype out_dtype,
                        const float* decay, const float* kv_init, const void* o,
                        const float* kv_final, int32_t items_seqs) {
  if (num_seqs < 0) return fail(LA_ERR_INVALID_ARG, "num_seqs = %d < 0", num_seqs);
  if (total_tokens < 0)
    return fail(LA_ERR_INVALID_ARG, "total_tokens = %lld < 0", (long long)total_tokens);
  if (total_tokens >= (int64_t)1 << 31)
    return fail(LA_ERR_INVALID_ARG, "total_tokens = %lld does not fit int32 cu_seqlens",
                (long long)total_tokens);
  la_status st = check_heads_dim(num_heads, head_dim);
  if (st != LA_OK) return st;
  if (!valid_dtype(in_dtype)) return fail(LA_ERR_INVALID_ARG, "in_dtype = %d", (int)in_dtype);
  if (!valid_dtype(out_dtype)) return fail(LA_ERR_INVALID_ARG, "out_dtype = %d", (int)out_dtype);
  if (in_dtype == LA_FP32 && out_dtype == LA_BF16)
    return fail(LA_ERR_UNSUPPORTED, "fp32 input with bf16 output is not supported");
  if ((st = check_decay(decay, num_heads)) != LA_OK) return st;
  if (!cu_seqlens_host) return fail(LA_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
  if ((st = check_cu(cu_seqlens_host, num_seqs)) != LA_OK) return st;
  if ((int64_t)cu_seqlens_host[num_seqs] != total_tokens)
    return fail(LA_ERR_INVALID_ARG, "cu_seqlens[%d] = %d != total_tokens = %lld", num_seqs,
                cu_seqlens_host[num_seqs], (long long)total_tokens);
  if (num_seqs == 0) return ok();
  if (!cu_seqlens_dev) return fail(LA_ERR_INVALID_ARG, "cu_seqlens_dev is NULL");
  if (total_tokens > 0 && (!q || !k || !v || !o))
    return fail(LA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL when total_tokens > 0");

  const void* ptrs[] = {q, k, v, o, kv_init, kv_final};
  const char* names[] = {"q", "k", "v", "o", "kv_init", "kv_final"};
  for (int i = 0; i < 6; ++i)
    if (!aligned16(ptrs[i]))
      return fail(LA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);

  const int cols = in_dtype == LA_BF16 ? la::kBf16Cols : la::kF32Cols;
  const int64_t items = (int64_t)items_seqs * num_heads * (head_dim / cols);
  if (items >= ((int64_t)1 << 31))
    return fail(LA_ERR_UNSUPPORTED, "%lld work items exceed the grid limit", (long long)items);

  // Aliasing: o and kv_final are written; they may overlap no input, except
  // that kv_final may be exactly kv_init.
  const size_t tok_bytes = (size_t)total_tokens * num_heads * head_dim;
  const size_t state_bytes = (size_t)num_seqs * num_heads * head_dim * head_dim * 4;
  const Range rq = range("q", q, tok_bytes * dtype_size(in_dtype));
  const Range rk = range("k", k, tok_bytes * dtype_size(in_dtype));
  const Range rv = range("v", v, tok_bytes * dtype_size(in_dtype));
  const Range ro = range("o", o, tok_bytes * dtype_size(out_dtype));
  const Range ri = range("kv_init", kv_init, kv_init ? state_bytes : 0);
  const Range rf = range("kv_final", kv_final, kv_final ? state_bytes : 0);
  const Range* ins[] = {&rq, &rk, &rv, &ri};
  for (const Range* in : ins) {
    if (overlap(ro, *in)) return fail(LA_ERR_INVALID_ARG, "o overlaps %s", in->name);
    if (in == &ri && kv_init == kv_final) continue;
    if (overlap(rf, *in)) return fail(LA_ERR_INVALID_ARG, "kv_final overlaps %s", in->name);
  }
  if (overlap(ro, rf)) return fail(LA_ERR_INVALID_ARG, "o overlaps kv_final");
  return LA_OK;
}

// Compute units of the current device (0 if unknown), cached per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The wide bf16 kernel (one workgroup per chain, d = 128) reads every input
// row once per chain instead of once per 32-column slice; it is chosen when
// there are at least as many chains as compute units, so that it fills the
// GPU.
bool use_wide(int64_t chains, int32_t head_dim) {
  const int cus = device_cus();
  return head_dim == 128 && cus > 0 && chains >= cus;
}

// Longest sequences first: a grid with more chains than compute units runs
// in waves of workgroups, and a long chain that starts in a late wave
// stretches the launch.  Ties keep the index order; batches of one
// sequence or more than kMaxOrder sequences keep the identity order.
void set_order(la::PrefillArgs& a, const int32_t* cu_host, int32_t num_seqs) {
  a.ordered = 0;
  if (num_seqs < 2 || num_seqs > la::kMaxOrder) return;
  std::vector<int> idx(num_seqs);
  for (int i = 0; i < num_seqs; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) {
    return cu_host[x + 1] - cu_host[x] > cu_host[y + 1] - cu_host[y];
  });
  for (int i = 0; i < num_seqs; ++i) {
    a.seq_order[i] = (uint16_t)idx[i];
    if (idx[i] != i) a.ordered = 1;
  }
}

// Stride for the decode's walk through the batch: about 0.618 * batch, made
// coprime to it so that i -> (i * step) % batch is a permutation.  Walking
// the states in this scattered order, rather than in index order, avoids
// the slow cases of streaming neighbouring states at once (median decode of
// 256 x 64 states: 362-365 us scattered vs 389-392 us in order).
int32_t batch_stride(int32_t batch) {
  if (batch < 3) return 1;
  int64_t step = (int64_t)((double)batch * 0.6180339887498949);
  auto gcd = [](int64_t x, int64_t y) {
    while (y) { const int64_t t = x % y; x = y; y = t; }
    return x;
  };
  while (gcd(step, batch) != 1) ++step;
  return (int32_t)step;
}

la_status check_segment_len(int32_t segment_len) {
  if (segment_len <= 0 || segment_len % 64 != 0)
    return fail(LA_ERR_INVALID_ARG, "segment_len = %d is not a positive multiple of 64",
                segment_len);
  return LA_OK;
}

// Byte offsets of the segmented-prefill workspace sections (each 256 B
// aligned): cu_seg [n+1], init_slot [n], final_slot [n], seq_first [S+1]
// (int32), then fp32 states [(n + S), H, d, d], n = number of segments.
struct SegmentLayout {
  int32_t num_segments;
  int32_t segment_len;
  size_t cu_seg, init_slot, final_slot, seq_first, states, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

la_status segment_layout(const int32_t* cu, int32_t num_seqs, int32_t num_heads,
                         int32_t head_dim, int32_t segment_len, SegmentLayout* lay) {
  int64_t n = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t len = (int64_t)cu[s + 1] - cu[s];
    n += len <= 0 ? 1 : (len + segment_len - 1) / segment_len;
  }
  if (n + num_seqs >= ((int64_t)1 << 31))
    return fail(LA_ERR_UNSUPPORTED, "%lld segments exceed the int32 range", (long long)n);
  lay->num_segments = (int32_t)n;
  lay->segment_len = segment_len;
  size_t off = 0;
  lay->cu_seg = off;
  off = align256(off + (size_t)(n + 1) * 4);
  lay->init_slot = off;
  off = align256(off + (size_t)n * 4);
  lay->final_slot = off;
  off = align256(off + (size_t)n * 4);
  lay->seq_first = off;
  off = align256(off + (size_t)(num_seqs + 1) * 4);
  lay->states = off;
  off += (size_t)(n + num_seqs) * num_heads * head_dim * head_dim * 4;
  lay->total = off;
  return LA_OK;
}

// Decode with num_states states in kv; sequence b uses state slots[b] (or b
// when slots is NULL).  The slot array has been validated by the caller.
la_status decode_common(const void* q, const void* k, const void* v, float* kv,
                        int32_t num_states, const int32_t* slots_dev, const int32_t* slots_host,
                        const float* decay, int32_t batch, int32_t num_heads, int32_t head_dim,
                        la_dtype in_dtype, void* o, void* stream);

la_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

la_status decode_common(const void* q, const void* k, const void* v, float* kv,
                        int32_t num_states, const int32_t* slots_dev, const int32_t* slots_host,
                        const float* decay, int32_t batch, int32_t num_heads, int32_t head_dim,
                        la_dtype in_dtype, void* o, void* stream) {
  (void)slots_host;
  if (batch < 0) return fail(LA_ERR_INVALID_ARG, "batch = %d < 0", batch);
  la_status st = check_heads_dim(num_heads, head_dim);
  if (st != LA_OK) return st;
  if (!valid_dtype(in_dtype)) return fail(LA_ERR_INVALID_ARG, "in_dtype = %d", (int)in_dtype);
  if ((st = check_decay(decay, num_heads)) != LA_OK) return st;
  if (batch == 0) return ok();
  if (!q || !k || !v || !kv || !o)
    return fail(LA_ERR_INVALID_ARG, "q, k, v, kv and o must be non-NULL");
  const void* ptrs[] = {q, k, v, kv, o};
  const char* names[] = {"q", "k", "v", "kv", "o"};
  for (int i = 0; i < 5; ++i)
    if (!aligned16(ptrs[i]))
      return fail(LA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  if ((int64_t)batch * num_heads >= ((int64_t)1 << 31))
    return fail(LA_ERR_UNSUPPORTED, "batch * num_heads exceeds the grid limit");

  const size_t vec_bytes = (size_t)batch * num_heads * head_dim * dtype_size(in_dtype);
  const Range rq = range("q", q, vec_bytes), rk = range("k", k, vec_bytes),
              rv = range("v", v, vec_bytes), ro = range("o", o, vec_bytes);
  const Range rs = range("kv", kv, (size_t)num_states * num_heads * head_dim * head_dim * 4);
  const Range* others[] = {&rq, &rk, &rv, &rs};
  for (const Range* x : others)
    if (overlap(ro, *x)) return fail(LA_ERR_INVALID_ARG, "o overlaps %s", x->name);
  const Range* vecs[] = {&rq, &rk, &rv};
  for (const Range* x : vecs)
    if (overlap(rs, *x)) return fail(LA_ERR_INVALID_ARG, "kv overlaps %s", x->name);

  la::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv = kv;
  a.slots = slots_dev;
  a.o = o;
  a.batch = batch;
  a.num_heads = num_heads;
  a.b_step = batch_stride(batch);
  for (int32_t h = 0; h < num_heads; ++h) a.decay[h] = decay[h];
  hipError_t e = la::launch_decode(a, head_dim, in_dtype, static_cast<hipStream_t>(stream));
  return hip_status(e, "la_decode launch");
}

}  // namespace

extern "C" {

const char* la_status_str(la_status s) {
  switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_HIP: return "LA_ERR_HIP";
  }
  return "LA_STATUS_UNKNOWN";
}

const char* la_last_error(void) { return g_err; }

la_status la_prefill(const void* q, const void* k, const void* v,
                     const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                     int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                     int32_t head_dim, la_dtype in_dtype, la_dtype out_dtype,
                     const float* decay, const float* kv_init, void* o, float* kv_final,
                     void* stream) {
  la_status st = check_prefill(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                               num_heads, head_dim, in_dtype, out_dtype, decay, kv_init, o,
                               kv_final, num_seqs);
  if (st != LA_OK || num_seqs == 0) return st;

  la::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_seqlens = cu_seqlens_dev;
  a.kv_init = kv_init;
  a.o = o;
  a.kv_final = kv_final;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  const int cols = in_dtype == LA_BF16 ? la::kBf16Cols : la::kF32Cols;
  a.num_items = (int32_t)((int64_t)num_seqs * num_heads * (head_dim / cols));
  for (int32_t h = 0; h < num_heads; ++h) a.log2_decay[h] = (float)log2((double)decay[h]);
  set_order(a, cu_seqlens_host, num_seqs);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (in_dtype != LA_BF16) {
    e = la::launch_prefill_f32(a, head_dim, out_dtype, s);
  } else if (use_wide((int64_t)num_seqs * num_heads, head_dim)) {
    a.num_items = num_seqs * num_heads;
    e = la::launch_prefill_wide(a, out_dtype, false, false, s);
  } else {
    e = la::launch_prefill_bf16(a, head_dim, out_dtype, false, false, s);
  }
  return hip_status(e, "la_prefill launch");
}

la_status la_prefill_pool(const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                          int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                          int32_t head_dim, la_dtype in_dtype, la_dtype out_dtype,
                          const float* decay, float* kv_pool, int32_t pool_size,
                          const int32_t* slots_dev, const int32_t* slots_host, void* o,
                          void* stream) {
  if (in_dtype != LA_BF16 && valid_dtype(in_dtype))
    return fail(LA_ERR_UNSUPPORTED, "the pool prefill takes bf16 inputs only");
  if (pool_size < 0) return fail(LA_ERR_INVALID_ARG, "pool_size = %d < 0", pool_size);
  // the pool stands in for kv_init / kv_final; its own checks follow
  la_status st = check_prefill(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                               num_heads, head_dim, in_dtype, out_dtype, decay, nullptr, o,
                               nullptr, num_seqs);
  if (st != LA_OK || num_seqs == 0) return st;
  if (!kv_pool) return fail(LA_ERR_INVALID_ARG, "kv_pool is NULL");
  if (!aligned16(kv_pool)) return fail(LA_ERR_INVALID_ARG, "kv_pool is not 16-byte aligned");
  if (!slots_dev || !slots_host)
    return fail(LA_ERR_INVALID_ARG, "slots_dev and slots_host must be non-NULL");
  // every slot in range and used once (two sequences on one state would race)
  std::vector<uint8_t> used((size_t)pool_size, 0);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t x = slots_host[s];
    if (x < 0 || x >= pool_size)
      return fail(LA_ERR_INVALID_ARG, "slots[%d] = %d is outside [0, %d)", s, x, pool_size);
    if (used[(size_t)x]) return fail(LA_ERR_INVALID_ARG, "slot %d is used twice", x);
    used[(size_t)x] = 1;
  }
  const size_t tok = (size_t)total_tokens * num_heads * head_dim;
  const Range rp = range("kv_pool", kv_pool, (size_t)pool_size * num_heads * head_dim * head_dim * 4);
  const Range others[] = {range("q", q, tok * 2), range("k", k, tok * 2), range("v", v, tok * 2),
                          range("o", o, tok * dtype_size(out_dtype))};
  for (const Range& r : others)
    if (overlap(rp, r)) return fail(LA_ERR_INVALID_ARG, "kv_pool overlaps %s", r.name);

  la::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_seqlens = cu_seqlens_dev;
  a.kv_init = kv_pool;
  a.kv_final = kv_pool;
  a.init_slot = slots_dev;
  a.final_slot = slots_dev;
  a.o = o;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_items = (int32_t)((int64_t)num_seqs * num_heads * (head_dim / la::kBf16Cols));
  for (int32_t h = 0; h < num_heads; ++h) a.log2_decay[h] = (float)log2((double)decay[h]);
  set_order(a, cu_seqlens_host, num_seqs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (use_wide((int64_t)num_seqs * num_heads, head_dim)) {
    a.num_items = num_seqs * num_heads;
    e = la::launch_prefill_wide(a, out_dtype, false, false, s);
  } else {
    e = la::launch_prefill_bf16(a, head_dim, out_dtype, false, false, s);
  }
  return hip_status(e, "la_prefill_pool launch");
}

// One chain of every (sequence, head), cut into segments: the plan, every
// segment's local state from a zero state, the prefix over the segments, and
// every segment's outputs from the state at its start.  `reverse` runs the
// chain backwards in time: the segments are then taken from the last, so the
// slots of a segment's start state and of its local state trade places (see
// launch_segment_prefix).  Arguments have been validated; ws holds the
// layout `lay`; kv_init / kv_final may be NULL.  With outputs_only the plan
// and the segment start states already in ws are used as they are (only the
// output pass runs; kv_init and kv_final are then unused).
la_status segmented_chain(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_dev,
                          int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                          la_dtype out_dtype, const float* l2, const float* kv_init, void* o,
                          float* kv_final, const SegmentLayout& lay, char* ws, bool reverse,
                          hipStream_t s, bool outputs_only = false) {
  int32_t* cu_seg = reinterpret_cast<int32_t*>(ws + lay.cu_seg);
  int32_t* init_slot = reinterpret_cast<int32_t*>(ws + lay.init_slot);
  int32_t* final_slot = reinterpret_cast<int32_t*>(ws + lay.final_slot);
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + lay.seq_first);
  float* states = reinterpret_cast<float*>(ws + lay.states);
  int32_t* start_slot = reverse ? final_slot : init_slot;  // state entering a segment
  int32_t* local_slot = reverse ? init_slot : final_slot;  // its local state

  la::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_seqlens = cu_seg;
  a.num_seqs = lay.num_segments;
  a.num_heads = num_heads;
  a.num_items = lay.num_segments * num_heads * (head_dim / la::kBf16Cols);
  for (int32_t h = 0; h < num_heads; ++h) a.log2_decay[h] = l2[h];
  const bool wide = use_wide((int64_t)lay.num_segments * num_heads, head_dim);
  if (wide) a.num_items = lay.num_segments * num_heads;
  hipError_t e;
  if (!outputs_only) {
    e = la::launch_segment_plan(cu_seqlens_dev, num_seqs, lay.segment_len, cu_seg, init_slot,
                                final_slot, seq_first, s);
    if (e != hipSuccess) return hip_status(e, "segmented plan launch");

    // pass 1: local decayed state of every segment, from a zero state
    a.kv_final = states;
    a.final_slot = local_slot;
    e = wide ? la::launch_prefill_wide(a, LA_BF16, true, reverse, s)
             : la::launch_prefill_bf16(a, head_dim, LA_BF16, true, reverse, s);
    if (e != hipSuccess) return hip_status(e, "segmented state pass launch");

    // pass 2: states at every segment start (and the final states)
    e = la::launch_segment_prefix(cu_seg, seq_first, num_seqs, num_heads, head_dim, l2, kv_init,
                                  states, kv_final, reverse, s);
    if (e != hipSuccess) return hip_status(e, "segmented prefix launch");
  }

  // pass 3: outputs of every segment from its start state
  a.kv_init = states;
  a.init_slot = start_slot;
  a.kv_final = nullptr;
  a.final_slot = nullptr;
  a.o = o;
  e = wide ? la::launch_prefill_wide(a, out_dtype, false, reverse, s)
           : la::launch_prefill_bf16(a, head_dim, out_dtype, false, reverse, s);
  return hip_status(e, "segmented output pass launch");
}

la_status la_prefill_segmented_workspace_size(int32_t num_seqs, const int32_t* cu_seqlens_host,
                                              int32_t num_heads, int32_t head_dim,
                                              int32_t segment_len, size_t* bytes) {
  if (!bytes) return fail(LA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  if (num_seqs < 0) return fail(LA_ERR_INVALID_ARG, "num_seqs = %d < 0", num_seqs);
  la_status st = check_heads_dim(num_heads, head_dim);
  if (st != LA_OK) return st;
  if ((st = check_segment_len(segment_len)) != LA_OK) return st;
  if (!cu_seqlens_host) return fail(LA_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
  if ((st = check_cu(cu_seqlens_host, num_seqs)) != LA_OK) return st;
  SegmentLayout lay;
  if ((st = segment_layout(cu_seqlens_host, num_seqs, num_heads, head_dim, segment_len, &lay)) != LA_OK)
    return st;
  *bytes = lay.total;
  return ok();
}

la_status la_prefill_segmented(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                               int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                               int32_t head_dim, la_dtype in_dtype, la_dtype out_dtype,
                               const float* decay, const float* kv_init, void* o,
                               float* kv_final, int32_t segment_len, void* workspace,
                               size_t workspace_bytes, void* stream) {
  la_status st = check_segment_len(segment_len);
  if (st != LA_OK) return st;
  if (in_dtype != LA_BF16 && valid_dtype(in_dtype))
    return fail(LA_ERR_UNSUPPORTED, "the segmented prefill takes bf16 inputs only");
  if ((st = check_prefill(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                          num_heads, head_dim, in_dtype, out_dtype, decay, kv_init, o, kv_final,
                          num_seqs)) != LA_OK)
    return st;
  if (num_seqs == 0) return ok();
  SegmentLayout lay;
  if ((st = segment_layout(cu_seqlens_host, num_seqs, num_heads, head_dim, segment_len, &lay)) != LA_OK)
    return st;
  if (!workspace) return fail(LA_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned16(workspace)) return fail(LA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (workspace_bytes < lay.total)
    return fail(LA_ERR_INVALID_ARG, "workspace_bytes = %zu < %zu required", workspace_bytes,
                lay.total);
  // The workspace may overlap no argument buffer.
  {
    const size_t tok = (size_t)total_tokens * num_heads * head_dim;
    const size_t sb = (size_t)num_seqs * num_heads * head_dim * head_dim * 4;
    const Range rw = range("workspace", workspace, lay.total);
    const Range others[] = {range("q", q, tok * 2), range("k", k, tok * 2), range("v", v, tok * 2),
                            range("o", o, tok * dtype_size(out_dtype)),
                            range("kv_init", kv_init, kv_init ? sb : 0),
                            range("kv_final", kv_final, kv_final ? sb : 0)};
    for (const Range& r : others)
      if (overlap(rw, r)) return fail(LA_ERR_INVALID_ARG, "workspace overlaps %s", r.name);
  }
  const int64_t items = (int64_t)lay.num_segments * num_heads * (head_dim / la::kBf16Cols);
  if (items >= ((int64_t)1 << 31) ||
      (int64_t)num_seqs * num_heads * (head_dim * head_dim / 1024) >= ((int64_t)1 << 31))
    return fail(LA_ERR_UNSUPPORTED, "%lld work items exceed the grid limit", (long long)items);

  float l2[LA_MAX_HEADS];
  for (int32_t h = 0; h < num_heads; ++h) l2[h] = (float)log2((double)decay[h]);
  return segmented_chain(q, k, v, cu_seqlens_dev, num_seqs, num_heads, head_dim, out_dtype, l2,
                         kv_init, o, kv_final, lay, static_cast<char*>(workspace), false,
                         static_cast<hipStream_t>(stream));
}

la_status la_prefill_backward_workspace_size(int32_t num_seqs, int32_t num_heads,
                                             int32_t head_dim, size_t* bytes) {
  if (!bytes) return fail(LA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  if (num_seqs < 0) return fail(LA_ERR_INVALID_ARG, "num_seqs = %d < 0", num_seqs);
  la_status st = check_heads_dim(num_heads, head_dim);
  if (st != LA_OK) return st;
  *bytes = (size_t)num_seqs * num_heads * head_dim * head_dim * 4;
  return ok();
}

// Checks shared by the backward entry points, up to the point where a call
// without sequences has nothing left to do.
la_status check_backward_args(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                              int32_t head_dim, la_dtype in_dtype, la_dtype grad_dtype,
                              const float* decay, const float* dkv_final,
                              const int32_t* cu_seqlens_host) {
  if (num_seqs < 0) return fail(LA_ERR_INVALID_ARG, "num_seqs = %d < 0", num_seqs);
  if (total_tokens < 0 || total_tokens >= (int64_t)1 << 31)
    return fail(LA_ERR_INVALID_ARG, "total_tokens = %lld out of range", (long long)total_tokens);
  la_status st = check_heads_dim(num_heads, head_dim);
  if (st != LA_OK) return st;
  if (!valid_dtype(in_dtype)) return fail(LA_ERR_INVALID_ARG, "in_dtype = %d", (int)in_dtype);
  if (!valid_dtype(grad_dtype))
    return fail(LA_ERR_INVALID_ARG, "grad_dtype = %d", (int)grad_dtype);
  if (in_dtype != LA_BF16)
    return fail(LA_ERR_UNSUPPORTED, "the backward takes bf16 inputs only");
  if ((st = check_decay(decay, num_heads)) != LA_OK) return st;
  if (dkv_final) {
    for (int32_t h = 0; h < num_heads; ++h)
      if (decay[h] < 0x1p-64f)
        return fail(LA_ERR_UNSUPPORTED,
                    "decay[%d] = %g < 2^-64 with a final-state gradient is not supported", h,
                    (double)decay[h]);
  }
  if (!cu_seqlens_host) return fail(LA_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
  if ((st = check_cu(cu_seqlens_host, num_seqs)) != LA_OK) return st;
  if ((int64_t)cu_seqlens_host[num_seqs] != total_tokens)
    return fail(LA_ERR_INVALID_ARG, "cu_seqlens[%d] = %d != total_tokens = %lld", num_seqs,
                cu_seqlens_host[num_seqs], (long long)total_tokens);
  return LA_OK;
}

// The buffers of a backward call with sequences: present where needed,
// 16-byte aligned, the grid within its limits, and the outputs and ws_bytes
// of workspace (0: none needed, it may be NULL) overlapping nothing else.
la_status check_backward_buffers(const void* q, const void* k, const void* v, const void* d_o,
                                 const int32_t* cu_seqlens_dev, int32_t num_seqs,
                                 int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                                 la_dtype grad_dtype, const float* kv_init,
                                 const float* dkv_final, void* dq, void* dk, void* dv,
                                 float* dkv_init, void* workspace, size_t workspace_bytes,
                                 size_t ws_bytes) {
  if (!cu_seqlens_dev) return fail(LA_ERR_INVALID_ARG, "cu_seqlens_dev is NULL");
  if (total_tokens > 0 && (!q || !k || !v || !d_o || !dq || !dk || !dv))
    return fail(LA_ERR_INVALID_ARG,
                "q, k, v, d_o, dq, dk and dv must be non-NULL when total_tokens > 0");
  const size_t sb = (size_t)num_seqs * num_heads * head_dim * head_dim * 4;
  if (ws_bytes > 0 && !workspace) return fail(LA_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes > 0 && workspace_bytes < ws_bytes)
    return fail(LA_ERR_INVALID_ARG, "workspace_bytes = %zu < %zu required", workspace_bytes,
                ws_bytes);
  const void* ptrs[] = {q, k, v, d_o, dq, dk, dv, kv_init, dkv_final, dkv_init, workspace};
  const char* names[] = {"q", "k", "v", "d_o", "dq", "dk", "dv", "kv_init", "dkv_final",
                         "dkv_init", "workspace"};
  for (int i = 0; i < 11; ++i)
    if (!aligned16(ptrs[i]))
      return fail(LA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  const int64_t items = (int64_t)num_seqs * num_heads * (head_dim / la::kBf16Cols);
  if (items >= ((int64_t)1 << 31) || (int64_t)num_seqs * num_heads * 16 >= ((int64_t)1 << 31))
    return fail(LA_ERR_UNSUPPORTED, "%lld work items exceed the grid limit", (long long)items);
  // Outputs and the workspace overlap nothing else.
  const size_t tok = (size_t)total_tokens * num_heads * head_dim;
  const Range ins[] = {range("q", q, tok * 2), range("k", k, tok * 2), range("v", v, tok * 2),
                       range("d_o", d_o, tok * 2), range("kv_init", kv_init, kv_init ? sb : 0),
                       range("dkv_final", dkv_final, dkv_final ? sb : 0)};
  const Range outs[] = {range("dq", dq, tok * dtype_size(grad_dtype)),
                        range("dk", dk, tok * dtype_size(grad_dtype)),
                        range("dv", dv, tok * dtype_size(grad_dtype)),
                        range("dkv_init", dkv_init, dkv_init ? sb : 0),
                        range("workspace", workspace, ws_bytes)};
  for (int i = 0; i < 5; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(LA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, r.name);
    for (int j = i + 1; j < 5; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(LA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  return LA_OK;
}

la_status la_prefill_backward(const void* q, const void* k, const void* v, const void* d_o,
                              const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                              int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                              int32_t head_dim, la_dtype in_dtype, la_dtype grad_dtype,
                              const float* decay, const float* kv_init, const float* dkv_final,
                              void* dq, void* dk, void* dv, float* dkv_init, void* workspace,
                              size_t workspace_bytes, void* stream) {
  la_status st = check_backward_args(num_seqs, total_tokens, num_heads, head_dim, in_dtype,
                                     grad_dtype, decay, dkv_final, cu_seqlens_host);
  if (st != LA_OK || num_seqs == 0) return st == LA_OK ? ok() : st;
  const size_t sb = (size_t)num_seqs * num_heads * head_dim * head_dim * 4;
  const bool need_ws = kv_init || dkv_final;
  if ((st = check_backward_buffers(q, k, v, d_o, cu_seqlens_dev, num_seqs, total_tokens,
                                   num_heads, head_dim, grad_dtype, kv_init, dkv_final, dq, dk,
                                   dv, dkv_init, workspace, workspace_bytes,
                                   need_ws ? sb : 0)) != LA_OK)
    return st;
  const int64_t items = (int64_t)num_seqs * num_heads * (head_dim / la::kBf16Cols);

  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  float one[LA_MAX_HEADS], inv[LA_MAX_HEADS], lam[LA_MAX_HEADS];
  la::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.cu_seqlens = cu_seqlens_dev;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_items = (int32_t)items;
  for (int32_t h = 0; h < num_heads; ++h) {
    a.log2_decay[h] = (float)log2((double)decay[h]);
    one[h] = 1.0f;
    inv[h] = (float)(1.0 / (double)decay[h]);
    lam[h] = decay[h];
  }
  set_order(a, cu_seqlens_host, num_seqs);
  if (head_dim == 128) {
    // The three chains are independent: one launch of the wide kernel runs
    // them side by side (3 S H workgroups), each reading its initial state
    // straight from kv_init / dkv_final (transposed, scaled by 1/lambda) and
    // writing dS0 = lambda x the dV chain's final state.  No workspace.
    la::BackwardPasses bp;
    memset(&bp, 0, sizeof(bp));
    bp.pass[0] = {d_o, v, k, dq, kv_init, nullptr, 0, 1, 0.0f, 0.0f};          // dQ
    bp.pass[1] = {v, d_o, q, dk, dkv_final, nullptr, 1, 1, -1.0f, 0.0f};       // dK
    bp.pass[2] = {k, q, d_o, dv, dkv_final, dkv_init, 1, 0, -1.0f, 1.0f};      // dV, dS0
    a.num_items = 3 * num_seqs * num_heads;
    const hipError_t e = la::launch_backward_wide(a, bp, grad_dtype, s);
    return e != hipSuccess ? hip_status(e, "la_prefill_backward launch") : ok();
  }
  // d = 64: three launches of the 32-column kernel (or of the wide kernel
  // when there are enough chains to fill the GPU) with the states
  // transformed in the workspace between them.
  const bool wide = use_wide((int64_t)num_seqs * num_heads, head_dim);
  auto pass = [&](bool reverse) {
    if (!wide) return la::launch_prefill_bf16(a, head_dim, grad_dtype, false, reverse, s);
    la::PrefillArgs w = a;
    w.num_items = num_seqs * num_heads;
    return la::launch_prefill_wide(w, grad_dtype, false, reverse, s);
  };
  hipError_t e;
  // dQ: the forward chain with dO as queries, V as keys, K as values, S0^T
  if (kv_init) {
    e = la::launch_state_transform(kv_init, ws, num_seqs, num_heads, head_dim, true, one, s);
    if (e != hipSuccess) return hip_status(e, "la_prefill_backward state launch");
  }
  a.q = d_o;
  a.k = v;
  a.v = k;
  a.kv_init = kv_init ? ws : nullptr;
  a.o = dq;
  e = pass(false);
  if (e != hipSuccess) return hip_status(e, "la_prefill_backward dq launch");
  // dK: backwards in time, V as queries, dO as keys, Q as values, dS_L^T / lambda
  if (dkv_final) {
    e = la::launch_state_transform(dkv_final, ws, num_seqs, num_heads, head_dim, true, inv, s);
    if (e != hipSuccess) return hip_status(e, "la_prefill_backward state launch");
  }
  a.q = v;
  a.k = d_o;
  a.v = q;
  a.kv_init = dkv_final ? ws : nullptr;
  a.o = dk;
  e = pass(true);
  if (e != hipSuccess) return hip_status(e, "la_prefill_backward dk launch");
  // dV: backwards in time, K as queries, Q as keys, dO as values, dS_L / lambda;
  // its final state is dS0 / lambda
  if (dkv_final) {
    e = la::launch_state_transform(dkv_final, ws, num_seqs, num_heads, head_dim, false, inv, s);
    if (e != hipSuccess) return hip_status(e, "la_prefill_backward state launch");
  }
  a.q = k;
  a.k = q;
  a.v = d_o;
  a.kv_init = dkv_final ? ws : nullptr;
  a.o = dv;
  a.kv_final = dkv_init;
  e = pass(true);
  if (e != hipSuccess) return hip_status(e, "la_prefill_backward dv launch");
  if (dkv_init) {
    e = la::launch_state_transform(dkv_init, dkv_init, num_seqs, num_heads, head_dim, false, lam, s);
    if (e != hipSuccess) return hip_status(e, "la_prefill_backward state launch");
  }
  return ok();
}

la_status la_prefill_backward_segmented_workspace_size(int32_t num_seqs,
                                                       const int32_t* cu_seqlens_host,
                                                       int32_t num_heads, int32_t head_dim,
                                                       int32_t segment_len, size_t* bytes) {
  la_status st = la_prefill_segmented_workspace_size(num_seqs, cu_seqlens_host, num_heads,
                                                     head_dim, segment_len, bytes);
  if (st != LA_OK) return st;
  // the segment layout, then one set of S initial states
  *bytes = align256(*bytes) + (size_t)num_seqs * num_heads * head_dim * head_dim * 4;
  return ok();
}

la_status la_prefill_backward_segmented(
    const void* q, const void* k, const void* v, const void* d_o, const int32_t* cu_seqlens_dev,
    const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
    int32_t head_dim, la_dtype in_dtype, la_dtype grad_dtype, const float* decay,
    const float* kv_init, const float* dkv_final, void* dq, void* dk, void* dv, float* dkv_init,
    int32_t segment_len, void* workspace, size_t workspace_bytes, void* stream) {
  la_status st = check_segment_len(segment_len);
  if (st != LA_OK) return st;
  if ((st = check_backward_args(num_seqs, total_tokens, num_heads, head_dim, in_dtype,
                                grad_dtype, decay, dkv_final, cu_seqlens_host)) != LA_OK)
    return st;
  if (num_seqs == 0) return ok();
  SegmentLayout lay;
  if ((st = segment_layout(cu_seqlens_host, num_seqs, num_heads, head_dim, segment_len, &lay)) != LA_OK)
    return st;
  const size_t sb = (size_t)num_seqs * num_heads * head_dim * head_dim * 4;
  const size_t init_off = align256(lay.total);
  if ((st = check_backward_buffers(q, k, v, d_o, cu_seqlens_dev, num_seqs, total_tokens,
                                   num_heads, head_dim, grad_dtype, kv_init, dkv_final, dq, dk,
                                   dv, dkv_init, workspace, workspace_bytes, init_off + sb)) != LA_OK)
    return st;
  const int64_t items = (int64_t)lay.num_segments * num_heads * (head_dim / la::kBf16Cols);
  const int64_t tiles = head_dim / 32;  // the in-place transpose: one workgroup per tile pair
  if (items >= ((int64_t)1 << 31) ||
      (int64_t)num_seqs * num_heads * (head_dim * head_dim / 1024) >= ((int64_t)1 << 31) ||
      ((int64_t)lay.num_segments + num_seqs) * num_heads * (tiles * (tiles + 1) / 2) >=
          ((int64_t)1 << 31))
    return fail(LA_ERR_UNSUPPORTED, "%lld work items exceed the grid limit", (long long)items);

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* init = reinterpret_cast<float*>(ws + init_off);  // a chain's initial states
  float l2[LA_MAX_HEADS], one[LA_MAX_HEADS], inv[LA_MAX_HEADS], lam[LA_MAX_HEADS];
  for (int32_t h = 0; h < num_heads; ++h) {
    l2[h] = (float)log2((double)decay[h]);
    one[h] = 1.0f;
    inv[h] = (float)(1.0 / (double)decay[h]);
    lam[h] = decay[h];
  }
  // The three chains of la_prefill_backward one after the other, each cut
  // into segments; the chains share the segment workspace and the region of
  // initial states, in stream order.
  hipError_t e;
  // dQ: forwards with dO, V, K and initial state S0^T
  if (kv_init) {
    e = la::launch_state_transform(kv_init, init, num_seqs, num_heads, head_dim, true, one, s);
    if (e != hipSuccess) return hip_status(e, "la_prefill_backward_segmented state launch");
  }
  st = segmented_chain(d_o, v, k, cu_seqlens_dev, num_seqs, num_heads, head_dim, grad_dtype, l2,
                       kv_init ? init : nullptr, dq, nullptr, lay, ws, false, s);
  if (st != LA_OK) return st;
  // dK: backwards with V, dO, Q and dS_L^T / lambda; its final state is
  // (dS0 / lambda)^T
  if (dkv_final) {
    e = la::launch_state_transform(dkv_final, init, num_seqs, num_heads, head_dim, true, inv, s);
    if (e != hipSuccess) return hip_status(e, "la_prefill_backward_segmented state launch");
  }
  st = segmented_chain(v, d_o, q, cu_seqlens_dev, num_seqs, num_heads, head_dim, grad_dtype, l2,
                       dkv_final ? init : nullptr, dk, dkv_init, lay, ws, true, s);
  if (st != LA_OK) return st;
  // dV: backwards with K, Q, dO and dS_L / lambda.  Its keys and values are
  // the dK chain's values and keys, with the same decays and the transposed
  // initial state, so each of its states is the transpose of the dK chain's
  // state at the same point: the dK chain's segment start states, transposed
  // in place, are the dV chain's, and only its output pass runs.
  float* states = reinterpret_cast<float*>(ws + lay.states);
  e = la::launch_state_transpose_inplace(states, (lay.num_segments + num_seqs) * num_heads,
                                         num_heads, head_dim, one, s);
  if (e != hipSuccess) return hip_status(e, "la_prefill_backward_segmented state launch");
  st = segmented_chain(k, q, d_o, cu_seqlens_dev, num_seqs, num_heads, head_dim, grad_dtype, l2,
                       nullptr, dv, nullptr, lay, ws, true, s, true);
  if (st != LA_OK) return st;
  if (dkv_init) {  // dS0: lambda times the transpose of the dK chain's final state
    e = la::launch_state_transpose_inplace(dkv_init, num_seqs * num_heads, num_heads, head_dim,
                                           lam, s);
    if (e != hipSuccess) return hip_status(e, "la_prefill_backward_segmented state launch");
  }
  return ok();
}

la_status la_decode(const void* q, const void* k, const void* v, float* kv,
                    const float* decay, int32_t batch, int32_t num_heads, int32_t head_dim,
                    la_dtype in_dtype, void* o, void* stream) {
  return decode_common(q, k, v, kv, batch, nullptr, nullptr, decay, batch, num_heads, head_dim,
                       in_dtype, o, stream);
}

la_status la_decode_pool(const void* q, const void* k, const void* v, float* kv_pool,
                         int32_t pool_size, const int32_t* slots_dev, const int32_t* slots_host,
                         const float* decay, int32_t batch, int32_t num_heads, int32_t head_dim,
                         la_dtype in_dtype, void* o, void* stream) {
  if (batch < 0) return fail(LA_ERR_INVALID_ARG, "batch = %d < 0", batch);
  if (pool_size < 0) return fail(LA_ERR_INVALID_ARG, "pool_size = %d < 0", pool_size);
  if (batch > 0) {
    if (!slots_dev || !slots_host)
      return fail(LA_ERR_INVALID_ARG, "slots_dev and slots_host must be non-NULL");
    // every slot in range and used once (two sequences on one state would race)
    std::vector<uint8_t> used((size_t)pool_size, 0);
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t x = slots_host[b];
      if (x < 0 || x >= pool_size)
        return fail(LA_ERR_INVALID_ARG, "slots[%d] = %d is outside [0, %d)", b, x, pool_size);
      if (used[(size_t)x]) return fail(LA_ERR_INVALID_ARG, "slot %d is used twice", x);
      used[(size_t)x] = 1;
    }
  }
  return decode_common(q, k, v, kv_pool, pool_size, slots_dev, slots_host, decay, batch,
                       num_heads, head_dim, in_dtype, o, stream);
}

}  // extern "C"
