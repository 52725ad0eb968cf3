// Host side of the libla C ABI: argument validation, per-head decay
// preprocessing and kernel dispatch.  Every argument error is found here,
// before anything is enqueued; the library never synchronises and allocates
// no device memory.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "la.h"
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

la_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
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
  if (cu_seqlens_host[0] != 0)
    return fail(LA_ERR_INVALID_ARG, "cu_seqlens[0] = %d, expected 0", cu_seqlens_host[0]);
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (cu_seqlens_host[s + 1] < cu_seqlens_host[s])
      return fail(LA_ERR_INVALID_ARG, "cu_seqlens decreases at %d (%d -> %d)", s,
                  cu_seqlens_host[s], cu_seqlens_host[s + 1]);
  }
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
  const int64_t items = (int64_t)num_seqs * num_heads * (head_dim / cols);
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
  a.num_items = (int32_t)items;
  for (int32_t h = 0; h < num_heads; ++h) a.log2_decay[h] = (float)log2((double)decay[h]);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = in_dtype == LA_BF16 ? la::launch_prefill_bf16(a, head_dim, out_dtype, s)
                                     : la::launch_prefill_f32(a, head_dim, out_dtype, s);
  return hip_status(e, "la_prefill launch");
}

la_status la_decode(const void* q, const void* k, const void* v, float* kv,
                    const float* decay, int32_t batch, int32_t num_heads, int32_t head_dim,
                    la_dtype in_dtype, void* o, void* stream) {
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
  const Range rs = range("kv", kv, (size_t)batch * num_heads * head_dim * head_dim * 4);
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
  a.o = o;
  a.batch = batch;
  a.num_heads = num_heads;
  for (int32_t h = 0; h < num_heads; ++h) a.decay[h] = decay[h];
  hipError_t e = la::launch_decode(a, head_dim, in_dtype, static_cast<hipStream_t>(stream));
  return hip_status(e, "la_decode launch");
}

}  // extern "C"
