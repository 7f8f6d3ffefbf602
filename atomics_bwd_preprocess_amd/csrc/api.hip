// C ABI of the attention backward library: argument validation, then one or
// two kernel launches on the caller's stream.  No allocation, no state, no
// synchronisation.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>

#include "../../include/attn_bwd.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

attn_status_t ok() {
  g_last_error[0] = '\0';
  return ATTN_OK;
}

attn_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, ...)                                   \
  do {                                                       \
    if (!(cond)) return fail(ATTN_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

#define REQUIRE_TENSOR(ptr)                                                        \
  do {                                                                             \
    REQUIRE((ptr) != nullptr, "%s is NULL", #ptr);                                 \
    REQUIRE(aligned((ptr), 16), "%s is not 16-byte aligned", #ptr);                \
  } while (0)

#define REQUIRE_F32(ptr)                                                           \
  do {                                                                             \
    REQUIRE((ptr) != nullptr, "%s is NULL", #ptr);                                 \
    REQUIRE(aligned((ptr), 4), "%s is not 4-byte aligned", #ptr);                  \
  } while (0)

// Validates the problem description; fills `p`.
attn_status_t check_shape(const attn_shape_t* s, const int32_t* cu, bool need_cu_check,
                          attn::Problem& p) {
  REQUIRE(s != nullptr, "shape is NULL");
  REQUIRE(s->num_seqs >= 1, "num_seqs must be >= 1 (got %d)", s->num_seqs);
  REQUIRE(s->max_seqlen >= 1, "max_seqlen must be >= 1 (got %d)", s->max_seqlen);
  REQUIRE(s->total_tokens >= 0, "total_tokens must be >= 0 (got %d)", s->total_tokens);
  REQUIRE(s->hq >= 1 && s->hkv >= 1, "hq and hkv must be >= 1 (got %d, %d)", s->hq, s->hkv);
  REQUIRE(s->hq % s->hkv == 0, "hq (%d) must be a multiple of hkv (%d)", s->hq, s->hkv);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", s->head_dim);
  if (s->dtype != ATTN_F16 && s->dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", s->dtype);
  REQUIRE(s->causal == 0 || s->causal == 1, "causal must be 0 or 1 (got %d)", s->causal);
  REQUIRE(s->window >= 0, "window must be >= 0 (got %d)", s->window);
  REQUIRE(s->window == 0 || s->causal, "a sliding window requires causal = 1");
  REQUIRE(isfinite(s->scale) && s->scale > 0.0f, "scale must be finite and > 0");
  REQUIRE(s->layout == ATTN_LAYOUT_THD || s->layout == ATTN_LAYOUT_BHSD,
          "layout must be ATTN_LAYOUT_THD or ATTN_LAYOUT_BHSD (got %d)", s->layout);
  if (s->layout == ATTN_LAYOUT_BHSD) {
    REQUIRE(cu == nullptr, "the [B, H, S, D] layout is a dense batch: cu_seqlens must be NULL");
    REQUIRE((long long)s->num_seqs * s->max_seqlen == s->total_tokens,
            "the [B, H, S, D] layout needs total_tokens == num_seqs * max_seqlen");
    REQUIRE((long long)s->max_seqlen * s->head_dim < (1LL << 32),
            "max_seqlen * head_dim must fit 32 bits in the [B, H, S, D] layout");
  }
  // 64-bit element counts must fit the launch geometry and index math.
  const long long rows = (long long)s->total_tokens * s->hq;
  REQUIRE(rows * s->head_dim < (1LL << 40), "tensor too large");
  const long long blocks = (long long)((s->max_seqlen + 63) / 64) * s->num_seqs * s->hq;
  REQUIRE(blocks < (1LL << 31), "launch grid too large");
  if (need_cu_check && cu == nullptr)
    REQUIRE((long long)s->num_seqs * s->max_seqlen == s->total_tokens,
            "cu_seqlens is NULL but total_tokens != num_seqs * max_seqlen");
  if (cu != nullptr) REQUIRE(aligned(cu, 4), "cu_seqlens is not 4-byte aligned");
  p.num_seqs = s->num_seqs;
  p.max_seqlen = s->max_seqlen;
  p.total = s->total_tokens;
  p.hq = s->hq;
  p.hkv = s->hkv;
  p.d = s->head_dim;
  p.causal = s->causal != 0;
  p.window = s->window;
  p.scale = s->scale;
  p.bf16 = s->dtype == ATTN_BF16;
  p.bhsd = s->layout == ATTN_LAYOUT_BHSD;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd(const attn_shape_t* shape, const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens, const float* sink, void* o, float* lse,
                       hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, cu_seqlens, true, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(q);
  REQUIRE_TENSOR(k);
  REQUIRE_TENSOR(v);
  REQUIRE_TENSOR(o);
  REQUIRE_F32(lse);
  if (sink) REQUIRE(aligned(sink, 4), "sink is not 4-byte aligned");
  if (p.total == 0) return ok();
  return hip_status(attn::launch_fwd(p, q, k, v, cu_seqlens, sink, o, lse, stream), "attn_fwd");
}

attn_status_t attn_bwd_preprocess(const attn_shape_t* shape, const void* o, const void* dout,
                                  const float* lse, const int32_t* cu_seqlens,
                                  const float* sink, float* delta, float* dq_accum,
                                  float* dsink, hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, cu_seqlens, true, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(o);
  REQUIRE_TENSOR(dout);
  if (dq_accum) REQUIRE(aligned(dq_accum, 16), "dq_accum is not 16-byte aligned");
  REQUIRE_F32(delta);
  REQUIRE((sink == nullptr) == (dsink == nullptr), "sink and dsink must both be NULL or both set");
  if (sink) {
    REQUIRE_F32(lse);
    REQUIRE_F32(sink);
    REQUIRE_F32(dsink);
  }
  if (p.total == 0) {
    if (!sink) return ok();
  }
  return hip_status(attn::launch_preprocess(p, o, dout, lse, sink, delta, dq_accum, dsink, stream),
                    "attn_bwd_preprocess");
}

attn_status_t attn_bwd_dsink(const attn_shape_t* shape, const float* lse, const float* delta,
                             const float* sink, float* dsink, hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, nullptr, false, p);
  if (st != ATTN_OK) return st;
  REQUIRE_F32(lse);
  REQUIRE_F32(delta);
  REQUIRE_F32(sink);
  REQUIRE_F32(dsink);
  return hip_status(attn::launch_dsink(p, lse, delta, sink, dsink, stream), "attn_bwd_dsink");
}

attn_status_t attn_bwd(const attn_shape_t* shape, const void* q, const void* k, const void* v,
                       const void* dout, const float* lse, const float* delta,
                       const int32_t* cu_seqlens, float* dq_accum, void* dk, void* dv,
                       hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, cu_seqlens, true, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(q);
  REQUIRE_TENSOR(k);
  REQUIRE_TENSOR(v);
  REQUIRE_TENSOR(dout);
  REQUIRE_F32(lse);
  REQUIRE_F32(delta);
  REQUIRE_TENSOR(dq_accum);
  REQUIRE_TENSOR(dk);
  REQUIRE_TENSOR(dv);
  if (p.total == 0) return ok();
  return hip_status(attn::launch_bwd(p, q, k, v, dout, lse, delta, cu_seqlens, dq_accum, dk, dv,
                                     stream),
                    "attn_bwd");
}

attn_status_t attn_bwd_fused_cast(const attn_shape_t* shape, const void* q, const void* k,
                                  const void* v, const void* dout, const float* lse,
                                  const float* delta, const int32_t* cu_seqlens, float* dq_accum,
                                  int32_t* counters, void* dq, void* dk, void* dv,
                                  hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, cu_seqlens, true, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(q);
  REQUIRE_TENSOR(k);
  REQUIRE_TENSOR(v);
  REQUIRE_TENSOR(dout);
  REQUIRE_F32(lse);
  REQUIRE_F32(delta);
  REQUIRE_TENSOR(dq_accum);
  REQUIRE_TENSOR(counters);
  REQUIRE_TENSOR(dq);
  REQUIRE_TENSOR(dk);
  REQUIRE_TENSOR(dv);
  if (p.total == 0) return ok();
  hipError_t e;
  if (!p.causal || p.bhsd) {
    e = attn::launch_bwd(p, q, k, v, dout, lse, delta, cu_seqlens, dq_accum, dk, dv, stream);
    if (e != hipSuccess) return hip_status(e, "attn_bwd_fused_cast: main pass");
    return hip_status(attn::launch_postprocess(p, dq_accum, dq, stream), "attn_bwd_fused_cast: cast");
  }
  const long long n = ATTN_FUSED_CAST_COUNTERS(p.num_seqs, p.hq, p.max_seqlen);
  e = attn::launch_zero(reinterpret_cast<float*>(counters), (size_t)n, stream);
  if (e != hipSuccess) return hip_status(e, "attn_bwd_fused_cast: clearing the counters");
  return hip_status(attn::launch_bwd_fused_cast(p, q, k, v, dout, lse, delta, cu_seqlens, dq_accum,
                                                counters, dq, dk, dv, stream),
                    "attn_bwd_fused_cast");
}

attn_status_t attn_bwd_dkdv(const attn_shape_t* shape, const void* q, const void* k,
                            const void* v, const void* dout, const float* lse,
                            const float* delta, const int32_t* cu_seqlens, void* dk, void* dv,
                            hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, cu_seqlens, true, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(q);
  REQUIRE_TENSOR(k);
  REQUIRE_TENSOR(v);
  REQUIRE_TENSOR(dout);
  REQUIRE_F32(lse);
  REQUIRE_F32(delta);
  REQUIRE_TENSOR(dk);
  REQUIRE_TENSOR(dv);
  if (p.total == 0) return ok();
  return hip_status(attn::launch_bwd_dkdv(p, q, k, v, dout, lse, delta, cu_seqlens, dk, dv, stream),
                    "attn_bwd_dkdv");
}

attn_status_t attn_bwd_dq(const attn_shape_t* shape, const void* q, const void* k, const void* v,
                          const void* dout, const float* lse, const float* delta,
                          const int32_t* cu_seqlens, void* dq, hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, cu_seqlens, true, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(q);
  REQUIRE_TENSOR(k);
  REQUIRE_TENSOR(v);
  REQUIRE_TENSOR(dout);
  REQUIRE_F32(lse);
  REQUIRE_F32(delta);
  REQUIRE_TENSOR(dq);
  if (p.total == 0) return ok();
  return hip_status(attn::launch_bwd_dq(p, q, k, v, dout, lse, delta, cu_seqlens, dq, nullptr,
                                        nullptr, stream),
                    "attn_bwd_dq");
}

attn_status_t attn_bwd_dq_delta(const attn_shape_t* shape, const void* q, const void* k,
                                const void* v, const void* o, const void* dout, const float* lse,
                                const int32_t* cu_seqlens, float* delta, void* dq,
                                hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, cu_seqlens, true, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(q);
  REQUIRE_TENSOR(k);
  REQUIRE_TENSOR(v);
  REQUIRE_TENSOR(o);
  REQUIRE_TENSOR(dout);
  REQUIRE_F32(lse);
  REQUIRE_F32(delta);
  REQUIRE_TENSOR(dq);
  if (p.total == 0) return ok();
  return hip_status(attn::launch_bwd_dq(p, q, k, v, dout, lse, delta, cu_seqlens, dq, o, delta,
                                        stream),
                    "attn_bwd_dq_delta");
}

attn_status_t attn_bwd_split(const attn_shape_t* shape, const void* q, const void* k,
                             const void* v, const void* dout, const float* lse,
                             const float* delta, const int32_t* cu_seqlens, float* dq_accum,
                             float* dkv_partial, int32_t nsplit, hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, cu_seqlens, true, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(q);
  REQUIRE_TENSOR(k);
  REQUIRE_TENSOR(v);
  REQUIRE_TENSOR(dout);
  REQUIRE_F32(lse);
  REQUIRE_F32(delta);
  if (dq_accum) REQUIRE(aligned(dq_accum, 16), "dq_accum is not 16-byte aligned");
  REQUIRE_TENSOR(dkv_partial);
  REQUIRE(nsplit >= 1 && nsplit <= ATTN_MAX_SPLIT, "nsplit must be in [1, %d] (got %d)",
          ATTN_MAX_SPLIT, nsplit);
  if (p.total == 0) return ok();
  return hip_status(attn::launch_bwd_split(p, q, k, v, dout, lse, delta, cu_seqlens, dq_accum,
                                           dkv_partial, nsplit, stream),
                    "attn_bwd_split");
}

attn_status_t attn_bwd_dkv_reduce(const attn_shape_t* shape, const float* dkv_partial,
                                  int32_t nsplit, void* dk, void* dv, hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, nullptr, false, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(dkv_partial);
  REQUIRE_TENSOR(dk);
  REQUIRE_TENSOR(dv);
  REQUIRE(nsplit >= 1 && nsplit <= ATTN_MAX_SPLIT, "nsplit must be in [1, %d] (got %d)",
          ATTN_MAX_SPLIT, nsplit);
  if (p.total == 0) return ok();
  return hip_status(attn::launch_dkv_reduce(p, dkv_partial, nsplit, dk, dv, stream),
                    "attn_bwd_dkv_reduce");
}

attn_status_t attn_bwd_static(const attn_shape_t* shape, const void* q, const void* k,
                              const void* v, const void* dout, const float* lse,
                              const float* delta, const int32_t* cu_seqlens, void* dq, void* dk,
                              void* dv, hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, cu_seqlens, true, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(q);
  REQUIRE_TENSOR(k);
  REQUIRE_TENSOR(v);
  REQUIRE_TENSOR(dout);
  REQUIRE_F32(lse);
  REQUIRE_F32(delta);
  REQUIRE_TENSOR(dq);
  REQUIRE_TENSOR(dk);
  REQUIRE_TENSOR(dv);
  const unsigned long long n = (unsigned long long)p.total * p.hq * p.d;
  REQUIRE(n * 4 <= ATTN_STATIC_SCRATCH_BYTES,
          "attn_bwd_static: the dQ accumulator needs %llu bytes, more than the %u bytes of the "
          "library's scratch array (call attn_bwd with a caller-owned dq_accum instead)",
          n * 4, (unsigned)ATTN_STATIC_SCRATCH_BYTES);
  if (p.total == 0) return ok();
  float* acc = nullptr;
  hipError_t e = attn::static_scratch(&acc);
  if (e != hipSuccess) return hip_status(e, "attn_bwd_static: scratch array address");
  e = attn::launch_zero(acc, (size_t)n, stream);
  if (e != hipSuccess) return hip_status(e, "attn_bwd_static: clearing the accumulator");
  e = attn::launch_bwd(p, q, k, v, dout, lse, delta, cu_seqlens, acc, dk, dv, stream);
  if (e != hipSuccess) return hip_status(e, "attn_bwd_static: main pass");
  return hip_status(attn::launch_postprocess(p, acc, dq, stream), "attn_bwd_static: cast");
}

attn_status_t attn_bwd_postprocess(const attn_shape_t* shape, const float* dq_accum, void* dq,
                                   hipStream_t stream) {
  attn::Problem p;
  attn_status_t st = check_shape(shape, nullptr, false, p);
  if (st != ATTN_OK) return st;
  REQUIRE_TENSOR(dq_accum);
  REQUIRE_TENSOR(dq);
  if (p.total == 0) return ok();
  return hip_status(attn::launch_postprocess(p, dq_accum, dq, stream), "attn_bwd_postprocess");
}

const char* attn_status_string(attn_status_t status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_last_error; }

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
