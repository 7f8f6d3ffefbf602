// Backward preprocess and postprocess: the HBM-bound kernels around the main
// backward pass.
//
//  * preprocess  (tilelang-ascend PR "GQA Sink Backward BHSD": the merged
//    preprocess + dsink kernel, and Phase 0 / Phase 5 of its single backward
//    kernel): Delta = row sum of O * dO in fp32, zeroing of the fp32 dQ
//    accumulator (when the atomic dQ path uses one), and
//    dsink = -sum_t exp(sink - lse) * Delta.
//  * postprocess (same PR: the postprocess kernel that casts the fp32
//    accumulated gradient to fp16): dQ = RNE cast of scale x the fp32
//    accumulator (the main pass leaves the score scale out of dS).
//
// Algorithmic bytes (e = 2 bytes per 16-bit element, R = T * Hq rows):
//   delta kernel:  R * D * 2e (O, dO) + R * 4 (Delta) [+ R * D * 4 (zeroing)]
//   dsink kernel:  R * 8 (lse, Delta)
//   postprocess:   R * D * (4 + e)
#include "common.h"
#include "delta_dot.h"
#include "launch.h"

namespace attn {

// One workgroup: query head blockIdx.y, tokens [blockIdx.x * 64, +64).
// A row (token, head) is D contiguous elements read as 16-byte chunks by
// D / 8 consecutive lanes; the partial dot products are reduced across those
// lanes with xor shuffles (which stay inside a row group).  ZERO: also clear
// the row of the fp32 dQ accumulator.  Row (token t, head h) sits at
// (t - i) * hq * D + i * row + h * head, with i = t % S for [B, H, S, D]
// tensors (seq_len = S) and i = 0 for packed [T, H, D] ones (seq_len = 0).
template <typename T, int D, bool ZERO>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ o,
                                                    const T* __restrict__ dout,
                                                    float* __restrict__ delta,
                                                    float* __restrict__ dq_accum, int total,
                                                    int hq, int seq_len, uint32_t row,
                                                    uint32_t head) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerPass = 256 / kLanesPerRow;
  constexpr int kTokens = 64;
  const int h = blockIdx.y;
  const int sub = threadIdx.x % kLanesPerRow;
  const int r = threadIdx.x / kLanesPerRow;
#pragma unroll
  for (int pass = 0; pass < kTokens / kRowsPerPass; ++pass) {
    const int t = blockIdx.x * kTokens + pass * kRowsPerPass + r;
    float acc = 0.0f;
    if (t < total) {
      const int i = seq_len ? t % seq_len : 0;
      const size_t base = (size_t)(t - i) * hq * D + (size_t)i * row + (size_t)h * head + sub * 8;
      acc = dot8(ld16<T>(o + base), ld16<T>(dout + base), 0.0f);
      if constexpr (ZERO) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(dq_accum + base) = z;
        *reinterpret_cast<f32x4*>(dq_accum + base + 4) = z;
      }
    }
#pragma unroll
    for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (sub == 0 && t < total) delta[(size_t)h * total + t] = acc;
  }
}

// One workgroup per query head: dsink[h] = -sum_t exp(sink[h] - lse[h][t]) * delta[h][t],
// reduced in a fixed order (per-thread strided sums over four independent
// accumulators, then fixed trees across lanes and waves), so the result is
// deterministic and needs neither atomics nor prior zeroing.
constexpr int kDsinkThreads = 1024;
__global__ __launch_bounds__(kDsinkThreads) void dsink_kernel(const float* __restrict__ lse,
                                                              const float* __restrict__ delta,
                                                              const float* __restrict__ sink,
                                                              float* __restrict__ dsink, int total) {
  __shared__ float part[kDsinkThreads / 64];
  const int h = blockIdx.x;
  const float s = sink[h];
  const float* l = lse + (size_t)h * total;
  const float* dl = delta + (size_t)h * total;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int t = threadIdx.x;
  for (; t + 3 * kDsinkThreads < total; t += 4 * kDsinkThreads) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tu = t + u * kDsinkThreads;
      acc[u] += expf(s - l[tu]) * dl[tu];
    }
  }
  for (; t < total; t += kDsinkThreads) acc[0] += expf(s - l[t]) * dl[t];
  float a = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = 0.0f;
#pragma unroll
    for (int i = 0; i < kDsinkThreads / 64; i += 2) r += part[i] + part[i + 1];
    dsink[h] = -r;
  }
}

// dq[i] = RNE(scale * dq_accum[i]) for 8 consecutive elements per thread
// (the main pass accumulates dS' K with dS' = dS / scale).  dq and dq_accum
// share their layout, so the cast is flat.
template <typename T>
__global__ __launch_bounds__(256) void cast_kernel(const float* __restrict__ src,
                                                   T* __restrict__ dst, size_t n8, float scale) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(src + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(src + 8 * i + 4);
  typename V8<T>::type r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r[k] = to16<T>(a[k] * scale);
    r[k + 4] = to16<T>(b[k] * scale);
  }
  st16<T>(dst + 8 * i, r);
}

// dk[i] = RNE(sum_p part[p][0][i]), dv[i] = RNE(sum_p part[p][1][i]) over the
// nsplit fp32 partial slots in a fixed order (p ascending), 8 consecutive
// elements per thread; dk, dv and the slots share their layout.
template <typename T>
__global__ __launch_bounds__(256) void dkv_reduce_kernel(const float* __restrict__ part, int nsplit,
                                                         size_t n_kv, T* __restrict__ dk,
                                                         T* __restrict__ dv) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_kv / 8) return;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
      const float* src = part + ((size_t)s * 2 + which) * n_kv + 8 * i;
      a += *reinterpret_cast<const f32x4*>(src);
      b += *reinterpret_cast<const f32x4*>(src + 4);
    }
    typename V8<T>::type r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r[k] = to16<T>(a[k]);
      r[k + 4] = to16<T>(b[k]);
    }
    st16<T>((which ? dv : dk) + 8 * i, r);
  }
}

hipError_t launch_dsink(const Problem& p, const float* lse, const float* delta, const float* sink,
                        float* dsink, hipStream_t stream) {
  hipLaunchKernelGGL(dsink_kernel, dim3(p.hq), dim3(kDsinkThreads), 0, stream, lse, delta, sink,
                     dsink, p.total);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t preprocess_t(const Problem& p, const void* o, const void* dout,
                               const float* lse, const float* sink, float* delta,
                               float* dq_accum, float* dsink, hipStream_t stream) {
  if (p.total > 0) {
    dim3 grid((p.total + 63) / 64, p.hq);
    const int seq_len = p.bhsd ? p.max_seqlen : 0;
    const uint32_t row = p.bhsd ? (uint32_t)p.d : (uint32_t)p.hq * p.d;  // between rows of a head
    const uint32_t head = p.bhsd ? (uint32_t)p.max_seqlen * p.d : (uint32_t)p.d;
    if (dq_accum)
      hipLaunchKernelGGL((delta_kernel<T, D, true>), grid, dim3(256), 0, stream,
                         static_cast<const T*>(o), static_cast<const T*>(dout), delta, dq_accum,
                         p.total, p.hq, seq_len, row, head);
    else
      hipLaunchKernelGGL((delta_kernel<T, D, false>), grid, dim3(256), 0, stream,
                         static_cast<const T*>(o), static_cast<const T*>(dout), delta, dq_accum,
                         p.total, p.hq, seq_len, row, head);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (sink == nullptr) return hipSuccess;
  return launch_dsink(p, lse, delta, sink, dsink, stream);
}

hipError_t launch_preprocess(const Problem& p, const void* o, const void* dout, const float* lse,
                             const float* sink, float* delta, float* dq_accum, float* dsink,
                             hipStream_t stream) {
  if (p.bf16)
    return p.d == 64 ? preprocess_t<__bf16, 64>(p, o, dout, lse, sink, delta, dq_accum, dsink, stream)
                     : preprocess_t<__bf16, 128>(p, o, dout, lse, sink, delta, dq_accum, dsink, stream);
  return p.d == 64 ? preprocess_t<_Float16, 64>(p, o, dout, lse, sink, delta, dq_accum, dsink, stream)
                   : preprocess_t<_Float16, 128>(p, o, dout, lse, sink, delta, dq_accum, dsink, stream);
}

hipError_t launch_postprocess(const Problem& p, const float* dq_accum, void* dq,
                              hipStream_t stream) {
  const size_t n8 = (size_t)p.total * p.hq * p.d / 8;
  const dim3 grid((unsigned)((n8 + 255) / 256));
  if (p.bf16)
    hipLaunchKernelGGL(cast_kernel<__bf16>, grid, dim3(256), 0, stream, dq_accum,
                       static_cast<__bf16*>(dq), n8, p.scale);
  else
    hipLaunchKernelGGL(cast_kernel<_Float16>, grid, dim3(256), 0, stream, dq_accum,
                       static_cast<_Float16*>(dq), n8, p.scale);
  return hipGetLastError();
}

hipError_t launch_dkv_reduce(const Problem& p, const float* dkv_part, int nsplit, void* dk,
                             void* dv, hipStream_t stream) {
  const size_t n_kv = (size_t)p.total * p.hkv * p.d;
  const dim3 grid((unsigned)((n_kv / 8 + 255) / 256));
  if (p.bf16)
    hipLaunchKernelGGL(dkv_reduce_kernel<__bf16>, grid, dim3(256), 0, stream, dkv_part, nsplit,
                       n_kv, static_cast<__bf16*>(dk), static_cast<__bf16*>(dv));
  else
    hipLaunchKernelGGL(dkv_reduce_kernel<_Float16>, grid, dim3(256), 0, stream, dkv_part, nsplit,
                       n_kv, static_cast<_Float16*>(dk), static_cast<_Float16*>(dv));
  return hipGetLastError();
}

}  // namespace attn
