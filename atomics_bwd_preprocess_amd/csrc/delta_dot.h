// Delta's 8-element dot product, shared by the backward preprocess and the
// query-stationary dQ pass (which can form Delta itself).
#pragma once

#include "common.h"

namespace attn {

// acc + a . b over 8 elements, two per v_dot2_f32_{f16,bf16} (exact 16-bit
// products, fp32 accumulation), in a fixed order.  Written with the dot2
// builtins rather than as `acc += a[i] * b[i]` so that every instantiation
// of the delta kernel (with or without zeroing the accumulator) computes Delta
// with the same instructions: left to the compiler, the loop was lowered to
// dot2 in one build and to FMA chains in another, and the two backward paths
// read Delta from different instantiations (dK / dV must agree bit for bit).
// The query-stationary dQ pass can also form Delta (attn_bwd_dq_delta) with
// this same function and the preprocess's summation order.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8(f16x8 a, f16x8 b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2_t x = {a[2 * i], a[2 * i + 1]}, y = {b[2 * i], b[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2(x, y, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float dot8(bf16x8 a, bf16x8 b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_t x = {a[2 * i], a[2 * i + 1]}, y = {b[2 * i], b[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
  }
  return acc;
}

}  // namespace attn
