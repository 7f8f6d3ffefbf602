// Host-side launchers of the gfx950 kernels (called by the C ABI in api.hip
// after argument validation).  Every launcher only enqueues on `stream` and
// returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn_bwd.h"

namespace attn {

struct Problem {
  int num_seqs, max_seqlen, total, hq, hkv, d;
  bool causal;
  int window;
  float scale;
  bool bf16;
  bool bhsd;  // [B, H, S, D] tensors (dense batch) instead of packed [T, H, D]
};

// Element offset of local row i of head h of the sequence that starts at
// token a, in a tensor with H heads of D elements: packed [T, H, D], or
// [B, H, S, D] (dense batch, a = b * S).  q, o, dout, dq and dq_accum use
// the query heads, k, v, dk and dv the kv heads.  Rows of one head are
// H * D elements apart when packed and D apart in [B, H, S, D].
template <int D, bool BHSD>
__host__ __device__ __forceinline__ size_t row_off(int a, int i, int h, int H, int S) {
  if constexpr (BHSD)
    return ((size_t)a * H + (size_t)h * S + i) * D;
  else
    return ((size_t)(a + i) * H + h) * D;
}

hipError_t launch_fwd(const Problem& p, const void* q, const void* k, const void* v,
                      const int32_t* cu, const float* sink, void* o, float* lse,
                      hipStream_t stream);

// dsink only (Delta already written), fixed-order reduction per head.
hipError_t launch_dsink(const Problem& p, const float* lse, const float* delta, const float* sink,
                        float* dsink, hipStream_t stream);

hipError_t launch_preprocess(const Problem& p, const void* o, const void* dout, const float* lse,
                             const float* sink, float* delta, float* dq_accum, float* dsink,
                             hipStream_t stream);

hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const void* dout, const float* lse, const float* delta,
                      const int32_t* cu, float* dq_accum, void* dk, void* dv,
                      hipStream_t stream);

// Main pass (causal problems) that also casts dQ: per (sequence, query
// head, query block) arrival counters (zeroed before the launch) let the last
// contributing workgroup of a block write scale * dq_accum into dq.
hipError_t launch_bwd_fused_cast(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dout, const float* lse, const float* delta,
                                const int32_t* cu, float* dq_accum, int* counters, void* dq,
                                void* dk, void* dv, hipStream_t stream);

// Main pass without its dQ product (dK / dV only).
hipError_t launch_bwd_dkdv(const Problem& p, const void* q, const void* k, const void* v,
                           const void* dout, const float* lse, const float* delta,
                           const int32_t* cu, void* dk, void* dv, hipStream_t stream);

// Query-stationary dQ pass (dQ written once in the storage dtype).  With o
// non-null it forms Delta from O and dO itself (written to delta_out) instead
// of reading delta.
hipError_t launch_bwd_dq(const Problem& p, const void* q, const void* k, const void* v,
                         const void* dout, const float* lse, const float* delta,
                         const int32_t* cu, void* dq, const void* o, float* delta_out,
                         hipStream_t stream);

// Main pass with the pairs of every key block split over nsplit workgroups;
// fp32 dK / dV partials into dkv_part (no dQ product when dq_accum is NULL).
hipError_t launch_bwd_split(const Problem& p, const void* q, const void* k, const void* v,
                            const void* dout, const float* lse, const float* delta,
                            const int32_t* cu, float* dq_accum, float* dkv_part, int nsplit,
                            hipStream_t stream);

// Sum of the nsplit partial slots, cast to dk / dv.
hipError_t launch_dkv_reduce(const Problem& p, const float* dkv_part, int nsplit, void* dk,
                             void* dv, hipStream_t stream);

hipError_t launch_postprocess(const Problem& p, const float* dq_accum, void* dq,
                              hipStream_t stream);

// Size of the library-owned scratch array (scratch.hip), in bytes.
constexpr size_t kStaticScratchBytes = ATTN_STATIC_SCRATCH_BYTES;

// Device address of this device's scratch array (taken on the first call on
// the device, then cached per device).
hipError_t static_scratch(float** ptr);

// Zero n floats at p (n a multiple of 4, p 16-byte aligned) with a fill kernel.
hipError_t launch_zero(float* p, size_t n, hipStream_t stream);

}  // namespace attn
