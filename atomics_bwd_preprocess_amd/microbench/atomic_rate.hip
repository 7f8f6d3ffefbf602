// Device-wide rate of device-scope fp32 atomic adds on gfx950: the roof of
// the backward pass's dQ accumulation.  Not part of the attention ABI; the
// benchmark script loads it to measure that roof on the machine it runs on.
//
// Every wave adds to one 256-byte segment (64 consecutive floats, one lane
// each) per iteration, issued as a no-return buffer atomic like the main
// kernel's; the segments walk the buffer so no address is hot.  Bytes moved
// = 4 x threads x iterations.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void atomic_rate_kernel(float* buf, uint32_t nseg, int iters) {
  const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
  const uint32_t nwaves = (gridDim.x * 256u) >> 6;
  const uint32_t lane = threadIdx.x & 63u;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(buf, (short)0, (int)(nseg * 256u), 0x00020000);
  for (int k = 0; k < iters; ++k) {
    const uint32_t seg = (wave + (uint32_t)k * nwaves) % nseg;
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(1.0f, r, seg * 256u + lane * 4u, 0, 0);
  }
}

}  // namespace

// buf: device buffer of at least nseg * 64 floats (nseg * 256 < 2^31);
// blocks: workgroups of 256 threads.  Returns 0 or a hipError_t.
extern "C" int attn_microbench_atomic_rate(float* buf, uint32_t nseg, int blocks, int iters,
                                           hipStream_t stream) {
  if (buf == nullptr || nseg == 0 || (uint64_t)nseg * 256u >= (1ull << 31) || blocks <= 0 ||
      iters <= 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(atomic_rate_kernel, dim3(blocks), dim3(256), 0, stream, buf, nseg, iters);
  return (int)hipGetLastError();
}
