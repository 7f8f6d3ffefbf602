// Library-owned scratch memory for callers that cannot allocate.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, from module load until the process ends.  Its device address
// is taken once per device with hipGetSymbolAddress and kept; host code never
// passes the array's name to a kernel (on the host that name is a stand-in,
// not a device address).  Calls on one device share the array, so calls
// that overlap on one GPU race; the entry point clears what must start at
// zero on every call.
#include <mutex>

#include "launch.h"

namespace attn {

namespace {

constexpr size_t kScratchFloats = kStaticScratchBytes / sizeof(float);
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_ptr[kMaxDevices] = {};

// Zero n floats (n a multiple of 4) with 16-byte stores.
__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ p, size_t n4) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t static_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

hipError_t launch_zero(float* p, size_t n, hipStream_t stream) {
  const size_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const size_t want = (n4 + 255) / 256;
  const unsigned blocks = (unsigned)(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

}  // namespace attn
