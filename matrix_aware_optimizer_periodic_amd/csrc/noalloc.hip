// Device scratch of muon_step_noalloc: one file-scope array per device, for
// callers that cannot allocate device memory.
//
// The array holds what muon_step keeps in the caller's state buffer apart
// from the momentum: launch tables, the Newton-Schulz workspace of a chunk
// of matrices, the RowNorm column partials and the cross-workgroup counters.
// Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` only stands in for the symbol: its device address
// comes from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address is ever passed to kernels or copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "muon_internal.h"

namespace muon {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_fill_zero(hipStream_t s, void* p, size_t bytes) {
  if (bytes == 0) return hipSuccess;
  const int64_t words = int64_t(bytes / 4);
  const int64_t blocks = (words + 255) / 256;
  fill_zero_kernel<<<dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s>>>(
      static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace muon
