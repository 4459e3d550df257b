// AdamW for the non-matrix tensors and the pointer-table patch.
//
// The PaperDaily post on "Scaling Muon for Diffusion Transformers" (section
// "From 1.3B to 15B") keeps biases and normalisation parameters on AdamW
// while 2-D weights take the matrix-aware update; AdamW itself is the
// decoupled-weight-decay method of the post's reference [3].
#include <hip/hip_runtime.h>

#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_g(const void* g, int gdt, int64_t idx) {
  if (gdt == 1) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(g)[idx]) << 16);
  return static_cast<const float*>(g)[idx];
}

// One workgroup per chunk of up to kAdamChunk elements of one tensor.
// m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
// p = p (1 - lr wd) - lr (m / bc1) / (sqrt(v / bc2) + eps),
// bc1 = 1 - b1^(t+1), bc2 = 1 - b2^(t+1) supplied by the host.
__global__ __launch_bounds__(kThreads) void adamw_kernel(
    const AdamDev* __restrict__ ts, const AdamChunk* __restrict__ chunks, float lr, float b1,
    float b2, float eps, float wd, float bc1, float bc2) {
  const AdamChunk ck = chunks[blockIdx.x];
  const AdamDev t = ts[ck.tensor];
  const float keep = 1.0f - lr * wd;
  const float inv_bc1 = 1.0f / bc1, inv_bc2 = 1.0f / bc2;
  for (int i = threadIdx.x; i < ck.len; i += kThreads) {
    const int64_t e = ck.off + i;
    const float g = load_g(t.g, t.gdt, e);
    const float m = fmaf(b1, t.m[e], (1.0f - b1) * g);
    const float v = fmaf(b2, t.v[e], (1.0f - b2) * g * g);
    t.m[e] = m;
    t.v[e] = v;
    const float denom = sqrtf(v * inv_bc2) + eps;
    t.p[e] = fmaf(-lr, (m * inv_bc1) / denom, t.p[e] * keep);
  }
}

__global__ void patch_kernel(MatDev* __restrict__ mats, AdamDev* __restrict__ adams,
                             PatchArgs args) {
  const int k = threadIdx.x;
  if (k >= args.count) return;
  if (args.adam) {
    adams[args.idx[k]].p = static_cast<float*>(args.w[k]);
    adams[args.idx[k]].g = args.g[k];
  } else {
    mats[args.idx[k]].w = static_cast<float*>(args.w[k]);
    mats[args.idx[k]].g = args.g[k];
  }
}

}  // namespace

hipError_t launch_adamw(hipStream_t s, const AdamDev* t, const AdamChunk* chunks,
                        int64_t nchunks, float lr, float b1, float b2, float eps, float wd,
                        float bc1, float bc2) {
  if (nchunks <= 0) return hipSuccess;
  adamw_kernel<<<dim3(static_cast<unsigned>(nchunks)), dim3(kThreads), 0, s>>>(
      t, chunks, lr, b1, b2, eps, wd, bc1, bc2);
  return hipGetLastError();
}

hipError_t launch_patch(hipStream_t s, MatDev* mats, AdamDev* adams, const PatchArgs& args) {
  if (args.count <= 0) return hipSuccess;
  patch_kernel<<<dim3(1), dim3(64), 0, s>>>(mats, adams, args);
  return hipGetLastError();
}

}  // namespace muon
