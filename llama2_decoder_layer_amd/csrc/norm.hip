// RMSNorm of prefill rows ("Llama2架构与推理全解析" §1.2): for each token row,
// u = x / sqrt(mean(x^2) + eps) * gamma, reduced in float32.  One workgroup
// per row; 16-byte loads; wavefront shuffles, then LDS across the 4 waves.
// (Decode folds the norm into its projections instead.)
#include "common.cuh"
#include "kernels.h"

namespace ll {

template <int DT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* x, const void* gamma, void* u,
                                                      int H, float eps) {
  typedef typename Elt<DT>::T T;
  constexpr int E = Elt<DT>::PER16;
  const int row = blockIdx.x;
  const T* xr = reinterpret_cast<const T*>(x) + (size_t)row * H;
  T* ur = reinterpret_cast<T*>(u) + (size_t)row * H;
  const T* g = reinterpret_cast<const T*>(gamma);
  const int nch = H / E;
  float ss = 0.f;
  for (int c = threadIdx.x; c < nch; c += 256) {
    float f[E];
    unpack16<DT>(ld16(xr + c * E), f);
#pragma unroll
    for (int e = 0; e < E; ++e) ss += f[e] * f[e];
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  for (int c = threadIdx.x; c < nch; c += 256) {
    float f[E], gf[E];
    unpack16<DT>(ld16(xr + c * E), f);
    unpack16<DT>(ld16(g + c * E), gf);
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = f[e] * inv * gf[e];
    st16(ur + c * E, pack16<DT>(f));
  }
}

hipError_t launch_rmsnorm(int dt, const void* x, const void* gamma, void* u, int rows, int H,
                          float eps, hipStream_t s) {
  switch (dt) {
    case DT_F32: LL_LAUNCH(rmsnorm_kernel<DT_F32>, dim3(rows), dim3(256), 0, s, x, gamma, u, H, eps); break;
    case DT_BF16: LL_LAUNCH(rmsnorm_kernel<DT_BF16>, dim3(rows), dim3(256), 0, s, x, gamma, u, H, eps); break;
    default: LL_LAUNCH(rmsnorm_kernel<DT_F16>, dim3(rows), dim3(256), 0, s, x, gamma, u, H, eps); break;
  }
  return hipGetLastError();
}

}  // namespace ll
