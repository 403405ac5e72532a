// RMSNorm of prefill rows ("Llama2架构与推理全解析" §1.2): for each token row,
// u = x / sqrt(mean(x^2) + eps) * gamma, reduced in float32.  One workgroup
// per row; 16-byte loads; wavefront shuffles, then LDS across the 4 waves.
// (Decode at 1-4 tokens folds the norm into its projections instead.)
#include "common.cuh"
#include "kernels.h"

namespace ll {

// NC > 0: each thread holds its (at most NC) 16-byte chunks of the row and of
// gamma in registers, all loaded before the first use, so a row costs one
// round trip to memory and is read once.  NC = 0: any width, in two passes.
template <int DT, int NC>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* x, const void* gamma, void* u,
                                                      int H, float eps) {
  typedef typename Elt<DT>::T T;
  constexpr int E = Elt<DT>::PER16;
  const int row = blockIdx.x;
  const T* xr = reinterpret_cast<const T*>(x) + (size_t)row * H;
  T* ur = reinterpret_cast<T*>(u) + (size_t)row * H;
  const T* g = reinterpret_cast<const T*>(gamma);
  const int nch = H / E;
  __shared__ float part[4];
  float ss = 0.f;
  if constexpr (NC > 0) {
    u32x4 xv[NC], gv[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (c < nch) {
        xv[i] = ld16(xr + c * E);
        gv[i] = ld16(g + c * E);
      }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (threadIdx.x + 256 * i < nch) {
        float f[E];
        unpack16<DT>(xv[i], f);
#pragma unroll
        for (int e = 0; e < E; ++e) ss += f[e] * f[e];
      }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = part[0] + part[1] + part[2] + part[3];
    const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (c < nch) {
        float f[E], gf[E];
        unpack16<DT>(xv[i], f);
        unpack16<DT>(gv[i], gf);
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = f[e] * inv * gf[e];
        st16(ur + c * E, pack16<DT>(f));
      }
    }
  } else {
    for (int c = threadIdx.x; c < nch; c += 256) {
      float f[E];
      unpack16<DT>(ld16(xr + c * E), f);
#pragma unroll
      for (int e = 0; e < E; ++e) ss += f[e] * f[e];
    }
    ss = wave_sum(ss);
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
}

template <int DT>
static hipError_t rmsnorm_launch(const void* x, const void* gamma, void* u, int rows, int H,
                                 float eps, hipStream_t s) {
  const int per_thread = (H / Elt<DT>::PER16 + 255) / 256;
  const dim3 grid(rows), block(256);
  if (per_thread <= 1) LL_LAUNCH((rmsnorm_kernel<DT, 1>), grid, block, 0, s, x, gamma, u, H, eps);
  else if (per_thread <= 2) LL_LAUNCH((rmsnorm_kernel<DT, 2>), grid, block, 0, s, x, gamma, u, H, eps);
  else if (per_thread <= 4) LL_LAUNCH((rmsnorm_kernel<DT, 4>), grid, block, 0, s, x, gamma, u, H, eps);
  else if (per_thread <= 8) LL_LAUNCH((rmsnorm_kernel<DT, 8>), grid, block, 0, s, x, gamma, u, H, eps);
  else LL_LAUNCH((rmsnorm_kernel<DT, 0>), grid, block, 0, s, x, gamma, u, H, eps);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dt, const void* x, const void* gamma, void* u, int rows, int H,
                          float eps, hipStream_t s) {
  switch (dt) {
    case DT_F32: return rmsnorm_launch<DT_F32>(x, gamma, u, rows, H, eps, s);
    case DT_BF16: return rmsnorm_launch<DT_BF16>(x, gamma, u, rows, H, eps, s);
    default: return rmsnorm_launch<DT_F16>(x, gamma, u, rows, H, eps, s);
  }
}

}  // namespace ll
