// Decode-sized projections: y[m, n] = sum_k act(x)[m, k] W[n, k] for up to 32
// tokens m, streaming every weight byte once from HBM.
//
// Weights sit on the MFMA "A" side (16 output features per tile) and tokens on
// the "B" side (16 per tile, padded with zeros), so the k-reduction is done by
// v_mfma_f32_16x16x32_{bf16,f16} (or four 16x16x4_f32 for float32) instead of
// cross-lane shuffles.  Lane l of a wave reads 64 contiguous bytes of weight
// row l%16 per k-block; the four lane groups l/16 cover 256 contiguous bytes,
// so each row segment is fetched whole.  The waves of a workgroup split K and
// meet in LDS.
//
// Fusions: the attention / FFN RMSNorm is folded in (each lane accumulates
// sum x^2 of the slice it loads; the gain multiplies the B operand; 1/rms
// scales the result), and the epilogue does RoPE + the KV-cache append (QKV),
// the residual add (O, down), SwiGLU (gate/up) or float32 logits (LM head).
#include "common.cuh"
#include "epilogue.cuh"

namespace ll {

template <int DT, int EPI, bool NORM, int CT, int NW>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(ProjArgs a) {
  typedef typename Elt<DT>::T T;
  constexpr int E = Elt<DT>::PER16;   // elements per 16-byte chunk
  constexpr int KB = 16 * E;          // k per block: 4 lane groups x 4 chunks
  constexpr int NA = (EPI == EPI_SWIGLU) ? 2 : 1;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const int K = a.K;
  const int row0 = blockIdx.x * 16;

  // Weight rows of this lane (rows past N read row 0; their results are dropped).
  const int f_lane = row0 + r16;
  const int f_safe = f_lane < a.N ? f_lane : 0;
  const T* wp[NA];
  if constexpr (EPI == EPI_SWIGLU) {
    wp[0] = reinterpret_cast<const T*>(a.w[0]) + (size_t)f_safe * K;
    wp[1] = reinterpret_cast<const T*>(a.w[1]) + (size_t)f_safe * K;
  } else {
    wp[0] = seg_row<T>(a, f_safe);
  }
  // Token rows of this lane.
  const T* xp[CT];
  bool tv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int m = ct * 16 + r16;
    tv[ct] = m < a.M;
    xp[ct] = reinterpret_cast<const T*>(a.x) + (size_t)(tv[ct] ? m : 0) * K;
  }
  const T* gp = reinterpret_cast<const T*>(a.gamma);

  const int nkb = (K + KB - 1) / KB;
  const int kb0 = (nkb * wave) / NW;
  const int kb1 = (nkb * (wave + 1)) / NW;

  f32x4 acc[NA][CT];
#pragma unroll
  for (int n = 0; n < NA; ++n)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[n][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ssq[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) ssq[ct] = 0.f;

  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 wa[2][NA][4];
  // Software pipeline: weights of block kb+1 are in flight while kb is consumed.
  auto load_w = [&](int buf, int kb) {
    const int kbase = kb * KB + kg * 4 * E;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kbase + s * E;
#pragma unroll
      for (int n = 0; n < NA; ++n) wa[buf][n][s] = (k < K) ? ld16(wp[n] + k) : zero;
    }
  };
  if (kb0 < kb1) load_w(0, kb0);
  int buf = 0;
  for (int kb = kb0; kb < kb1; ++kb) {
    if (kb + 1 < kb1) load_w(buf ^ 1, kb + 1);
    const int kbase = kb * KB + kg * 4 * E;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kbase + s * E;
      const bool inb = k < K;
      u32x4 gv = zero;
      if constexpr (NORM) gv = inb ? ld16(gp + k) : zero;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        u32x4 xv = (inb && tv[ct]) ? ld16(xp[ct] + k) : zero;
        if constexpr (NORM) {
          float xf[E], gf[E];
          unpack16<DT>(xv, xf);
          unpack16<DT>(gv, gf);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            ssq[ct] += xf[e] * xf[e];
            xf[e] *= gf[e];
          }
          xv = pack16<DT>(xf);
        }
#pragma unroll
        for (int n = 0; n < NA; ++n) acc[n][ct] = mfma16_chunk<DT>(wa[buf][n][s], xv, acc[n][ct]);
      }
    }
    buf ^= 1;
  }

  // Cross-wave reduction.
  __shared__ f32x4 red[NW > 1 ? NW - 1 : 1][NA * CT][64];
  __shared__ float ssq_s[NW][CT * 16];
  if constexpr (NORM) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float v = ssq[ct];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (kg == 0) ssq_s[wave][ct * 16 + r16] = v;
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int n = 0; n < NA; ++n)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) red[wave - 1][n * CT + ct][lane] = acc[n][ct];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < NW; ++w)
#pragma unroll
    for (int n = 0; n < NA; ++n)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[n][ct] += red[w - 1][n * CT + ct][lane];

  // Epilogue: lane holds token column r16 (+16 ct), features row0 + kg*4 + 0..3.
  const int f = row0 + kg * 4;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int m = ct * 16 + r16;
    if (m >= a.M) continue;
    float scale = 1.f;
    if constexpr (NORM) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += ssq_s[w][ct * 16 + r16];
      scale = 1.0f / sqrtf(tot / (float)K + a.eps);
    }
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = acc[0][ct][i] * scale;
    if constexpr (EPI == EPI_LOGITS) {
      float* y = reinterpret_cast<float*>(a.y) + (size_t)m * a.N;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (f + i < a.N) y[f + i] = v[i];
    } else {
      if (f >= a.N) continue;  // N is a multiple of 4 for these epilogues
      if constexpr (EPI == EPI_RESID) {
        const T* r = reinterpret_cast<const T*>(a.resid) + (size_t)m * a.N + f;
        float rv[4];
        load4<DT>(r, rv);
        T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
        store4<DT>(y, rv[0] + v[0], rv[1] + v[1], rv[2] + v[2], rv[3] + v[3]);
      } else if constexpr (EPI == EPI_SWIGLU) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = silu(v[i]) * (acc[1][ct][i] * scale);
        T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
        store4<DT>(y, o[0], o[1], o[2], o[3]);
      } else {  // EPI_QKV
        qkv_epilogue4<DT>(a, a.tok0 + m, m, f, v);
      }
    }
  }
}

template <int DT, int EPI, bool NORM>
static hipError_t gemv_dispatch(const ProjArgs& a, hipStream_t s) {
  const int grid = (a.N + 15) / 16;
  const bool wide = grid <= 512;  // few row tiles: split K over 8 waves instead of 4
  if (a.M <= 16) {
    if (wide) hipLaunchKernelGGL((gemv_kernel<DT, EPI, NORM, 1, 8>), dim3(grid), dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gemv_kernel<DT, EPI, NORM, 1, 4>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (wide) hipLaunchKernelGGL((gemv_kernel<DT, EPI, NORM, 2, 8>), dim3(grid), dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gemv_kernel<DT, EPI, NORM, 2, 4>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int DT>
static hipError_t gemv_dt(int epi, const ProjArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_QKV: return gemv_dispatch<DT, EPI_QKV, true>(a, s);
    case EPI_RESID: return gemv_dispatch<DT, EPI_RESID, false>(a, s);
    case EPI_SWIGLU: return gemv_dispatch<DT, EPI_SWIGLU, true>(a, s);
    case EPI_LOGITS: return gemv_dispatch<DT, EPI_LOGITS, true>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(int dt, int epi, const ProjArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 32) return hipErrorInvalidValue;
  switch (dt) {
    case DT_F32: return gemv_dt<DT_F32>(epi, a, s);
    case DT_BF16: return gemv_dt<DT_BF16>(epi, a, s);
    case DT_F16: return gemv_dt<DT_F16>(epi, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ll
