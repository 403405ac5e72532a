// Epilogue pieces shared by the projection kernels (GEMV and GEMM).
#pragma once

#include "common.cuh"
#include "kernels.h"

namespace ll {

// Store 4 consecutive values into a tensor whose format is only known at run time.
__device__ __forceinline__ void store4_rt(void* base, size_t idx, int dt, float a, float b,
                                          float c, float d) {
  if (dt == DT_F32) {
    store4<DT_F32>(reinterpret_cast<float*>(base) + idx, a, b, c, d);
  } else if (dt == DT_BF16) {
    store4<DT_BF16>(reinterpret_cast<uint16_t*>(base) + idx, a, b, c, d);
  } else {
    store4<DT_F16>(reinterpret_cast<uint16_t*>(base) + idx, a, b, c, d);
  }
}

// Position of global token n: decode reads ctx_len of its sequence (clamped to
// [0, max_ctx]); prefill counts from start_pos.
__device__ __forceinline__ int token_position(const ProjArgs& a, int b, int t) {
  if (a.ctx_len) {
    int p = a.ctx_len[b];
    return p < 0 ? 0 : (p > a.max_ctx ? a.max_ctx : p);
  }
  return a.start_pos + t;
}

// QKV epilogue for four consecutive output features f..f+3 (f % 4 == 0) of
// global token n (row nl of this launch).  Features [0, nh*hd) are q, then nkv*hd of k, then v.
// q and k pairs (2i, 2i+1) are turned by pos * theta_i using the float32
// cos/sin tables; k and v are written into the caches at `pos` (contiguous,
// or through the block table of a paged cache).
template <int DT>
__device__ __forceinline__ void qkv_epilogue4(const ProjArgs& a, int n, int nl, int f, float* v) {
  const int b = n / a.T;
  const int t = n - b * a.T;
  const int pos = token_position(a, b, t);
  const int hd = a.hd;
  const int qdim = a.nh * hd;
  const int kdim = a.nkv * hd;
  if (f < qdim + kdim) {
    const int d = (f < qdim ? f : f - qdim) % hd;
    const size_t ti = (size_t)pos * (hd >> 1) + (d >> 1);
    const float c0 = a.rcos[ti], s0 = a.rsin[ti], c1 = a.rcos[ti + 1], s1 = a.rsin[ti + 1];
    const float x0 = v[0], y0 = v[1], x1 = v[2], y1 = v[3];
    v[0] = x0 * c0 - y0 * s0;
    v[1] = x0 * s0 + y0 * c0;
    v[2] = x1 * c1 - y1 * s1;
    v[3] = x1 * s1 + y1 * c1;
  }
  if (f < qdim) {
    if (a.q32) {
      f32x4 q = {v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(a.q32 + (size_t)nl * qdim + f) = q;
    } else {
      const int h = f / hd, d = f - h * hd;
      const size_t idx = (((size_t)b * a.nh + h) * a.T + t) * hd + d;
      store4_rt(a.q16, idx, a.kv_dt, v[0], v[1], v[2], v[3]);
    }
  } else if (f < qdim + kdim) {
    const int j = (f - qdim) / hd, d = (f - qdim) - j * hd;
    const size_t idx = kv_row(a.pages, b, j, pos, a.nkv, a.s_max, hd) + d;
    store4_rt(a.kc, idx, a.kv_dt, v[0], v[1], v[2], v[3]);
  } else {
    const int j = (f - qdim - kdim) / hd, d = (f - qdim - kdim) - j * hd;
    const size_t idx = kv_row(a.pages, b, j, pos, a.nkv, a.s_max, hd) + d;
    store4_rt(a.vc, idx, a.kv_dt, v[0], v[1], v[2], v[3]);
  }
}

// Two values of runtime format dt at base + idx (idx even).
__device__ __forceinline__ void store2_rt(void* base, size_t idx, int dt, float a, float b) {
  if (dt == DT_F32) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(base) + idx) = v;
  } else {
    const uint32_t w = dt == DT_BF16 ? pack2<DT_BF16>(a, b) : pack2<DT_F16>(a, b);
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
  }
}

// The QKV epilogue for one RoPE pair: features f, f + 1 (f even).
template <int DT>
__device__ __forceinline__ void qkv_epilogue2(const ProjArgs& a, int n, int nl, int f, float* v) {
  const int b = n / a.T;
  const int t = n - b * a.T;
  const int pos = token_position(a, b, t);
  const int hd = a.hd;
  const int qdim = a.nh * hd;
  const int kdim = a.nkv * hd;
  if (f < qdim + kdim) {
    const int d = (f < qdim ? f : f - qdim) % hd;
    const size_t ti = (size_t)pos * (hd >> 1) + (d >> 1);
    const float c0 = a.rcos[ti], s0 = a.rsin[ti];
    const float x0 = v[0], y0 = v[1];
    v[0] = x0 * c0 - y0 * s0;
    v[1] = x0 * s0 + y0 * c0;
  }
  if (f < qdim) {
    if (a.q32) {
      store2_rt(a.q32, (size_t)nl * qdim + f, DT_F32, v[0], v[1]);
    } else {
      const int h = f / hd, d = f - h * hd;
      const size_t idx = (((size_t)b * a.nh + h) * a.T + t) * hd + d;
      store2_rt(a.q16, idx, a.kv_dt, v[0], v[1]);
    }
  } else if (f < qdim + kdim) {
    const int j = (f - qdim) / hd, d = (f - qdim) - j * hd;
    store2_rt(a.kc, kv_row(a.pages, b, j, pos, a.nkv, a.s_max, hd) + d, a.kv_dt, v[0], v[1]);
  } else {
    const int j = (f - qdim - kdim) / hd, d = (f - qdim - kdim) - j * hd;
    store2_rt(a.vc, kv_row(a.pages, b, j, pos, a.nkv, a.s_max, hd) + d, a.kv_dt, v[0], v[1]);
  }
}

// Weight row pointer for output feature f of a segmented projection.
template <typename T>
__device__ __forceinline__ const T* seg_row(const ProjArgs& a, int f) {
  if (f < a.seg1) return reinterpret_cast<const T*>(a.w[0]) + (size_t)f * a.K;
  if (f < a.seg2) return reinterpret_cast<const T*>(a.w[1]) + (size_t)(f - a.seg1) * a.K;
  return reinterpret_cast<const T*>(a.w[2]) + (size_t)(f - a.seg2) * a.K;
}

}  // namespace ll
