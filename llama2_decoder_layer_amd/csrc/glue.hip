// Small kernels around the layer: RoPE angle tables, embedding gather, the
// greedy pick over logits and the per-row int8 weight quantiser.
#include "common.cuh"
#include "kernels.h"

namespace ll {

// cos/sin(m * theta^(-2i/hd)) in float64, rounded once to float32
// ("Llama2架构与推理全解析" §1.4: each dimension pair turns at its own rate).
__global__ void rope_table_kernel(float* c, float* sn, int max_pos, int hd, double theta) {
  const int half = hd / 2;
  const size_t total = (size_t)max_pos * half;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(idx / half);
    const int i = (int)(idx - (size_t)m * half);
    const double inv = pow(theta, -2.0 * (double)i / (double)hd);
    const double ang = (double)m * inv;
    c[idx] = (float)cos(ang);
    sn[idx] = (float)sin(ang);
  }
}

hipError_t launch_rope_table(float* c, float* sn, int max_pos, int hd, double theta, hipStream_t s) {
  const size_t total = (size_t)max_pos * (hd / 2);
  int grid = (int)((total + 255) / 256);
  if (grid > 4096) grid = 4096;
  LL_LAUNCH(rope_table_kernel, dim3(grid), dim3(256), 0, s, c, sn, max_pos, hd, theta);
  return hipGetLastError();
}

// h[i, :] = table[ids[i], :]   (ids clamped into [0, vocab)).
__global__ void embed_kernel(const uint8_t* table, const int32_t* ids, uint8_t* h, int row_bytes,
                             int vocab) {
  int id = ids[blockIdx.x];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
  const uint8_t* src = table + (size_t)id * row_bytes;
  uint8_t* dst = h + (size_t)blockIdx.x * row_bytes;
  for (int c = threadIdx.x; c < row_bytes / 16; c += blockDim.x) st16(dst + c * 16, ld16(src + c * 16));
}

hipError_t launch_embed(const void* table, const int32_t* ids, void* h, int n, int H, int vocab,
                        int dt, hipStream_t s) {
  const int row_bytes = H * (dt == DT_F32 ? 4 : 2);
  LL_LAUNCH(embed_kernel, dim3(n), dim3(256), 0, s, (const uint8_t*)table, ids, (uint8_t*)h,
                     row_bytes, vocab);
  return hipGetLastError();
}

// ids[i] = argmax_v logits[i, v]; ties go to the lowest index.  One
// workgroup of 1024 threads per row; each thread keeps eight loads in flight
// (elements v, v + 1024, ... of a 8192-element window), so a 32000-token row
// takes four round trips instead of 125 dependent ones.
constexpr int ARGMAX_THREADS = 1024;
constexpr int ARGMAX_UNROLL = 8;

__global__ __launch_bounds__(ARGMAX_THREADS) void argmax_kernel(const float* logits, int32_t* ids,
                                                                int vocab) {
  const float* r = logits + (size_t)blockIdx.x * vocab;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int v0 = threadIdx.x; v0 < vocab; v0 += ARGMAX_THREADS * ARGMAX_UNROLL) {
    float x[ARGMAX_UNROLL];
#pragma unroll
    for (int u = 0; u < ARGMAX_UNROLL; ++u) {
      const int v = v0 + u * ARGMAX_THREADS;
      x[u] = v < vocab ? r[v] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < ARGMAX_UNROLL; ++u)  // increasing index: the first hit of a value is the lowest
      if (x[u] > best) { best = x[u]; bi = v0 + u * ARGMAX_THREADS; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  constexpr int NW = ARGMAX_THREADS / 64;
  __shared__ float sb[NW];
  __shared__ int si[NW];
  if ((threadIdx.x & 63) == 0) { sb[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < NW; ++w)
      if (sb[w] > best || (sb[w] == best && si[w] < bi)) { best = sb[w]; bi = si[w]; }
    ids[blockIdx.x] = bi == 0x7fffffff ? 0 : bi;
  }
}

hipError_t launch_argmax(const float* logits, int32_t* ids, int n, int vocab, hipStream_t s) {
  LL_LAUNCH(argmax_kernel, dim3(n), dim3(ARGMAX_THREADS), 0, s, logits, ids, vocab);
  return hipGetLastError();
}

// Copy of positions [start, start + count) of contiguous caches into the
// pools of a paged cache, 16 bytes per thread; grid: (rows of 16-byte chunks,
// sequence * nkv).
__global__ __launch_bounds__(256) void kv_pages_write_kernel(const uint8_t* ks, const uint8_t* vs,
                                                             int s_max, int start, int count,
                                                             uint8_t* kp, uint8_t* vp, KvPages pg,
                                                             int nkv, int hd, int esz) {
  const int bj = blockIdx.y, b = bj / nkv, j = bj - b * nkv;
  const int cpr = hd * esz / 16;  // 16-byte chunks per row
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= count * cpr) return;
  const int t = idx / cpr, c = idx - t * cpr;
  const int pos = start + t;
  const size_t src = ((((size_t)b * nkv + j) * s_max + pos) * hd) * esz + (size_t)c * 16;
  const size_t dst = kv_row(pg, b, j, pos, nkv, 0, hd) * esz + (size_t)c * 16;
  st16(kp + dst, ld16(ks + src));
  st16(vp + dst, ld16(vs + src));
}

hipError_t launch_kv_pages_write(const void* k_src, const void* v_src, int s_max, int start,
                                 int count, void* k_pool, void* v_pool, const KvPages& pg,
                                 int batch, int nkv, int hd, int kv_dt, hipStream_t s) {
  const int esz = kv_dt == DT_F32 ? 4 : 2;
  const int n = count * (hd * esz / 16);
  LL_LAUNCH(kv_pages_write_kernel, dim3((n + 255) / 256, batch * nkv), dim3(256), 0, s,
            (const uint8_t*)k_src, (const uint8_t*)v_src, s_max, start, count, (uint8_t*)k_pool,
            (uint8_t*)v_pool, pg, nkv, hd, esz);
  return hipGetLastError();
}

// Weight-only int8 by rows: scale = max|w| / 127, q = rint(w / scale) in
// [-127, 127] (a zero row: scale 0, codes 0).  One workgroup per row; the
// division is the correctly rounded float32 one.
template <int DT>
__global__ __launch_bounds__(256) void quantize_w8_kernel(const void* w, int8_t* q, float* scale,
                                                          int cols) {
  typedef typename Elt<DT>::T T;
  __shared__ float red[4];
  const T* r = reinterpret_cast<const T*>(w) + (size_t)blockIdx.x * cols;
  int8_t* qr = q + (size_t)blockIdx.x * cols;
  float m = 0.f;
  for (int c = threadIdx.x; c < cols; c += 256) m = fmaxf(m, fabsf(Elt<DT>::to_f32(r[c])));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(m, 127.0f);
  if (threadIdx.x == 0) scale[blockIdx.x] = s;
  for (int c = threadIdx.x; c < cols; c += 256) {
    float v = 0.f;
    if (s > 0.f) v = fminf(127.f, fmaxf(-127.f, rintf(__fdiv_rn(Elt<DT>::to_f32(r[c]), s))));
    qr[c] = (int8_t)(int)v;
  }
}

// Weight-only int4 by rows: scale = max|w| / 7, code = rint(w / scale)
// clipped to [-7, 7] (a zero row: scale 0, codes 0), packed two to a byte:
// weight 2j in the low nibble of byte j, weight 2j + 1 in the high one.
template <int DT>
__global__ __launch_bounds__(256) void quantize_w4_kernel(const void* w, uint8_t* q, float* scale,
                                                          int cols) {
  typedef typename Elt<DT>::T T;
  __shared__ float red[4];
  const T* r = reinterpret_cast<const T*>(w) + (size_t)blockIdx.x * cols;
  uint8_t* qr = q + (size_t)blockIdx.x * (cols / 2);
  float m = 0.f;
  for (int c = threadIdx.x; c < cols; c += 256) m = fmaxf(m, fabsf(Elt<DT>::to_f32(r[c])));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(m, 7.0f);
  if (threadIdx.x == 0) scale[blockIdx.x] = s;
  auto code = [&](int c) -> uint32_t {
    float v = 0.f;
    if (s > 0.f) v = fminf(7.f, fmaxf(-7.f, rintf(__fdiv_rn(Elt<DT>::to_f32(r[c]), s))));
    return (uint32_t)(int)v & 15u;
  };
  for (int j = threadIdx.x; j < cols / 2; j += 256)
    qr[j] = (uint8_t)(code(2 * j) | (code(2 * j + 1) << 4));
}

hipError_t launch_quantize_w4(int dt, const void* w, uint8_t* q, float* scale, int rows, int cols,
                              hipStream_t s) {
  if (dt == DT_F32)
    LL_LAUNCH(quantize_w4_kernel<DT_F32>, dim3(rows), dim3(256), 0, s, w, q, scale, cols);
  else if (dt == DT_BF16)
    LL_LAUNCH(quantize_w4_kernel<DT_BF16>, dim3(rows), dim3(256), 0, s, w, q, scale, cols);
  else
    LL_LAUNCH(quantize_w4_kernel<DT_F16>, dim3(rows), dim3(256), 0, s, w, q, scale, cols);
  return hipGetLastError();
}

hipError_t launch_quantize_w8(int dt, const void* w, int8_t* q, float* scale, int rows, int cols,
                              hipStream_t s) {
  if (dt == DT_F32)
    LL_LAUNCH(quantize_w8_kernel<DT_F32>, dim3(rows), dim3(256), 0, s, w, q, scale, cols);
  else if (dt == DT_BF16)
    LL_LAUNCH(quantize_w8_kernel<DT_BF16>, dim3(rows), dim3(256), 0, s, w, q, scale, cols);
  else
    LL_LAUNCH(quantize_w8_kernel<DT_F16>, dim3(rows), dim3(256), 0, s, w, q, scale, cols);
  return hipGetLastError();
}

}  // namespace ll
