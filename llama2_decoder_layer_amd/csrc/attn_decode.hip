// Attention of single queries over the KV cache, split over context.
//
// One workgroup takes (query, KV head j, group of GC query heads that share j,
// chunk of positions).  It streams its chunk of K and V for head j once from
// HBM and serves all GC query heads from registers, so a GQA group costs one
// pass over its cache instead of GC.  HD/8 lanes cooperate on one key (8
// elements each).  Scores are kept in the log2 domain (q is pre-scaled by
// log2(e)/sqrt(head_dim)) so exp2 does the softmax.  Each split writes its
// running max m, sum l and unnormalised acc; attn_combine merges the splits
// (log-sum-exp) and writes o in the activation format.
#include "common.cuh"
#include "kernels.h"

namespace ll {

constexpr int CHUNK_MAX = 512;

__device__ __forceinline__ int query_position(const AttnDecodeArgs& a, int n, int* b_out) {
  const int b = n / a.T;
  *b_out = b;
  if (a.ctx_len) {
    int p = a.ctx_len[b];
    return p < 0 ? 0 : (p > a.max_ctx ? a.max_ctx : p);
  }
  return a.start_pos + (n - b * a.T);
}

// 8 consecutive cache elements of one key, as floats.
template <int KVDT>
__device__ __forceinline__ void load8(const typename Elt<KVDT>::T* p, float* f) {
  if constexpr (KVDT == DT_F32) {
    unpack16<DT_F32>(ld16(p), f);
    unpack16<DT_F32>(ld16(p + 4), f + 4);
  } else {
    unpack16<KVDT>(ld16(p), f);
  }
}

template <int KVDT, int HD, int GC>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnDecodeArgs a) {
  typedef typename Elt<KVDT>::T T;
  constexpr int LPK = HD / 8;      // lanes per key
  constexpr int KPI = 256 / LPK;   // keys per workgroup iteration
  const int split = blockIdx.x;
  const int g = a.nh / a.nkv;
  const int per_kv = g / GC;
  const int j = blockIdx.y / per_kv;
  const int h0 = j * g + (blockIdx.y - j * per_kv) * GC;
  const int n = blockIdx.z;
  int b;
  const int pos = query_position(a, n, &b);
  const int k_lo = split * a.chunk;
  const int k_hi = min(k_lo + a.chunk, pos + 1);
  if (k_lo >= k_hi) return;  // past this query's context: the combine skips it
  const int cnt = k_hi - k_lo;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = tid % LPK, slot = tid / LPK;

  float qf[GC][8];
  const float qscale = 1.44269504088896341f / sqrtf((float)HD);
#pragma unroll
  for (int i = 0; i < GC; ++i) {
    const float* qp = a.q + ((size_t)n * a.nh + h0 + i) * HD + sub * 8;
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(qp);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(qp + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[i][e] = q0[e] * qscale;
      qf[i][e + 4] = q1[e] * qscale;
    }
  }

  __shared__ float s_p[GC][CHUNK_MAX];
  __shared__ float s_m[GC], s_l[GC];
  __shared__ float s_acc[4][GC][HD];

  const size_t head_off = ((size_t)b * a.nkv + j) * a.s_max * HD + sub * 8;
  const T* kp = reinterpret_cast<const T*>(a.kc) + head_off;
  const T* vp = reinterpret_cast<const T*>(a.vc) + head_off;

  // Scores.
  for (int key = k_lo + slot; key < k_hi; key += KPI) {
    float kf[8];
    load8<KVDT>(kp + (size_t)key * HD, kf);
#pragma unroll
    for (int i = 0; i < GC; ++i) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d += qf[i][e] * kf[e];
#pragma unroll
      for (int o = LPK / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
      if (sub == 0) s_p[i][key - k_lo] = d;
    }
  }
  __syncthreads();

  // Softmax statistics of this chunk, one wave per head.
  for (int i = wave; i < GC; i += 4) {
    float mx = -INFINITY;
    for (int k = lane; k < cnt; k += 64) mx = fmaxf(mx, s_p[i][k]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int k = lane; k < cnt; k += 64) {
      const float p = exp2f(s_p[i][k] - mx);
      s_p[i][k] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      s_m[i] = mx;
      s_l[i] = sum;
    }
  }
  __syncthreads();

  // P V.
  float acc[GC][8];
#pragma unroll
  for (int i = 0; i < GC; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  for (int key = k_lo + slot; key < k_hi; key += KPI) {
    float vf[8];
    load8<KVDT>(vp + (size_t)key * HD, vf);
#pragma unroll
    for (int i = 0; i < GC; ++i) {
      const float p = s_p[i][key - k_lo];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] += p * vf[e];
    }
  }
  // Sum the key slots of each wave, then the four waves.
#pragma unroll
  for (int i = 0; i < GC; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) acc[i][e] += __shfl_xor(acc[i][e], o, 64);
  if (lane < LPK) {
#pragma unroll
    for (int i = 0; i < GC; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][i][sub * 8 + e] = acc[i][e];
  }
  __syncthreads();
  for (int idx = tid; idx < GC * HD; idx += 256) {
    const int i = idx / HD, d = idx - i * HD;
    const float v = s_acc[0][i][d] + s_acc[1][i][d] + s_acc[2][i][d] + s_acc[3][i][d];
    a.part_acc[(((size_t)n * a.nh + h0 + i) * a.nsplit + split) * HD + d] = v;
  }
  if (tid < GC) {
    const size_t pi = ((size_t)n * a.nh + h0 + tid) * a.nsplit + split;
    a.part_m[pi] = s_m[tid];
    a.part_l[pi] = s_l[tid];
  }
}

// o[n, h, :] = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s over the splits
// that hold part of query n's context.
template <int DT, int HD>
__global__ __launch_bounds__(HD) void attn_combine_kernel(AttnDecodeArgs a) {
  const int n = blockIdx.x / a.nh;
  const int h = blockIdx.x - n * a.nh;
  const int d = threadIdx.x;
  int b;
  const int pos = query_position(a, n, &b);
  const int nvalid = (pos + a.chunk) / a.chunk;  // ceil((pos + 1) / chunk)
  const size_t base = ((size_t)n * a.nh + h) * a.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < nvalid; ++s) M = fmaxf(M, a.part_m[base + s]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < nvalid; ++s) {
    const float w = exp2f(a.part_m[base + s] - M);
    L += w * a.part_l[base + s];
    acc += w * a.part_acc[(base + s) * HD + d];
  }
  typename Elt<DT>::T* o = reinterpret_cast<typename Elt<DT>::T*>(a.o);
  o[(size_t)n * a.nh * HD + h * HD + d] = Elt<DT>::from_f32(acc / L);
}

template <int KVDT, int HD>
static hipError_t split_launch(const AttnDecodeArgs& a, hipStream_t s) {
  const int g = a.nh / a.nkv;
  const int gc = (g % 8 == 0) ? 8 : (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
  dim3 grid(a.nsplit, a.nkv * (g / gc), a.nq);
  switch (gc) {
    case 8: hipLaunchKernelGGL((attn_split_kernel<KVDT, HD, 8>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_split_kernel<KVDT, HD, 4>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_split_kernel<KVDT, HD, 2>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((attn_split_kernel<KVDT, HD, 1>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int HD>
static hipError_t combine_launch(const AttnDecodeArgs& a, hipStream_t s) {
  dim3 grid(a.nq * a.nh);
  switch (a.act_dt) {
    case DT_F32: hipLaunchKernelGGL((attn_combine_kernel<DT_F32, HD>), grid, dim3(HD), 0, s, a); break;
    case DT_BF16: hipLaunchKernelGGL((attn_combine_kernel<DT_BF16, HD>), grid, dim3(HD), 0, s, a); break;
    default: hipLaunchKernelGGL((attn_combine_kernel<DT_F16, HD>), grid, dim3(HD), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t s) {
  if (a.chunk < 1 || a.chunk > CHUNK_MAX) return hipErrorInvalidValue;
  hipError_t e;
  if (a.hd == 128) {
    e = (a.kv_dt == DT_F32) ? split_launch<DT_F32, 128>(a, s)
      : (a.kv_dt == DT_BF16) ? split_launch<DT_BF16, 128>(a, s) : split_launch<DT_F16, 128>(a, s);
  } else {
    e = (a.kv_dt == DT_F32) ? split_launch<DT_F32, 64>(a, s)
      : (a.kv_dt == DT_BF16) ? split_launch<DT_BF16, 64>(a, s) : split_launch<DT_F16, 64>(a, s);
  }
  if (e != hipSuccess) return e;
  return a.hd == 128 ? combine_launch<128>(a, s) : combine_launch<64>(a, s);
}

}  // namespace ll
