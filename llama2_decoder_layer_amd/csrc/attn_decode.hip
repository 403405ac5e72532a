// Attention of single queries over the KV cache, split over context.
//
// One workgroup takes (query, KV head j, group of GC query heads that share j,
// chunk of positions).  It streams its chunk of K and V for head j once from
// HBM and serves all GC query heads from registers, so a GQA group costs one
// pass over its cache instead of GC.  HD/8 lanes cooperate on one key (8
// elements each); every thread issues the loads of all its keys (KPT of K and
// KPT of V) before using any, so a whole chunk is in flight at once.  Scores
// are kept in the log2 domain (q is pre-scaled by log2(e)/sqrt(head_dim)) so
// exp2 does the softmax.  Each split writes its running max m, sum l and
// unnormalised acc.
//
// attn_merge then combines the splits of one (query, head group) with
// log-sum-exp weights, o = sum 2^(m_s-M) acc_s / sum 2^(m_s-M) l_s, in a short
// second launch: the weights go to LDS in one parallel pass and the splits are
// summed by independent thread groups.  (Merging in the last-arriving split
// workgroup instead needs a device-scope release fence per workgroup, whose
// L2 write-back costs far more than a launch.)
#include "common.cuh"
#include "kernels.h"

namespace ll {

__device__ __forceinline__ int query_position(const AttnDecodeArgs& a, int n, int* b_out) {
  const int b = n / a.T;
  *b_out = b;
  if (a.ctx_len) {
    int p = a.ctx_len[b];
    return p < 0 ? 0 : (p > a.max_ctx ? a.max_ctx : p);
  }
  return a.start_pos + (n - b * a.T);
}

template <int KVDT, int HD, int GC, int KPT>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnDecodeArgs a) {
  typedef typename Elt<KVDT>::T T;
  constexpr int LPK = HD / 8;                   // lanes per key
  constexpr int KPI = 256 / LPK;                // keys per workgroup pass
  constexpr int CHUNK = KPI * KPT;              // keys per split
  constexpr int NC = (KVDT == DT_F32) ? 2 : 1;  // 16-byte chunks per lane per key
  const int split = blockIdx.x;
  const int g = a.nh / a.nkv;
  const int per_kv = g / GC;
  const int j = blockIdx.y / per_kv;
  const int h0 = j * g + (blockIdx.y - j * per_kv) * GC;
  const int n = blockIdx.z;
  int b;
  const int pos = query_position(a, n, &b);
  const int k_lo = split * CHUNK;
  const int k_hi = min(k_lo + CHUNK, pos + 1);
  if (k_lo >= k_hi) return;  // past this query's context: not counted, not merged
  const int cnt = k_hi - k_lo;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = tid % LPK, slot = tid / LPK;

  // Issue every K and V load of this thread first.
  const size_t head_off = ((size_t)b * a.nkv + j) * a.s_max * HD + sub * 8;
  const T* kp = reinterpret_cast<const T*>(a.kc) + head_off;
  const T* vp = reinterpret_cast<const T*>(a.vc) + head_off;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 kr[KPT][NC], vr[KPT][NC];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = k_lo + slot + i * KPI;
    const bool ok = key < k_hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[i][c] = ok ? ld16(kp + (size_t)key * HD + c * (8 / NC)) : zero;
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = k_lo + slot + i * KPI;
    const bool ok = key < k_hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) vr[i][c] = ok ? ld16(vp + (size_t)key * HD + c * (8 / NC)) : zero;
  }

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

  __shared__ float s_p[GC][CHUNK];
  __shared__ float s_m[GC], s_l[GC];
  __shared__ float s_acc[4][GC][HD];

  // Scores.
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    float kf[8];
#pragma unroll
    for (int c = 0; c < NC; ++c) unpack16<KVDT>(kr[i][c], kf + c * (8 / NC));
    const int kk = slot + i * KPI;
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d += qf[h][e] * kf[e];
#pragma unroll
      for (int o = LPK / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
      if (sub == 0 && kk < cnt) s_p[h][kk] = d;
    }
  }
  __syncthreads();

  // Softmax statistics of this chunk, one wave per head.
  for (int h = wave; h < GC; h += 4) {
    float mx = -INFINITY;
    for (int k = lane; k < cnt; k += 64) mx = fmaxf(mx, s_p[h][k]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int k = lane; k < cnt; k += 64) {
      const float p = exp2f(s_p[h][k] - mx);
      s_p[h][k] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      s_m[h] = mx;
      s_l[h] = sum;
    }
  }
  __syncthreads();

  // P V from the V rows already in registers.
  float acc[GC][8];
#pragma unroll
  for (int h = 0; h < GC; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int kk = slot + i * KPI;
    if (kk < cnt) {
      float vf[8];
#pragma unroll
      for (int c = 0; c < NC; ++c) unpack16<KVDT>(vr[i][c], vf + c * (8 / NC));
#pragma unroll
      for (int h = 0; h < GC; ++h) {
        const float p = s_p[h][kk];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] += p * vf[e];
      }
    }
  }
  // Sum the key slots of each wave, then the four waves.
#pragma unroll
  for (int h = 0; h < GC; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o, 64);
  if (lane < LPK) {
#pragma unroll
    for (int h = 0; h < GC; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][h][sub * 8 + e] = acc[h][e];
  }
  __syncthreads();
  for (int idx = tid; idx < GC * HD; idx += 256) {
    const int h = idx / HD, d = idx - h * HD;
    const float v = s_acc[0][h][d] + s_acc[1][h][d] + s_acc[2][h][d] + s_acc[3][h][d];
    a.part_acc[(((size_t)n * a.nh + h0 + h) * a.nsplit + split) * HD + d] = v;
  }
  if (tid < GC) {
    const size_t pi = ((size_t)n * a.nh + h0 + tid) * a.nsplit + split;
    a.part_m[pi] = s_m[tid];
    a.part_l[pi] = s_l[tid];
  }
}

// GQA variant for 16-bit caches with GC = 4 or 8 query heads per workgroup.
// The scores of a 16-key tile come from v_mfma_f32_16x16x32 with K in the A
// layout (lane: key r16, dims 32s + 8(l/16) of slice s, loaded straight from
// the cache as 64-byte row pieces) and the group's queries in the B layout
// (head r16; columns past GC are zero), so no cross-lane dot-product
// reductions are needed.  Each of the 4 waves scores KW = 16 TW keys; the
// workgroup's max comes through LDS, P = 2^(S - max) goes to LDS as
// [key][head], and P V runs on the VALU with each lane holding 8 dims of its
// V rows (V would need a transpose to be an MFMA operand).  Queries are
// rounded to the cache format for the MFMA.  Output: the same partials as
// attn_split_kernel, one split per CH = 64 TW keys.
template <int KVDT, int HD, int GC, int TW>
__global__ __launch_bounds__(256) void attn_gqa_kernel(AttnDecodeArgs a) {
  typedef typename Elt<KVDT>::T T;
  constexpr int NS = HD / 32;   // 32-dim slices: MFMAs per 16-key tile
  constexpr int KW = 16 * TW;   // keys per wave
  constexpr int CH = 4 * KW;    // keys per workgroup
  constexpr int DGN = HD / 8;   // 8-dim groups of a row
  constexpr int KG = 64 / DGN;  // V rows per wave load instruction
  constexpr int KPL = KW / KG;  // V rows per lane
  const int split = blockIdx.x;
  const int g = a.nh / a.nkv;
  const int per_kv = g / GC;
  const int j = blockIdx.y / per_kv;
  const int h0 = j * g + (blockIdx.y - j * per_kv) * GC;
  const int n = blockIdx.z;
  int b;
  const int pos = query_position(a, n, &b);
  const int k_lo = split * CH;
  const int k_hi = min(k_lo + CH, pos + 1);
  if (k_lo >= k_hi) return;  // past this query's context: not counted, not merged

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int kw0 = k_lo + wave * KW;
  const size_t head_off = ((size_t)b * a.nkv + j) * a.s_max * HD;
  const T* kp = reinterpret_cast<const T*>(a.kc) + head_off;
  const T* vp = reinterpret_cast<const T*>(a.vc) + head_off;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  u32x4 kr[TW][NS];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int key = kw0 + 16 * t + r16;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kr[t][s] = key < k_hi ? ld16(kp + (size_t)key * HD + 32 * s + 8 * g4) : zero;
  }
  const int vdg = lane % DGN, vkey = lane / DGN;
  u32x4 vr[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int key = kw0 + vkey + KG * i;
    vr[i] = key < k_hi ? ld16(vp + (size_t)key * HD + 8 * vdg) : zero;
  }

  const float qscale = 1.44269504088896341f / sqrtf((float)HD);
  u32x4 qb[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (r16 < GC) {
      const float* qp = a.q + ((size_t)n * a.nh + h0 + r16) * HD + 32 * s + 8 * g4;
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(qp);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(qp + 4);
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = q0[e] * qscale;
        f[e + 4] = q1[e] * qscale;
      }
      qb[s] = pack16<KVDT>(f);
    } else {
      qb[s] = zero;
    }
  }

  // Scores: lane holds head r16, keys 16t + 4 g4 + i of its wave.
  f32x4 sc[TW];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) c = mfma16_chunk<KVDT>(kr[t][s], qb[s], c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kw0 + 16 * t + 4 * g4 + i >= k_hi) c[i] = -INFINITY;
      mx = fmaxf(mx, c[i]);
    }
    sc[t] = c;
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  __shared__ float s_mx[4][16], s_l[4][16];
  __shared__ float s_p[CH][GC];
  __shared__ float s_acc[4][GC][HD];
  if (g4 == 0) s_mx[wave][r16] = mx;
  __syncthreads();
  // Wave 0 always holds a valid key, so the workgroup maximum is finite.
  const float M = fmaxf(fmaxf(s_mx[0][r16], s_mx[1][r16]), fmaxf(s_mx[2][r16], s_mx[3][r16]));
  float lsum = 0.f;
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2f(sc[t][i] - M);
      lsum += p;
      if (r16 < GC) s_p[wave * KW + 16 * t + 4 * g4 + i][r16] = p;
    }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (g4 == 0) s_l[wave][r16] = lsum;
  __syncthreads();

  // P V over this lane's V rows (rows past the context are zero, as is P).
  float acc[GC][8];
#pragma unroll
  for (int h = 0; h < GC; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int kl = wave * KW + vkey + KG * i;
    float vf[8];
    unpack16<KVDT>(vr[i], vf);
    float p[GC];
#pragma unroll
    for (int h = 0; h < GC; h += 4) {
      const f32x4 p4 = *reinterpret_cast<const f32x4*>(&s_p[kl][h]);
      p[h] = p4[0]; p[h + 1] = p4[1]; p[h + 2] = p4[2]; p[h + 3] = p4[3];
    }
#pragma unroll
    for (int h = 0; h < GC; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += p[h] * vf[e];
  }
#pragma unroll
  for (int h = 0; h < GC; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = DGN; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o, 64);
  if (lane < DGN) {
#pragma unroll
    for (int h = 0; h < GC; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][h][vdg * 8 + e] = acc[h][e];
  }
  __syncthreads();
  for (int idx = tid; idx < GC * HD; idx += 256) {
    const int h = idx / HD, d = idx - h * HD;
    const float v = s_acc[0][h][d] + s_acc[1][h][d] + s_acc[2][h][d] + s_acc[3][h][d];
    a.part_acc[(((size_t)n * a.nh + h0 + h) * a.nsplit + split) * HD + d] = v;
  }
  if (tid < GC) {
    const size_t pi = ((size_t)n * a.nh + h0 + tid) * a.nsplit + split;
    a.part_m[pi] = fmaxf(fmaxf(s_mx[0][tid], s_mx[1][tid]), fmaxf(s_mx[2][tid], s_mx[3][tid]));
    a.part_l[pi] = s_l[0][tid] + s_l[1][tid] + s_l[2][tid] + s_l[3][tid];
  }
}

// Merge of the splits of one (query, head group).  The 256 threads form
// HD/4 groups of 4 consecutive dims x 1024/HD split groups; each sums every
// (1024/HD)-th split with float4 loads, and the split groups meet in LDS.
template <int HD, int GC>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnDecodeArgs a) {
  constexpr int DG = HD / 4;    // 4-dim groups per head
  constexpr int SG = 256 / DG;  // split groups
  extern __shared__ float w_s[];  // [GC][nsplit]: 2^(m_s - M) / L
  __shared__ f32x4 part[SG][GC * DG];
  const int g = a.nh / a.nkv;
  const int per_kv = g / GC;
  const int j = blockIdx.y / per_kv;
  const int h0 = j * g + (blockIdx.y - j * per_kv) * GC;
  const int n = blockIdx.z;
  int b;
  const int pos = query_position(a, n, &b);
  const int nvalid = (pos + a.chunk) / a.chunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t base0 = ((size_t)n * a.nh + h0) * a.nsplit;
  for (int h = wave; h < GC; h += 4) {
    const float* pm = a.part_m + base0 + (size_t)h * a.nsplit;
    const float* pl = a.part_l + base0 + (size_t)h * a.nsplit;
    float mx = -INFINITY;
    for (int sp = lane; sp < nvalid; sp += 64) mx = fmaxf(mx, pm[sp]);
    mx = wave_max(mx);
    float L = 0.f;
    for (int sp = lane; sp < nvalid; sp += 64) {
      const float w = exp2f(pm[sp] - mx);
      w_s[h * a.nsplit + sp] = w;
      L += w * pl[sp];
    }
    L = wave_sum(L);
    const float inv = 1.0f / L;
    for (int sp = lane; sp < nvalid; sp += 64) w_s[h * a.nsplit + sp] *= inv;
  }
  __syncthreads();
  const int dg = tid % DG, sg = tid / DG;
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    const float* pa = a.part_acc + (base0 + (size_t)h * a.nsplit) * HD + dg * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int sp = sg; sp < nvalid; sp += SG)
      acc += w_s[h * a.nsplit + sp] * *reinterpret_cast<const f32x4*>(pa + (size_t)sp * HD);
    part[sg][h * DG + dg] = acc;
  }
  __syncthreads();
  for (int idx = tid; idx < GC * DG; idx += 256) {
    f32x4 v = part[0][idx];
#pragma unroll
    for (int k = 1; k < SG; ++k) v += part[k][idx];
    const int h = idx / DG, d = (idx - h * DG) * 4;
    const size_t oi = (size_t)n * a.nh * HD + (size_t)(h0 + h) * HD + d;
    if (a.act_dt == DT_F32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + oi) = v;
    } else if (a.act_dt == DT_BF16) {
      store4<DT_BF16>(reinterpret_cast<uint16_t*>(a.o) + oi, v[0], v[1], v[2], v[3]);
    } else {
      store4<DT_F16>(reinterpret_cast<uint16_t*>(a.o) + oi, v[0], v[1], v[2], v[3]);
    }
  }
}

// Keys per thread for a chunk size (chunk = KPT * 256 / (HD / 8)).
template <int KVDT, int HD, int GC>
static hipError_t split_launch_kpt(const AttnDecodeArgs& a, dim3 grid, hipStream_t s) {
  constexpr int KPI = 256 / (HD / 8);
  switch (a.chunk / KPI) {
    case 2: LL_LAUNCH((attn_split_kernel<KVDT, HD, GC, 2>), grid, dim3(256), 0, s, a); break;
    case 4: LL_LAUNCH((attn_split_kernel<KVDT, HD, GC, 4>), grid, dim3(256), 0, s, a); break;
    case 8: LL_LAUNCH((attn_split_kernel<KVDT, HD, GC, 8>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KVDT, int HD, int GC>
static hipError_t gqa_launch_tw(const AttnDecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (a.chunk / 64) {
    case 1: LL_LAUNCH((attn_gqa_kernel<KVDT, HD, GC, 1>), grid, dim3(256), 0, s, a); break;
    case 2: LL_LAUNCH((attn_gqa_kernel<KVDT, HD, GC, 2>), grid, dim3(256), 0, s, a); break;
    case 4: LL_LAUNCH((attn_gqa_kernel<KVDT, HD, GC, 4>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KVDT, int HD>
static hipError_t split_launch(const AttnDecodeArgs& a, hipStream_t s) {
  const int g = a.nh / a.nkv;
  const int gc = attn_heads_per_group(g);
  dim3 grid(a.nsplit, a.nkv * (g / gc), a.nq);
  if constexpr (KVDT != DT_F32) {
    if (attn_uses_gqa_kernel(a.kv_dt, g)) {
      if (gc == 8) return gqa_launch_tw<KVDT, HD, 8>(a, grid, s);
      return gqa_launch_tw<KVDT, HD, 4>(a, grid, s);
    }
  }
  switch (gc) {
    case 8: return split_launch_kpt<KVDT, HD, 8>(a, grid, s);
    case 4: return split_launch_kpt<KVDT, HD, 4>(a, grid, s);
    case 2: return split_launch_kpt<KVDT, HD, 2>(a, grid, s);
    default: return split_launch_kpt<KVDT, HD, 1>(a, grid, s);
  }
}

int attn_heads_per_group(int g) { return (g % 8 == 0) ? 8 : (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1; }

bool attn_uses_gqa_kernel(int kv_dt, int g) {
  return kv_dt != DT_F32 && attn_heads_per_group(g) >= 4;
}

int attn_pick_chunk(int hd, int max_keys, int queries, int nkv, int g, int kv_dt) {
  const int gc = attn_heads_per_group(g);
  const int groups = nkv * (g / gc);
  if (attn_uses_gqa_kernel(kv_dt, g)) {
    // Chunk 64, 128 or 256 keys: the largest that still gives >= 2048 workgroups.
    int tw = 4;
    while (tw > 1 && (int64_t)((max_keys + 64 * tw - 1) / (64 * tw)) * queries * groups < 2048)
      tw >>= 1;
    while ((max_keys + 64 * tw - 1) / (64 * tw) > ATTN_MAX_SPLITS) {
      if (tw >= 4) return -1;
      tw *= 2;
    }
    return 64 * tw;
  }
  // Keys per thread 2..8 (at most 4 with 8 heads per group), chunk = kpt * 256 / (hd / 8):
  // the largest chunk that still gives >= 2048 workgroups, and never more than
  // ATTN_MAX_SPLITS splits (the merge keeps one weight per split in LDS).
  const int kpi = 256 / (hd / 8);
  const int kpt_max = gc >= 8 ? 4 : 8;
  int pick = 2;
  for (int kpt = kpt_max; kpt >= 2; kpt >>= 1) {
    const int64_t wgs = (int64_t)((max_keys + kpt * kpi - 1) / (kpt * kpi)) * queries * groups;
    pick = kpt;
    if (wgs >= 2048) break;
  }
  while ((max_keys + pick * kpi - 1) / (pick * kpi) > ATTN_MAX_SPLITS) {
    if (pick >= kpt_max) return -1;
    pick *= 2;
  }
  return pick * kpi;
}

template <int HD>
static hipError_t merge_launch(const AttnDecodeArgs& a, hipStream_t s) {
  const int g = a.nh / a.nkv;
  const int gc = attn_heads_per_group(g);
  dim3 grid(1, a.nkv * (g / gc), a.nq);
  const size_t sh = (size_t)gc * a.nsplit * sizeof(float);
  switch (gc) {
    case 8: LL_LAUNCH((attn_merge_kernel<HD, 8>), grid, dim3(256), sh, s, a); break;
    case 4: LL_LAUNCH((attn_merge_kernel<HD, 4>), grid, dim3(256), sh, s, a); break;
    case 2: LL_LAUNCH((attn_merge_kernel<HD, 2>), grid, dim3(256), sh, s, a); break;
    default: LL_LAUNCH((attn_merge_kernel<HD, 1>), grid, dim3(256), sh, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.hd == 128) {
    e = (a.kv_dt == DT_F32) ? split_launch<DT_F32, 128>(a, s)
      : (a.kv_dt == DT_BF16) ? split_launch<DT_BF16, 128>(a, s) : split_launch<DT_F16, 128>(a, s);
  } else {
    e = (a.kv_dt == DT_F32) ? split_launch<DT_F32, 64>(a, s)
      : (a.kv_dt == DT_BF16) ? split_launch<DT_BF16, 64>(a, s) : split_launch<DT_F16, 64>(a, s);
  }
  if (e != hipSuccess) return e;
  return a.hd == 128 ? merge_launch<128>(a, s) : merge_launch<64>(a, s);
}

}  // namespace ll
