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
  const T* kp = reinterpret_cast<const T*>(a.kc) + sub * 8;
  const T* vp = reinterpret_cast<const T*>(a.vc) + sub * 8;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // Row of each key; keys past the chunk are not loaded.  Paged caches: when
  // a pass of KPI keys sits in one block, its block index is wave-uniform.
  size_t rows[KPT];
  const bool uniform_pass = a.pages.table && KPI <= (1 << a.pages.log2_bs);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = k_lo + slot + i * KPI;
    const int kk = key < k_hi ? key : k_lo;
    if (uniform_pass) {
      const int blk = kv_block_uniform(a.pages, b, min(k_lo + i * KPI, k_hi - 1));
      rows[i] = ((((size_t)blk * a.nkv + j) << a.pages.log2_bs) +
                 (kk & ((1 << a.pages.log2_bs) - 1))) * HD;
    } else {
      rows[i] = kv_row(a.pages, b, j, kk, a.nkv, a.s_max, HD);
    }
  }
  u32x4 kr[KPT][NC], vr[KPT][NC];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = k_lo + slot + i * KPI;
    const bool ok = key < k_hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[i][c] = ok ? ld16_stream(kp + rows[i] + c * (8 / NC)) : zero;
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = k_lo + slot + i * KPI;
    const bool ok = key < k_hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) vr[i][c] = ok ? ld16_stream(vp + rows[i] + c * (8 / NC)) : zero;
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

// GQA variant for 16-bit caches with GC = 4 or 8 query heads per workgroup;
// both products run on the matrix cores.
//
// Scores of a 16-key tile: v_mfma_f32_16x16x32 with K in the A layout (lane:
// key r16, dims 32s + 8(l/16) of slice s) and the group's queries in the B
// layout (head r16; columns past GC are zero).  The result leaves lane l with
// head l%16 and keys 4(l/16) + 0..3, which is exactly the A layout of a
// 16x16x16 MFMA with P as A (heads x keys), so P V needs no data movement
// for P.  V (keys x dims) is the B operand, read with ds_read_b64_tr_b16,
// which hands lane l the 4 keys of k-group l/16 for dim l%16.
//
// Each wave streams its own keys, 16 per iteration (keys k_lo + 64 it +
// 16 wave + [0, 16)), with an online softmax, so the waves never wait for each
// other until the end, where their (max, sum, acc) are combined in LDS.  The
// K and V rows of an iteration go to the wave's own LDS ring by
// global_load_lds, two iterations ahead, with explicit wait counts: every
// vector-memory load in the loop is such a DMA.  (Register loads in flight
// next to LDS loads make the compiler wait for all of them before any use.)
// The 16-byte chunks of a K row are XOR-swizzled by row & 15 (fragment reads
// of 16 rows hit 16 bank groups) and those of a V row by 2 (row & 3) (the 16
// lanes of a transposed read hit 16 bank pairs); the swizzle is applied on
// the global side, since the DMA writes each instruction's 1 KB linearly.
// Queries and P are rounded to the cache format for the MFMAs.  Output: the
// same partials as attn_split_kernel, one split per a.chunk keys; with a
// single split (a whole context per workgroup) the normalised output itself,
// and no merge follows.  NW waves per workgroup: 4 for split contexts, 8 for
// whole ones.
template <int KVDT, int HD, int GC, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_gqa_kernel(AttnDecodeArgs a) {
  typedef typename Elt<KVDT>::T T;
  constexpr int NS = HD / 32;         // 32-dim slices: score MFMAs per tile
  constexpr int ND = HD / 16;         // 16-dim output tiles: P V MFMAs per tile
  constexpr int KW = 16;              // keys per wave and iteration
  constexpr int WI = NW * KW;         // keys per workgroup and iteration
  constexpr int ROW = HD * 2;         // bytes of one K or V row
  constexpr int TILE = KW * ROW;      // one wave's K (or V) rows of one iteration
  constexpr int TI = TILE / 1024;     // DMA instructions per tile
  constexpr int RPI = 1024 / ROW;     // rows per DMA instruction
  constexpr int CPR = ROW / 16;       // 16-byte chunks per row
  constexpr int WAVE_LDS = 4 * TILE;  // K and V rings of one wave
  constexpr int RING = NW * WAVE_LDS;
  static_assert(NW * GC * HD * 4 <= RING, "the wave sums reuse the rings");
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
  if (k_lo >= k_hi) return;  // past this query's context: not counted, not merged
  const int nit = (k_hi - k_lo + WI - 1) / WI;

  // One LDS object (a second one would make the compiler wait for every
  // outstanding load before each LDS read): per-wave K and V rings, then
  // per-wave rescale factors, maxima and sums.  The cross-wave sums reuse the
  // rings.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[RING + 3 * NW * 16 * 4];
  float* s_alpha = reinterpret_cast<float*>(lds + RING);  // [NW][16]
  float* s_m = s_alpha + NW * 16;                         // [NW][16]
  float* s_l = s_m + NW * 16;                             // [NW][16]
  float* s_acc = reinterpret_cast<float*>(lds);           // [NW][GC][HD] after the loop

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  uint8_t* kring = lds + wave * WAVE_LDS;  // [2][TILE]
  uint8_t* vring = kring + 2 * TILE;       // [2][TILE]
  const T* kp = reinterpret_cast<const T*>(a.kc);
  const T* vp = reinterpret_cast<const T*>(a.vc);
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // The queries, before any DMA is in flight.  Lanes past GC read head h0 and
  // use zeros.
  const float qscale = 1.44269504088896341f / sqrtf((float)HD);
  u32x4 qb[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float* qp = a.q + ((size_t)n * a.nh + h0 + (r16 < GC ? r16 : 0)) * HD + 32 * s + 8 * g4;
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(qp);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(qp + 4);
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = q0[e] * qscale;
      f[e + 4] = q1[e] * qscale;
    }
    qb[s] = r16 < GC ? pack16<KVDT>(f) : zero;
  }

  // Rows past the chunk's end read the last valid row (finite values whose
  // scores are masked and whose P is zero).  Iteration it uses buffer it & 1
  // and refills it with iteration it + 2 once consumed; every iteration
  // issues the same 2 TI loads (past the end they repeat the last row), so
  // the wait counts below are exact.  DMA instruction i fills rows
  // RPI i + l / CPR; lane l fetches the row's logical chunk (l % CPR) ^ swz.
  // Paged caches: a wave's 16 keys (16-aligned) sit in one block of at least
  // 16 positions, and rows clamped to the last key stay in it, so the block
  // index is wave-uniform and comes from a scalar load.
  auto load_tile = [&](const T* src, uint8_t* dst, int it, bool is_k) {
    const int kb = k_lo + WI * it + KW * wave;
    size_t base;  // element offset of row 0 of the key's block, or of the head
    int kmask;
    if (a.pages.table) {
      const int blk = kv_block_uniform(a.pages, b, min(kb, k_hi - 1));
      base = (((size_t)blk * a.nkv + j) << a.pages.log2_bs) * HD;
      kmask = (1 << a.pages.log2_bs) - 1;
    } else {
      base = ((size_t)b * a.nkv + j) * a.s_max * HD;
      kmask = -1;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r = i * RPI + lane / CPR;
      const int key = min(kb + r, k_hi - 1);
      const int c = (lane % CPR) ^ (is_k ? (r & (CPR - 1)) : 2 * (r & 3));
      dma16_stream(src + (base + (size_t)(key & kmask) * HD + c * 8), dst + i * 1024);
    }
  };
  // K fragment of slice s: row r16, logical chunk 4s + g4.
  auto k_operand = [&](int buf, int s) {
    return ld16(kring + buf * TILE + r16 * ROW + (((4 * s + g4) ^ (r16 & (CPR - 1))) << 4));
  };
  // Transposed V read for output tile t: lane (g4, 4e + q) points at row
  // 4 g4 + e, dims 16 t + 4q .. +3 (ds_read_tr16: the caller waits for the
  // results itself).
  const int e4 = r16 >> 2, q4 = r16 & 3;
  const uint32_t vaddr = lds_addr(vring) + (4 * g4 + e4) * ROW + 8 * (q4 & 1);
  auto v_operand = [&](int buf, int t) {
    return ds_read_tr16(vaddr + buf * TILE + (((2 * t + (q4 >> 1)) ^ (2 * e4)) << 4));
  };
  load_tile(kp, kring, 0, true);
  load_tile(vp, vring, 0, false);
  load_tile(kp, kring + TILE, 1, true);
  load_tile(vp, vring + TILE, 1, false);

  float m_run = -INFINITY;  // running max of head r16 over this wave's keys
  float l_run = 0.f;        // this lane's share of the running sum
  f32x4 o[ND];              // lane: dim 16t + r16 of heads 4 g4 + 0..3
#pragma unroll
  for (int t = 0; t < ND; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One iteration; past nit every key is masked and it changes nothing.
  auto iteration = [&](int it, int buf) {
    const int kb = k_lo + WI * it + KW * wave;
    // K(it) has landed once only V(it), K(it+1) and V(it+1) may be outstanding.
    wait_vmcnt<3 * TI>();
    __builtin_amdgcn_sched_barrier(0);
    // Scores: lane holds head r16, keys kb + 4 g4 + i.
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) c = mfma16_chunk<KVDT>(k_operand(buf, s), qb[s], c);
    // The fragment reads are done before the K buffer is refilled.
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    load_tile(kp, kring + buf * TILE, it + 2, true);
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kb + 4 * g4 + i >= k_hi) c[i] = -INFINITY;
      mt = fmaxf(mt, c[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    // No valid key yet for this wave: keep everything at zero.
    const bool none = (m_new == -INFINITY);
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float pf[4];
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pf[i] = none ? 0.f : __builtin_amdgcn_exp2f(c[i] - m_new);
      ls += pf[i];
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
    // Rescale factors of heads 4 g4 + 0..3 (held by lanes r16 = head); this
    // wave's LDS accesses complete in order.
    if (g4 == 0) s_alpha[wave * 16 + r16] = alpha;
    const f32x4 al = *reinterpret_cast<const f32x4*>(&s_alpha[wave * 16 + 4 * g4]);
#pragma unroll
    for (int t = 0; t < ND; ++t) o[t] *= al;
    u32x2 pa;
    pa[0] = pack2<KVDT>(pf[0], pf[1]);
    pa[1] = pack2<KVDT>(pf[2], pf[3]);
    // V(it) has landed once only K(it+1), V(it+1) and K(it+2) may be outstanding.
    wait_vmcnt<3 * TI>();
    __builtin_amdgcn_sched_barrier(0);
    u32x2 vb[ND];
#pragma unroll
    for (int t = 0; t < ND; ++t) vb[t] = v_operand(buf, t);
    wait_lgkmcnt0();  // the transposed reads have landed (and the buffer may be refilled)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < ND; ++t) o[t] = mfma16k16<KVDT>(pa, vb[t], o[t]);
    load_tile(vp, vring + buf * TILE, it + 2, false);
  };
  for (int it = 0; it < nit; it += 2) {
    iteration(it, 0);
    iteration(it + 1, 1);
  }

  // This wave's totals (l over the four lanes of each head); the rings are
  // reused once every wave's loads have landed.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g4 + i;
    if (h < GC) {
#pragma unroll
      for (int t = 0; t < ND; ++t) s_acc[(wave * GC + h) * HD + 16 * t + r16] = o[t][i];
    }
  }
  if (g4 == 0) {
    s_m[wave * 16 + r16] = m_run;
    s_l[wave * 16 + r16] = l_run;
  }
  __syncthreads();
  // Combine the waves (wave 0 always holds a valid key, so M is finite).
  auto wave_max_m = [&](int h) {
    float M = s_m[h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w * 16 + h]);
    return M;
  };
  for (int idx = tid; idx < GC * HD; idx += NW * 64) {
    const int h = idx / HD, d = idx - h * HD;
    const float M = wave_max_m(h);
    float v = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (s_m[w * 16 + h] != -INFINITY) {
        const float sc = exp2f(s_m[w * 16 + h] - M);
        v += sc * s_acc[(w * GC + h) * HD + d];
        l += sc * s_l[w * 16 + h];
      }
    if (a.nsplit == 1) {
      // The whole context: the normalised output (no merge follows).
      const size_t oi = (size_t)n * a.nh * HD + (size_t)(h0 + h) * HD + d;
      const float o = v / l;
      if (a.act_dt == DT_F32) reinterpret_cast<float*>(a.o)[oi] = o;
      else if (a.act_dt == DT_BF16) reinterpret_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(o);
      else reinterpret_cast<uint16_t*>(a.o)[oi] = f32_to_f16(o);
    } else {
      a.part_acc[(((size_t)n * a.nh + h0 + h) * a.nsplit + split) * HD + d] = v;
      if (d == 0) {
        const size_t pi = ((size_t)n * a.nh + h0 + h) * a.nsplit + split;
        a.part_m[pi] = M;
        a.part_l[pi] = l;
      }
    }
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
  const int dg = tid % DG, sg = tid / DG;
  // This thread's first split of every head is loaded before the weights are
  // computed, so with at most SG splits the partials take one round trip.
  f32x4 first[GC];
#pragma unroll
  for (int h = 0; h < GC; ++h)
    first[h] = sg < nvalid ? *reinterpret_cast<const f32x4*>(
                                 a.part_acc + ((base0 + (size_t)h * a.nsplit + sg) * HD + dg * 4))
                           : f32x4{0.f, 0.f, 0.f, 0.f};
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
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    const float* pa = a.part_acc + (base0 + (size_t)h * a.nsplit) * HD + dg * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (sg < nvalid) acc = w_s[h * a.nsplit + sg] * first[h];
#pragma unroll 4
    for (int sp = sg + SG; sp < nvalid; sp += SG)
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
  if (a.nsplit == 1)
    LL_LAUNCH((attn_gqa_kernel<KVDT, HD, GC, 8>), grid, dim3(512), 0, s, a);
  else
    LL_LAUNCH((attn_gqa_kernel<KVDT, HD, GC, 4>), grid, dim3(256), 0, s, a);
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
    // With a workgroup per CU or more at one split per query and group, whole
    // contexts (8-wave workgroups, no merge launch); the longest context then
    // sets the time as it does with 2048-key chunks.
    if ((int64_t)queries * groups >= 256) return (max_keys + 127) / 128 * 128;
    // Otherwise chunks of 256, 512, 1024 or 2048 keys: the largest that still gives >= 512
    // workgroups (counted at the longest context).  Longer chunks mean fewer
    // partials to merge and fewer per-workgroup tails; measured on the 70B
    // batch-32 decode, 2048 beats both 1024 and 4096.
    int nit = 8;
    while (nit > 1 && (int64_t)((max_keys + 256 * nit - 1) / (256 * nit)) * queries * groups < 512)
      nit >>= 1;
    while ((max_keys + 256 * nit - 1) / (256 * nit) > ATTN_MAX_SPLITS) {
      if (nit >= 8) return -1;
      nit *= 2;
    }
    return 256 * nit;
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
  // A single split of the GQA kernel wrote the output itself.
  if (a.nsplit == 1 && attn_uses_gqa_kernel(a.kv_dt, a.nh / a.nkv)) return hipSuccess;
  return a.hd == 128 ? merge_launch<128>(a, s) : merge_launch<64>(a, s);
}

}  // namespace ll
