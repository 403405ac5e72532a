// Prefill projections: y[m, n] = sum_k u[m, k] W[n, k] for many tokens m.
//
// The tile is computed transposed, D[feature, token] = W u^T, so that the four
// consecutive output features a lane holds (v_mfma_f32_32x32x16 result layout)
// give lane-local RoPE pairs, lane-local SwiGLU (gate and up land in the same
// lane) and 8-byte stores.
//
// Workgroup tile BM weight rows x BN tokens x 64 k, four waves.  Both operands
// are staged through LDS, double buffered.  A 64-k row slice is 128 bytes, so
// two rows share one 256-byte sweep of the 64 LDS banks; the 16-byte chunk c of
// row r is stored at chunk c ^ ((r >> 1) & 7), which gives the 16 rows a
// ds_read_b128 serves per cycle 16 distinct bank groups.  The
// large tile (256 x 256, a 128 x 128 wave tile, 256 accumulators per lane in
// AGPRs) halves LDS and L2 traffic per flop against 128 x 128; the small tile
// keeps enough workgroups for the narrower projections.  Tiles are numbered so
// that each XCD (workgroup i runs on XCD i mod 8) gets a contiguous run and,
// within it, groups of GROUP_M weight panels share token panels in L2.
#include "common.cuh"
#include "epilogue.cuh"

namespace ll {

constexpr int GBK = 64;   // k per stage
constexpr int GROUP_M = 4;
#ifndef GEMM_BIG_WAVES
#define GEMM_BIG_WAVES 8
#endif

// QKV epilogue of the prefill GEMMs for four consecutive features f..f+3 of
// token (b, t) at position pos: RoPE on q/k pairs, q to [B, nh, T, hd], k/v
// into the caches, all in the cache format KVDT (a template parameter, so the
// whole tile epilogue stays small enough to unroll with the accumulators in
// registers).
template <int KVDT>
__device__ __forceinline__ void gemm_qkv_store(const ProjArgs& a, int b, int t, int pos, int f,
                                               float* v) {
  typedef typename Elt<KVDT>::T KT;
  const int hd = a.hd;
  const int qd = a.nh * hd, kd = a.nkv * hd;
  if (f < qd + kd) {
    const int d = (f < qd ? f : f - qd) % hd;
    const size_t ti = (size_t)pos * (hd >> 1) + (d >> 1);
    const float c0 = a.rcos[ti], s0 = a.rsin[ti], c1 = a.rcos[ti + 1], s1 = a.rsin[ti + 1];
    const float x0 = v[0], y0 = v[1], x1 = v[2], y1 = v[3];
    v[0] = x0 * c0 - y0 * s0;
    v[1] = x0 * s0 + y0 * c0;
    v[2] = x1 * c1 - y1 * s1;
    v[3] = x1 * s1 + y1 * c1;
  }
  KT* dst;
  if (f < qd) {
    const int h = f / hd;
    dst = reinterpret_cast<KT*>(a.q16) + (((size_t)b * a.nh + h) * a.T + t) * hd + (f - h * hd);
  } else {
    const int g = f < qd + kd ? f - qd : f - qd - kd;
    const int j = g / hd;
    KT* cache = reinterpret_cast<KT*>(f < qd + kd ? a.kc : a.vc);
    dst = cache + (((size_t)b * a.nkv + j) * a.s_max + pos) * hd + (g - j * hd);
  }
  store4<KVDT>(dst, v[0], v[1], v[2], v[3]);
}

template <int DT, int EPI, int BM, int BN, int KVDT>
__global__ __launch_bounds__(256) void gemm_kernel(ProjArgs a) {
  typedef typename Elt<DT>::T T;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int FM = SWI ? BM / 2 : BM;               // output features per tile
  // Wave layout: 2 x 2 over (rows, tokens); SwiGLU: 1 x 4 so a wave holds both
  // the gate and the up rows of its features.
  constexpr int RB = SWI ? BM / 32 : BM / 64;         // 32-row blocks per wave
  constexpr int CB = SWI ? BN / 128 : BN / 64;        // 32-token blocks per wave
  constexpr int AR = BM * 8 / 256;                    // A chunks per thread per stage
  constexpr int BR = BN * 8 / 256;                    // B chunks per thread per stage

  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][BM * GBK];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][BN * GBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const int ntm = (a.N + FM - 1) / FM;
  const int ntn = (a.M + BN - 1) / BN;

  // Tile order: contiguous per XCD, then grouped.
  const int nb = gridDim.x;
  int b2 = blockIdx.x;
  if ((nb & 7) == 0) b2 = (b2 & 7) * (nb >> 3) + (b2 >> 3);
  const int per_group = GROUP_M * ntn;
  const int grp = b2 / per_group;
  const int first_m = grp * GROUP_M;
  const int gm = min(ntm - first_m, GROUP_M);
  const int in_grp = b2 - grp * per_group;
  const int tile_m = first_m + in_grp % gm;
  const int tile_n = in_grp / gm;
  const int f0 = tile_m * FM;
  const int n0 = tile_n * BN;

  // Global -> LDS assignment: 8 chunks of 16 bytes per 64-k row slice.
  const int lc = tid & 7;   // chunk
  const int lr = tid >> 3;  // first row; rows lr + 32 i
  const T* arow[AR];
  const T* brow[BR];
  bool av[AR], bv[BR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    const int r = lr + 32 * i;
    if constexpr (SWI) {
      const int f = f0 + (r % FM);
      av[i] = f < a.N;
      const T* base = reinterpret_cast<const T*>(r < FM ? a.w[0] : a.w[1]);
      arow[i] = base + (size_t)(av[i] ? f : 0) * K;
    } else {
      const int f = f0 + r;
      av[i] = f < a.N;
      arow[i] = seg_row<T>(a, av[i] ? f : 0);
    }
  }
#pragma unroll
  for (int i = 0; i < BR; ++i) {
    const int m = n0 + lr + 32 * i;
    bv[i] = m < a.M;
    brow[i] = reinterpret_cast<const T*>(a.x) + (size_t)(bv[i] ? m : 0) * K;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 ra[AR], rb[BR];
  auto gload = [&](int kt) {
    const int k = kt * GBK + lc * 8;
    const bool kin = k < K;
#pragma unroll
    for (int i = 0; i < AR; ++i) ra[i] = (kin && av[i]) ? ld16(arow[i] + k) : zero;
#pragma unroll
    for (int i = 0; i < BR; ++i) rb[i] = (kin && bv[i]) ? ld16(brow[i] + k) : zero;
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AR; ++i) {
      const int r = lr + 32 * i;
      st16(&lds_a[buf][r * GBK + ((lc ^ ((r >> 1) & 7)) << 3)], ra[i]);
    }
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      const int r = lr + 32 * i;
      st16(&lds_b[buf][r * GBK + ((lc ^ ((r >> 1) & 7)) << 3)], rb[i]);
    }
  };

  // Wave placement inside the tile.
  int row_base[RB], col_base[CB];
  if constexpr (SWI) {
#pragma unroll
    for (int r = 0; r < RB; ++r) row_base[r] = r * 32;
#pragma unroll
    for (int c = 0; c < CB; ++c) col_base[c] = wave * (BN / 4) + c * 32;
  } else {
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int r = 0; r < RB; ++r) row_base[r] = wm * (BM / 2) + r * 32;
#pragma unroll
    for (int c = 0; c < CB; ++c) col_base[c] = wn * (BN / 2) + c * 32;
  }
  const int l32 = lane & 31, h2 = lane >> 5;

  f32x16 acc[RB][CB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.f;

  // MFMA fragments of one 16-k step, double buffered so the LDS reads of step
  // s+1 are in flight while step s multiplies.
  u32x4 fa[2][RB], fb[2][CB];
  auto lread = [&](int buf, int s, int slot) {
    const int ch = s * 2 + h2;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = row_base[r] + l32;
      fa[slot][r] = ld16(&lds_a[buf][row * GBK + ((ch ^ ((row >> 1) & 7)) << 3)]);
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int col = col_base[c] + l32;
      fb[slot][c] = ld16(&lds_b[buf][col * GBK + ((ch ^ ((col >> 1) & 7)) << 3)]);
    }
  };

  const int nkt = (K + GBK - 1) / GBK;
  gload(0);
  lstore(0);
  __syncthreads();
  lread(0, 0, 0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < GBK / 16; ++s) {
      if (s + 1 < GBK / 16) lread(cur, s + 1, (s + 1) & 1);
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c) acc[r][c] = mfma32<DT>(fa[s & 1][r], fb[s & 1][c], acc[r][c]);
    }
    if (kt + 1 < nkt) {
      lstore(cur ^ 1);
      __syncthreads();
      lread(cur ^ 1, 0, 0);
    }
  }

  // Epilogue.  acc[r][c][i]: feature row_base[r] + (i/4)*8 + h2*4 + i%4,
  // token col_base[c] + l32.
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int m = n0 + col_base[c] + l32;
    if (m >= a.M) continue;
    const int mb = m / a.T, mt = m - mb * a.T, mpos = a.start_pos + mt;  // QKV only
#pragma unroll
    for (int r = 0; r < (SWI ? RB / 2 : RB); ++r) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int f = f0 + row_base[r] + g4 * 8 + h2 * 4;
        if (f >= a.N) continue;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = acc[r][c][g4 * 4 + i];
        if constexpr (EPI == EPI_RESID) {
          const T* rp = reinterpret_cast<const T*>(a.resid) + (size_t)m * a.N + f;
          float rv[4];
          load4<DT>(rp, rv);
          T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
          store4<DT>(y, rv[0] + v[0], rv[1] + v[1], rv[2] + v[2], rv[3] + v[3]);
        } else if constexpr (SWI) {
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = silu(v[i]) * acc[r + RB / 2][c][g4 * 4 + i];
          T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
          store4<DT>(y, o[0], o[1], o[2], o[3]);
        } else {
          gemm_qkv_store<KVDT>(a, mb, mt, mpos, f, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant (K % 32 == 0).  Operands move global -> LDS with
// global_load_lds_dwordx4 (lane l of a wave writes bytes [16 l, 16 l + 16) of
// the LDS destination), so no registers stage them and no ds_write is issued;
// the swizzled LDS layout comes from permuting each lane's global address.
// 32-k stages, NST of them in LDS, loads NST-1 stages ahead of the multiply.
// A 32-k row slice is 64 bytes, four rows per 256-byte bank sweep: chunk c of
// row r is stored at chunk c ^ ((r >> 2) & 3).
// ---------------------------------------------------------------------------
// Occupancy target per SIMD: 4 waves on a 256 x 256 tile hold 256 accumulator
// registers each (one wave per SIMD); 8 waves hold 128 (two per SIMD, so one
// wave's barrier and LDS waits overlap the other's MFMAs).  Telling the
// compiler lets it keep fragments in flight instead of chasing occupancy.
template <int BM, int NW>
struct DmaOcc { static constexpr int waves = (BM == 256 && NW == 4) ? 1 : 2; };

template <int DT, int EPI, int BM, int BN, int KVDT, int NW>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(DmaOcc<BM, NW>::waves, DmaOcc<BM, NW>::waves)))
void gemm_dma_kernel(ProjArgs a) {
  typedef typename Elt<DT>::T T;
  constexpr int BK = 32;
  constexpr int NST = 4;
  constexpr int ROWB = BK * 2;                 // 64 bytes per row slice
  constexpr int RPI = 16;                      // rows per 1 KB wave instruction
  constexpr int AI = BM / RPI / NW;            // A instructions per wave per stage
  constexpr int BI = BN / RPI / NW;
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int FM = SWI ? BM / 2 : BM;
  // Wave grid over (rows, tokens): 2 x NW/2; SwiGLU 1 x NW (gate and up rows
  // of a feature in the same wave).
  constexpr int WN = SWI ? NW : NW / 2;        // waves along tokens
  constexpr int RB = SWI ? BM / 32 : BM / 64;
  constexpr int CB = BN / WN / 32;

  __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const int ntm = (a.N + FM - 1) / FM;
  const int ntn = (a.M + BN - 1) / BN;
  const int nb = gridDim.x;
  int b2 = blockIdx.x;
  if ((nb & 7) == 0) b2 = (b2 & 7) * (nb >> 3) + (b2 >> 3);
  const int per_group = GROUP_M * ntn;
  const int grp = b2 / per_group;
  const int first_m = grp * GROUP_M;
  const int gm = min(ntm - first_m, GROUP_M);
  const int in_grp = b2 - grp * per_group;
  const int tile_m = first_m + in_grp % gm;
  const int tile_n = in_grp / gm;
  const int f0 = tile_m * FM;
  const int n0 = tile_n * BN;

  // DMA sources: lane l fills row (l / 4) of its 16-row slab, physical chunk
  // l % 4, i.e. logical chunk (l % 4) ^ ((row >> 2) & 3).  Rows past N or M
  // read row 0 (their results are never stored).
  const int rr = lane >> 2, pc = lane & 3;
  const T* asrc[AI];
  const T* bsrc[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (wave * AI + i) * RPI + rr;
    const int c = pc ^ ((r >> 2) & 3);
    const T* row;
    if constexpr (SWI) {
      const int f = f0 + (r % FM);
      row = reinterpret_cast<const T*>(r < FM ? a.w[0] : a.w[1]) + (size_t)(f < a.N ? f : 0) * K;
    } else {
      const int f = f0 + r;
      row = seg_row<T>(a, f < a.N ? f : 0);
    }
    asrc[i] = row + c * 8;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int r = (wave * BI + i) * RPI + rr;
    const int c = pc ^ ((r >> 2) & 3);
    const int m = n0 + r;
    bsrc[i] = reinterpret_cast<const T*>(a.x) + (size_t)(m < a.M ? m : 0) * K + c * 8;
  }
  auto issue = [&](int st, int kt) {
    uint8_t* base = lds + st * STAGE;
    const int k = kt * BK;
#pragma unroll
    for (int i = 0; i < AI; ++i) dma16(asrc[i] + k, base + (wave * AI + i) * 1024);
#pragma unroll
    for (int i = 0; i < BI; ++i) dma16(bsrc[i] + k, base + BM * ROWB + (wave * BI + i) * 1024);
  };

  int row_base[RB], col_base[CB];
  if constexpr (SWI) {
#pragma unroll
    for (int r = 0; r < RB; ++r) row_base[r] = r * 32;
#pragma unroll
    for (int c = 0; c < CB; ++c) col_base[c] = wave * (BN / WN) + c * 32;
  } else {
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int r = 0; r < RB; ++r) row_base[r] = wm * (BM / 2) + r * 32;
#pragma unroll
    for (int c = 0; c < CB; ++c) col_base[c] = wn * (BN / WN) + c * 32;
  }
  const int l32 = lane & 31, h2 = lane >> 5;
  int aoff[RB], boff[CB];  // byte offsets of this lane's fragment rows (chunk added per step)
#pragma unroll
  for (int r = 0; r < RB; ++r) aoff[r] = (row_base[r] + l32) * ROWB;
#pragma unroll
  for (int c = 0; c < CB; ++c) boff[c] = BM * ROWB + (col_base[c] + l32) * ROWB;
  const int swz_a = ((l32 >> 2) & 3);  // row_base is a multiple of 32: (row >> 2) & 3 == (l32 >> 2) & 3

  f32x16 acc[RB][CB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.f;

  // Fragments of the two 16-k steps of a stage: X = step 0, Y = step 1.
  u32x4 xa[RB], xb[CB], ya[RB], yb[CB];
  auto read_x = [&](int st) {
    const uint8_t* base = lds + st * STAGE;
    const int chb = ((0 + h2) ^ swz_a) * 16;
#pragma unroll
    for (int r = 0; r < RB; ++r) xa[r] = ld16(base + aoff[r] + chb);
#pragma unroll
    for (int c = 0; c < CB; ++c) xb[c] = ld16(base + boff[c] + chb);
  };
  auto read_y = [&](int st) {
    const uint8_t* base = lds + st * STAGE;
    const int chb = ((2 + h2) ^ swz_a) * 16;
#pragma unroll
    for (int r = 0; r < RB; ++r) ya[r] = ld16(base + aoff[r] + chb);
#pragma unroll
    for (int c = 0; c < CB; ++c) yb[c] = ld16(base + boff[c] + chb);
  };
  // Wait until this wave's DMA of a stage has landed: at most the loads of the
  // `newer` stages issued after it may still be outstanding.
  auto wait_stage = [&](int newer) {
    if (newer >= 3) wait_vmcnt<3 * (AI + BI)>();
    else if (newer == 2) wait_vmcnt<2 * (AI + BI)>();
    else if (newer == 1) wait_vmcnt<1 * (AI + BI)>();
    else wait_vmcnt<0>();
  };

  const int nkt = K / BK;
#pragma unroll
  for (int st = 0; st < NST; ++st)
    if (st < nkt) issue(st, st);
  wait_stage(min(NST, nkt) - 1);
  __builtin_amdgcn_s_barrier();
  read_x(0);

  // Per stage kt: read step 1 while step 0 multiplies; then (all of stage kt
  // read, stage kt+1 landed everywhere) refill stage kt's buffer with stage
  // kt+NST and read stage kt+1's step 0 while step 1 multiplies.  Barriers are
  // bare s_barrier: the waits that make them safe are explicit.  The
  // sched_barriers pin this order (the scheduler would otherwise sink each
  // fragment read next to its first use).
  for (int kt = 0; kt < nkt; ++kt) {
    const int st = kt % NST;
    // First half of step 0's MFMAs (its fragments were read a step earlier),
    // then the reads of step 1, then the rest of step 0.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RB / 2; ++r)
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[r][c] = mfma32<DT>(xa[r], xb[c], acc[r][c]);
    __builtin_amdgcn_sched_barrier(0);
    read_y(st);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = RB / 2; r < RB; ++r)
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[r][c] = mfma32<DT>(xa[r], xb[c], acc[r][c]);
    __builtin_amdgcn_sched_barrier(0);
    // Unconditional (the last stage reads a valid buffer it never uses): a
    // branch here makes the wait-count pass wait for these reads before the
    // step-1 MFMAs below.
    wait_lgkmcnt0();
    wait_stage(max(min(kt + NST, nkt) - 1 - (kt + 1), 0));
    __builtin_amdgcn_s_barrier();
    if (kt + NST < nkt) issue(st, kt + NST);
    read_x((kt + 1) % NST);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[r][c] = mfma32<DT>(ya[r], yb[c], acc[r][c]);
    __builtin_amdgcn_sched_barrier(0);
  }

#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int m = n0 + col_base[c] + l32;
    if (m >= a.M) continue;
    const int mb = m / a.T, mt = m - mb * a.T, mpos = a.start_pos + mt;  // QKV only
#pragma unroll
    for (int r = 0; r < (SWI ? RB / 2 : RB); ++r) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int f = f0 + row_base[r] + g4 * 8 + h2 * 4;
        if (f >= a.N) continue;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = acc[r][c][g4 * 4 + i];
        if constexpr (EPI == EPI_RESID) {
          const T* rp = reinterpret_cast<const T*>(a.resid) + (size_t)m * a.N + f;
          float rv[4];
          load4<DT>(rp, rv);
          T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
          store4<DT>(y, rv[0] + v[0], rv[1] + v[1], rv[2] + v[2], rv[3] + v[3]);
        } else if constexpr (SWI) {
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = silu(v[i]) * acc[r + RB / 2][c][g4 * 4 + i];
          T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
          store4<DT>(y, o[0], o[1], o[2], o[3]);
        } else {
          gemm_qkv_store<KVDT>(a, mb, mt, mpos, f, v);
        }
      }
    }
  }
}

// 256 x 256 tiles when they still give ~3 rounds of workgroups over the CUs.
static bool use_big_tile(int epi, int N, int M) {
  const int fm = (epi == EPI_SWIGLU) ? 128 : 256;
  const long tiles = (long)((N + fm - 1) / fm) * ((M + 255) / 256);
  return tiles >= 3 * 256;
}

template <int DT, int EPI, int BM, int BN, int KVDT>
static hipError_t gemm_launch(const ProjArgs& a, hipStream_t s) {
  const int fm = (EPI == EPI_SWIGLU) ? BM / 2 : BM;
  const int ntiles = ((a.N + fm - 1) / fm) * ((a.M + BN - 1) / BN);
  LL_LAUNCH((gemm_kernel<DT, EPI, BM, BN, KVDT>), dim3(ntiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int EPI, int BM, int BN, int KVDT, int NW>
static hipError_t gemm_dma_launch(const ProjArgs& a, hipStream_t s) {
  const int fm = (EPI == EPI_SWIGLU) ? BM / 2 : BM;
  const int ntiles = ((a.N + fm - 1) / fm) * ((a.M + BN - 1) / BN);
  LL_LAUNCH((gemm_dma_kernel<DT, EPI, BM, BN, KVDT, NW>), dim3(ntiles), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <int DT, int EPI, int KVDT>
static hipError_t gemm_epi(const ProjArgs& a, hipStream_t s) {
  const bool big = use_big_tile(EPI, a.N, a.M);
  if (a.K % 32 == 0)
    return big ? gemm_dma_launch<DT, EPI, 256, 256, KVDT, GEMM_BIG_WAVES>(a, s)
               : gemm_dma_launch<DT, EPI, 128, 128, KVDT, 4>(a, s);
  return big ? gemm_launch<DT, EPI, 256, 256, KVDT>(a, s) : gemm_launch<DT, EPI, 128, 128, KVDT>(a, s);
}

template <int DT>
static hipError_t gemm_dt(int epi, const ProjArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_QKV:
      if (a.kv_dt == DT_BF16) return gemm_epi<DT, EPI_QKV, DT_BF16>(a, s);
      if (a.kv_dt == DT_F16) return gemm_epi<DT, EPI_QKV, DT_F16>(a, s);
      return hipErrorInvalidValue;
    case EPI_RESID: return gemm_epi<DT, EPI_RESID, DT>(a, s);
    case EPI_SWIGLU: return gemm_epi<DT, EPI_SWIGLU, DT>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int dt, int epi, const ProjArgs& a, hipStream_t s) {
  if (dt == DT_BF16) return gemm_dt<DT_BF16>(epi, a, s);
  if (dt == DT_F16) return gemm_dt<DT_F16>(epi, a, s);
  return hipErrorInvalidValue;
}

}  // namespace ll
