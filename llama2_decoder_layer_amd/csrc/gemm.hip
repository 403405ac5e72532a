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
    dst = cache + kv_row(a.pages, b, j, pos, a.nkv, a.s_max, hd) + (g - j * hd);
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
// Direct-to-LDS variant (K % 32 == 0; K % 64 == 0 for 256 x 256 tiles).
// Operands move global -> LDS with global_load_lds_dwordx4 (lane l of a wave
// writes bytes [16 l, 16 l + 16) of the LDS destination), so no registers
// stage them and no ds_write is issued; the swizzled LDS layout comes from
// permuting each lane's global address.  BK-k stages, NST of them in LDS,
// loads NST-1 stages ahead of the multiply.  A row slice is 2 BK bytes, and
// the rows sharing a 256-byte bank sweep get distinct chunk orders: chunk c
// of row r is stored at c ^ ((r / rows_per_sweep) % chunks_per_row).
// ---------------------------------------------------------------------------
// Occupancy target per SIMD: 4 waves on a 256 x 256 tile hold 256 accumulator
// registers each (one wave per SIMD); 8 waves hold 128 (two per SIMD, so one
// wave's barrier and LDS waits overlap the other's MFMAs).  Telling the
// compiler lets it keep fragments in flight instead of chasing occupancy.
template <int BM, int NW>
struct DmaOcc { static constexpr int waves = (BM == 256 && NW == 4) ? 1 : 2; };

// Tile geometry of the direct-to-LDS kernel.  Wave grid over (rows, tokens):
// 2 x NW/2, each wave BM/2 rows x 2 BN/NW tokens.  With SwiGLU the tile's
// rows are FM gate rows then the FM matching up rows, and wave half wm takes
// gate rows [wm FM/2, (wm+1) FM/2) with the up rows of the same features, so
// gate and up of a feature meet in one lane.
template <int EPI, int BM, int BN, int NW>
struct DmaTile {
  static constexpr bool SWI = (EPI == EPI_SWIGLU);
  static constexpr int FM = SWI ? BM / 2 : BM;     // output features per tile
  static constexpr int WN = NW / 2;                // waves along tokens
  static constexpr int RB = BM / 64;               // 32-row blocks per wave
  static constexpr int CB = BN / WN / 32;          // 32-token blocks per wave
  static constexpr int ACC = RB * CB * 16;         // accumulators per lane
};

// Tile t -> first feature and first token: groups of GROUP_M weight panels,
// token panels inner.
__device__ __forceinline__ void dma_tile_origin(int t, int ntm, int ntn, int fm, int bn, int& f0,
                                                int& n0) {
  const int per_group = GROUP_M * ntn;
  const int grp = t / per_group;
  const int first_m = grp * GROUP_M;
  const int gm = min(ntm - first_m, GROUP_M);
  const int in_grp = t - grp * per_group;
  f0 = (first_m + in_grp % gm) * fm;
  n0 = (in_grp / gm) * bn;
}

// First row and token of each 32 x 32 accumulator block of this wave.
template <int EPI, int BM, int BN, int NW>
__device__ __forceinline__ void dma_wave_bases(int wave, int (&row_base)[DmaTile<EPI, BM, BN, NW>::RB],
                                               int (&col_base)[DmaTile<EPI, BM, BN, NW>::CB]) {
  typedef DmaTile<EPI, BM, BN, NW> G;
  const int wm = wave / G::WN, wn = wave % G::WN;
  if constexpr (G::SWI) {
    // blocks [0, RB/2): gate rows; [RB/2, RB): the up rows of the same features
#pragma unroll
    for (int r = 0; r < G::RB; ++r)
      row_base[r] = (r < G::RB / 2 ? 0 : G::FM) + wm * (G::FM / 2) + (r % (G::RB / 2)) * 32;
  } else {
#pragma unroll
    for (int r = 0; r < G::RB; ++r) row_base[r] = wm * (BM / 2) + r * 32;
  }
#pragma unroll
  for (int c = 0; c < G::CB; ++c) col_base[c] = wn * (BN / G::WN) + c * 32;
}

// Epilogue of one 32 x 32 accumulator block (rows from row0, token m) from a
// lane's accumulators: residual add, SwiGLU (up: the matching up block), or
// RoPE + KV append.
template <int DT, int EPI, int KVDT>
__device__ __forceinline__ void dma_store_block(const ProjArgs& a, const f32x16& acc,
                                                const f32x16& up, int row0, int m, int h2) {
  typedef typename Elt<DT>::T T;
  const int mb = m / a.T, mt = m - mb * a.T, mpos = a.start_pos + mt;  // QKV only
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const int f = row0 + g4 * 8 + h2 * 4;
    if (f >= a.N) continue;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = acc[g4 * 4 + i];
    if constexpr (EPI == EPI_RESID) {
      const T* rp = reinterpret_cast<const T*>(a.resid) + (size_t)m * a.N + f;
      float rv[4];
      load4<DT>(rp, rv);
      T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
      store4<DT>(y, rv[0] + v[0], rv[1] + v[1], rv[2] + v[2], rv[3] + v[3]);
    } else if constexpr (EPI == EPI_SWIGLU) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = silu(v[i]) * up[g4 * 4 + i];
      T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
      store4<DT>(y, o[0], o[1], o[2], o[3]);
    } else {
      gemm_qkv_store<KVDT>(a, mb, mt, mpos, f, v);
    }
  }
}

// Epilogue of one tile from a lane's accumulators.
template <int DT, int EPI, int BM, int BN, int KVDT, int NW>
__device__ __forceinline__ void dma_store_tile(const ProjArgs& a,
                                               f32x16 (&acc)[DmaTile<EPI, BM, BN, NW>::RB]
                                                            [DmaTile<EPI, BM, BN, NW>::CB],
                                               int f0, int n0, int wave, int lane) {
  typedef DmaTile<EPI, BM, BN, NW> G;
  int row_base[G::RB], col_base[G::CB];
  dma_wave_bases<EPI, BM, BN, NW>(wave, row_base, col_base);
  const int l32 = lane & 31, h2 = lane >> 5;
#pragma unroll
  for (int c = 0; c < G::CB; ++c) {
    const int m = n0 + col_base[c] + l32;
    if (m >= a.M) continue;
#pragma unroll
    for (int r = 0; r < (G::SWI ? G::RB / 2 : G::RB); ++r)
      dma_store_block<DT, EPI, KVDT>(a, acc[r][c], acc[G::SWI ? r + G::RB / 2 : r][c],
                                     f0 + row_base[r], m, h2);
  }
}

// Pipeline: k per stage and stages in LDS.  The 256 x 256 and 192 x 256
// tiles take 64-k stages (half the barriers per MFMA of 32-k stages), two of
// them (128 and 112 KB).
#ifndef GEMM_BIG_BK
#define GEMM_BIG_BK 64
#endif
template <int BM>
struct DmaPipe {
  static constexpr int BK = (BM >= 192) ? GEMM_BIG_BK : 32;
  static constexpr int NST = (BK == 64) ? 2 : 4;
};

// Workgroups [0, full_tiles) each take a whole tile.  When the tiles do not
// fill a whole number of rounds over the CUs, the remaining tiles are split
// along K into ksplit parts, one workgroup each, so the last round is full;
// those write float32 partials (accumulator quads of all threads in turn, so
// the stores and loads coalesce) and gemm_split_reduce_kernel sums them and
// applies the epilogue.
template <int DT, int EPI, int BM, int BN, int KVDT, int NW>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(DmaOcc<BM, NW>::waves, DmaOcc<BM, NW>::waves)))
void gemm_dma_kernel(ProjArgs a, float* part, int full_tiles, int ksplit) {
  typedef typename Elt<DT>::T T;
  constexpr int BK = DmaPipe<BM>::BK;
  constexpr int NST = DmaPipe<BM>::NST;
  constexpr int KS = BK / 16;                  // 16-k MFMA steps per stage
  constexpr int ROWB = BK * 2;                 // bytes per row slice (64 or 128)
  constexpr int LPR = ROWB / 16;               // lanes per row in a DMA instruction
  constexpr int RPI = 64 / LPR;                // rows per 1 KB wave instruction
  constexpr int RPS = 256 / ROWB;              // rows per 256-byte bank sweep
  constexpr int CPR = ROWB / 16;               // 16-byte chunks per row slice
  constexpr int AI = BM / RPI / NW;            // A instructions per wave per stage
  constexpr int BI = BN / RPI / NW;
  constexpr int STAGE = (BM + BN) * ROWB;
  typedef DmaTile<EPI, BM, BN, NW> G;
  constexpr bool SWI = G::SWI;
  constexpr int FM = G::FM;
  constexpr int RB = G::RB;
  constexpr int CB = G::CB;

  __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const int ntm = (a.N + FM - 1) / FM;
  const int ntn = (a.M + BN - 1) / BN;
  // Workgroup i runs on XCD i % 8: give each XCD a contiguous range of the
  // whole tiles and, separately, of the split parts, so every XCD gets its
  // share of both.
  int b2 = blockIdx.x;
  {
    const bool in_full = b2 < full_tiles;
    const int lo = in_full ? 0 : full_tiles;
    const int n = in_full ? full_tiles : gridDim.x - full_tiles;
    const int i = b2 - lo;
    if ((n & 7) == 0) b2 = lo + (i & 7) * (n >> 3) + (i >> 3);
  }
  // Whole tile, or one K part of a split tile.
  const int nkt_all = K / BK;
  int tile = b2, kt_begin = 0, kt_end = nkt_all, pidx = -1;
  if (b2 >= full_tiles) {
    pidx = b2 - full_tiles;
    tile = full_tiles + pidx / ksplit;
    const int per = (nkt_all + ksplit - 1) / ksplit;
    kt_begin = min(nkt_all, (pidx % ksplit) * per);
    kt_end = min(nkt_all, kt_begin + per);
  }
  int f0, n0;
  dma_tile_origin(tile, ntm, ntn, FM, BN, f0, n0);

  // DMA sources: lane l fills row l / LPR of its RPI-row slab, physical chunk
  // l % LPR, i.e. logical chunk (l % LPR) ^ ((row / RPS) % CPR): the rows that
  // share a 256-byte bank sweep get distinct chunk orders.  Rows past N or M
  // read row 0 (their results are never stored).
  const int rr = lane / LPR, pc = lane % LPR;
  const T* asrc[AI];
  const T* bsrc[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (wave * AI + i) * RPI + rr;
    const int c = pc ^ ((r / RPS) % CPR);
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
    const int c = pc ^ ((r / RPS) % CPR);
    const int m = n0 + r;
    bsrc[i] = reinterpret_cast<const T*>(a.x) + (size_t)(m < a.M ? m : 0) * K + c * 8;
  }
  auto issue = [&](int st, int kt) {
    uint8_t* base = lds + st * STAGE;
    const int k = (kt_begin + kt) * BK;
#pragma unroll
    for (int i = 0; i < AI; ++i) dma16(asrc[i] + k, base + (wave * AI + i) * 1024);
#pragma unroll
    for (int i = 0; i < BI; ++i) dma16(bsrc[i] + k, base + BM * ROWB + (wave * BI + i) * 1024);
  };

  int row_base[RB], col_base[CB];
  dma_wave_bases<EPI, BM, BN, NW>(wave, row_base, col_base);
  const int l32 = lane & 31, h2 = lane >> 5;
  int aoff[RB], boff[CB];  // byte offsets of this lane's fragment rows (chunk added per step)
#pragma unroll
  for (int r = 0; r < RB; ++r) aoff[r] = (row_base[r] + l32) * ROWB;
#pragma unroll
  for (int c = 0; c < CB; ++c) boff[c] = BM * ROWB + (col_base[c] + l32) * ROWB;
  // row_base is a multiple of 32, so (row / RPS) % CPR == (l32 / RPS) % CPR.
  const int swz_a = (l32 / RPS) % CPR;

  f32x16 acc[RB][CB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.f;

  // Two fragment sets alternate over the 16-k steps: the next step's
  // fragments are read while the current step multiplies.
  u32x4 fa[2][RB], fb[2][CB];
  auto read_set = [&](auto set, int st, int ks) {
    constexpr int S = decltype(set)::value;
    const uint8_t* base = lds + st * STAGE;
    const int chb = ((2 * ks + h2) ^ swz_a) * 16;
#pragma unroll
    for (int r = 0; r < RB; ++r) fa[S][r] = ld16(base + aoff[r] + chb);
#pragma unroll
    for (int c = 0; c < CB; ++c) fb[S][c] = ld16(base + boff[c] + chb);
  };
  // Wait until this wave's DMA of a stage has landed: at most the loads of the
  // `newer` stages issued after it may still be outstanding.
  auto wait_stage = [&](int newer) {
    if (newer >= 3) wait_vmcnt<3 * (AI + BI)>();
    else if (newer == 2) wait_vmcnt<2 * (AI + BI)>();
    else if (newer == 1) wait_vmcnt<1 * (AI + BI)>();
    else wait_vmcnt<0>();
  };

  const int nkt = kt_end - kt_begin;
  if constexpr (NST == 2) {
    // Two 64-k stages.  Stage kt+1 streams into the other buffer while stage
    // kt is multiplied, its DMA instructions spread between the MFMAs of the
    // stage's first half (one per MPD MFMAs) instead of issued as a burst
    // after the barrier: a burst of 8 x 1 KB per wave filled the vector-memory
    // queue, and the in-order issue held every wave's next MFMAs behind it
    // (13B gate/up 1190 -> 1139 us, 70B gate/up at 1024 tokens 1010 -> 981 us,
    // on one box with alternating builds).  The stage then ends with this
    // wave's DMA of stage kt+1 landed (vmcnt 0), all fragment reads of stage
    // kt done, and the one barrier, after which stage kt+1's first fragments
    // are read.
    constexpr int NDMA = AI + BI;                       // DMA instructions per wave per stage
    constexpr int MPD = (KS * RB * CB) / (2 * NDMA);    // MFMAs between two of them
    static_assert(MPD >= 1 && NDMA * MPD <= KS * RB * CB / 2,
                  "every DMA of a stage is issued before its sync point");
    auto issue_one = [&](int st, int kt, int i) {
      uint8_t* base = lds + st * STAGE;
      const int k = (kt_begin + kt) * BK;
      if (i < AI) dma16(asrc[i] + k, base + (wave * AI + i) * 1024);
      else dma16(bsrc[i - AI] + k, base + BM * ROWB + (wave * BI + (i - AI)) * 1024);
    };
    issue(0, 0);
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    read_set(ic<0>{}, 0, 0);
    for (int kt = 0; kt < nkt; ++kt) {
      const int st = kt & 1;
      const bool pre = kt + 1 < nkt;
      static_for<0, KS>([&](auto KSI) {
        constexpr int ks = decltype(KSI)::value;
        constexpr int S = ks & 1;
        static_for<0, RB * CB>([&](auto MI) {
          constexpr int m = decltype(MI)::value;
          constexpr int g = ks * RB * CB + m;  // MFMA index within the stage
          __builtin_amdgcn_sched_barrier(0);
          acc[m / CB][m % CB] = mfma32<DT>(fa[S][m / CB], fb[S][m % CB], acc[m / CB][m % CB]);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr ((g + 1) % MPD == 0 && (g + 1) / MPD <= NDMA) {
            if (pre) issue_one(st ^ 1, kt + 1, (g + 1) / MPD - 1);
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (m == RB * CB / 2 - 1) {  // mid-step: the next step's fragments
            if constexpr (ks + 1 < KS) {
              read_set(ic<S ^ 1>{}, st, ks + 1);
            } else {
              // Unconditional (the last stage reads a valid buffer it never
              // uses): a branch here makes the wait-count pass wait for these
              // reads before the MFMAs that follow.
              wait_lgkmcnt0();
              wait_vmcnt<0>();
              __builtin_amdgcn_s_barrier();
              read_set(ic<S ^ 1>{}, st ^ 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int st = 0; st < NST; ++st)
      if (st < nkt) issue(st, st);
    wait_stage(min(NST, nkt) - 1);
    __builtin_amdgcn_s_barrier();
    read_set(ic<0>{}, 0, 0);

    // Per 16-k step: the first half of its MFMAs, then the reads of the next
    // step, then the second half.  After the first half of a stage's last step
    // (all of the stage read, the next stage landed everywhere) comes the one
    // barrier of the stage; then the buffer just finished is refilled with
    // stage kt+NST and the next stage's first step is read.  Barriers are bare
    // s_barrier: the waits that make them safe are explicit.  The
    // sched_barriers pin this order (the scheduler would otherwise sink each
    // fragment read next to its first use).
    for (int kt = 0; kt < nkt; ++kt) {
      const int st = kt % NST;
      static_for<0, KS>([&](auto KSI) {
        constexpr int ks = decltype(KSI)::value;
        constexpr int S = ks & 1;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < RB / 2; ++r)
#pragma unroll
          for (int c = 0; c < CB; ++c) acc[r][c] = mfma32<DT>(fa[S][r], fb[S][c], acc[r][c]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ks + 1 < KS) {
          read_set(ic<S ^ 1>{}, st, ks + 1);
        } else {
          wait_lgkmcnt0();
          wait_stage(max(min(kt + NST, nkt) - 1 - (kt + 1), 0));
          __builtin_amdgcn_s_barrier();
          if (kt + NST < nkt) issue(st, kt + NST);
          read_set(ic<S ^ 1>{}, (kt + 1) % NST, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = RB / 2; r < RB; ++r)
#pragma unroll
          for (int c = 0; c < CB; ++c) acc[r][c] = mfma32<DT>(fa[S][r], fb[S][c], acc[r][c]);
      });
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (pidx >= 0) {  // one K part of a split tile: float32 partials, [part][quad][thread]
    f32x4* p = reinterpret_cast<f32x4*>(part) + (size_t)pidx * (G::ACC / 4) * (NW * 64) + tid;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {acc[r][c][4 * q], acc[r][c][4 * q + 1], acc[r][c][4 * q + 2],
                           acc[r][c][4 * q + 3]};
          p[(size_t)((r * CB + c) * 4 + q) * (NW * 64)] = v;
        }
    return;
  }
  dma_store_tile<DT, EPI, BM, BN, KVDT, NW>(a, acc, f0, n0, wave, lane);
}

// Sum of the K parts of each split tile, then the tile's epilogue.  A thread
// takes BPT of the 32 x 32 accumulator blocks of one lane of the tile, one
// 32-token column of them (SwiGLU: one gate block and its up block), and
// loads every part of them before adding any; the part count KS is a
// template argument.  Measured against one thread per lane summing all its
// blocks part by part (13B O/down at 4096 tokens, 4 parts; the stack's O/down
// and gate/up at 1024 tokens, 2 parts): 28.9, 25.1 and 18.1 us; with the
// parts batched 24.8, 24.6, 16.4 us; a column of four blocks per thread
// (one for SwiGLU) 17.9, 24.0, 13.5 us; two blocks 20.2, 28.1 us; one block
// 21.3, 29.7 us.
constexpr int SPLIT_REDUCE_THREADS = 256;
constexpr int SPLIT_REDUCE_BPT = 4;
template <int EPI, int RBO>
constexpr int split_reduce_bpt() {
  return (EPI == EPI_SWIGLU || RBO % SPLIT_REDUCE_BPT != 0) ? 1 : SPLIT_REDUCE_BPT;
}
template <int DT, int EPI, int BM, int BN, int KVDT, int NW, int KS>
__global__ __launch_bounds__(SPLIT_REDUCE_THREADS) void gemm_split_reduce_kernel(
    ProjArgs a, const float* part, int full_tiles) {
  typedef DmaTile<EPI, BM, BN, NW> G;
  constexpr int RBO = G::SWI ? G::RB / 2 : G::RB;  // output row blocks per lane
  constexpr int BPT = split_reduce_bpt<EPI, RBO>();  // of them per thread
  static_assert(RBO % BPT == 0, "row blocks per thread");
  constexpr int TT = NW * 64 * (RBO / BPT) * G::CB;  // threads per tile
  static_assert(TT % SPLIT_REDUCE_THREADS == 0, "whole workgroups per tile");
  constexpr int PER_TILE = TT / SPLIT_REDUCE_THREADS;
  const int tile_local = blockIdx.x / PER_TILE;
  const int t = (blockIdx.x - tile_local * PER_TILE) * SPLIT_REDUCE_THREADS + threadIdx.x;
  // Consecutive threads take consecutive lanes of one block: the partial loads
  // of a warp read consecutive 16-byte quads.
  const int blk = t / (NW * 64), tid = t - blk * (NW * 64);
  const int r0 = (blk / G::CB) * BPT, c = blk % G::CB;
  const int lane = tid & 63, wave = tid >> 6;
  const int tile = full_tiles + tile_local;
  const f32x4* p0 = reinterpret_cast<const f32x4*>(part) +
                    (size_t)(tile_local * KS) * (G::ACC / 4) * (NW * 64) + tid;
  auto sum_block = [&](int rr) {
    f32x4 v[KS][4];
#pragma unroll
    for (int sp = 0; sp < KS; ++sp)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[sp][q] = __builtin_nontemporal_load(p0 + (size_t)sp * (G::ACC / 4) * (NW * 64) +
                                              (size_t)((rr * G::CB + c) * 4 + q) * (NW * 64));
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int sp = 0; sp < KS; ++sp)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * q + i] += v[sp][q][i];
    return acc;
  };
  f32x16 acc[BPT], up[BPT];
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    acc[b] = sum_block(r0 + b);
    up[b] = G::SWI ? sum_block(r0 + b + G::RB / 2) : acc[b];
  }
  const int ntm = (a.N + G::FM - 1) / G::FM;
  const int ntn = (a.M + BN - 1) / BN;
  int f0, n0;
  dma_tile_origin(tile, ntm, ntn, G::FM, BN, f0, n0);
  int row_base[G::RB], col_base[G::CB];
  dma_wave_bases<EPI, BM, BN, NW>(wave, row_base, col_base);
  const int m = n0 + col_base[c] + (lane & 31);
  if (m >= a.M) return;
#pragma unroll
  for (int b = 0; b < BPT; ++b)
    dma_store_block<DT, EPI, KVDT>(a, acc[b], up[b], f0 + row_base[r0 + b], m, lane >> 5);
}

// Workgroups resident at once with 256 x 256 tiles (one per CU on gfx950's
// 256 CUs): a "round".
constexpr int GEMM_ROUND = 256;
#ifndef GEMM_BIG_MIN_FRAC
#define GEMM_BIG_MIN_FRAC 4
#endif

static long big_tiles(int epi, int N, int M) {
  const int fm = (epi == EPI_SWIGLU) ? 128 : 256;
  return (long)((N + fm - 1) / fm) * ((M + 255) / 256);
}

// Register-staged kernel: 256 x 256 tiles when they give ~3 rounds.
static bool use_big_tile(int epi, int N, int M) { return big_tiles(epi, N, M) >= 3 * GEMM_ROUND; }

// Direct-to-LDS kernel: 256 x 256 tiles from one full round on; a partly
// filled last round is made full by splitting its tiles along K.
struct DmaSplit {
  int full, ksplit, grid;
};
static DmaSplit dma_split(long ntiles, int nkt) {
  DmaSplit d{(int)ntiles, 1, (int)ntiles};
  const long full = (ntiles / GEMM_ROUND) * GEMM_ROUND, rem = ntiles - full;
  if (rem == 0) return d;
  // The tiles of the last round split into as many K parts as still fit in
  // one round (at most 4).  Rounding up instead would spill the parts into a
  // second round and finish no sooner than whole tiles, plus the reduction:
  // the 70B QKV at 1024 tokens (160 tiles) took 250 us in 320 half-K parts
  // against 206 us unsplit (three parts in two rounds: 231 us).
  const int ks = (int)std::min<long>(std::min<long>(GEMM_ROUND / rem, 4), nkt);
  if (ks < 2) return d;
  d.full = (int)full;
  d.ksplit = ks;
  d.grid = (int)(full + rem * ks);
  return d;
}
// 256 x 256 tiles from a quarter round on (smaller launches split along K).
static bool dma_big(int epi, int N, int M, int K) {
  return K % DmaPipe<256>::BK == 0 && big_tiles(epi, N, M) >= GEMM_ROUND / GEMM_BIG_MIN_FRAC;
}

size_t gemm_partial_bytes(int epi, int N, int M, int K) {
  if (K % 32 != 0 || !dma_big(epi, N, M, K)) return 0;
  const DmaSplit d = dma_split(big_tiles(epi, N, M), K / DmaPipe<256>::BK);
  // 512 threads x 128 accumulators (8 waves, 256 x 256 tile) per K part
  return (size_t)(d.grid - d.full) * 512 * 128 * sizeof(float);
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
  const long ntiles = (long)((a.N + fm - 1) / fm) * ((a.M + BN - 1) / BN);
  DmaSplit d{(int)ntiles, 1, (int)ntiles};
  if (BM == 256) d = dma_split(ntiles, a.K / DmaPipe<BM>::BK);
  if (d.grid != d.full && !a.part) return hipErrorInvalidValue;
  LL_LAUNCH((gemm_dma_kernel<DT, EPI, BM, BN, KVDT, NW>), dim3(d.grid), dim3(NW * 64), 0, s, a,
            a.part, d.full, d.ksplit);
  if (d.grid != d.full) {
    static_assert(DmaTile<EPI, 256, 256, GEMM_BIG_WAVES>::ACC * GEMM_BIG_WAVES * 64 == 512 * 128,
                  "partial size per K part");
    typedef DmaTile<EPI, BM, BN, NW> G;
    constexpr int RBO = G::SWI ? G::RB / 2 : G::RB;
    const int per_tile = NW * 64 * (RBO / split_reduce_bpt<EPI, RBO>()) * G::CB / SPLIT_REDUCE_THREADS;
    const dim3 rg(((int)ntiles - d.full) * per_tile);
    const dim3 rb(SPLIT_REDUCE_THREADS);
    const float* pp = a.part;
    switch (d.ksplit) {  // dma_split makes 2, 3 or 4 parts
      case 2: LL_LAUNCH((gemm_split_reduce_kernel<DT, EPI, BM, BN, KVDT, NW, 2>), rg, rb, 0, s, a, pp, d.full); break;
      case 3: LL_LAUNCH((gemm_split_reduce_kernel<DT, EPI, BM, BN, KVDT, NW, 3>), rg, rb, 0, s, a, pp, d.full); break;
      case 4: LL_LAUNCH((gemm_split_reduce_kernel<DT, EPI, BM, BN, KVDT, NW, 4>), rg, rb, 0, s, a, pp, d.full); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

// 192 x 256 tiles (three 32-row blocks per wave) where the 256 x 256 tiles
// fill more than half of one round, too many to split along K, and the
// 192-row tiles still fit in one round: the launch then ends after 3/4 of a
// 256-row tile's work.  The 70B QKV at 1024 tokens (160 tiles of 256 rows,
// 216 of 192): 206-212 -> 167.5 us, with identical results (each output's sum
// runs in the same order).  SwiGLU tiles keep 256 rows (gate and up halves).
static bool dma_mid(int epi, int N, int M, int K) {
  if (epi == EPI_SWIGLU || K % 64 != 0 || !dma_big(epi, N, M, K)) return false;
  const long t256 = big_tiles(epi, N, M);
  const long t192 = (long)((N + 191) / 192) * ((M + 255) / 256);
  return t256 < GEMM_ROUND && 2 * t256 > GEMM_ROUND && t192 <= GEMM_ROUND;
}

template <int DT, int EPI, int KVDT>
static hipError_t gemm_epi(const ProjArgs& a, hipStream_t s) {
  if (a.K % 32 == 0) {
    if (dma_mid(EPI, a.N, a.M, a.K)) return gemm_dma_launch<DT, EPI, 192, 256, KVDT, 8>(a, s);
    return dma_big(EPI, a.N, a.M, a.K) ? gemm_dma_launch<DT, EPI, 256, 256, KVDT, GEMM_BIG_WAVES>(a, s)
                                  : gemm_dma_launch<DT, EPI, 128, 128, KVDT, 4>(a, s);
  }
  const bool big = use_big_tile(EPI, a.N, a.M);
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
