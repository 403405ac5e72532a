// Weight-streaming projection for up to 32 tokens in a 16-bit format:
// D[f, m] = sum_k W[f, k] x[m, k], every weight byte read once from HBM.
//
// A workgroup owns 64 weight rows (SwiGLU: 32 gate + the 32 matching up rows)
// and all token slots (32, the missing ones read token 0 and are dropped), over
// one K range.  Weights and activations move global -> LDS by
// global_load_lds in 256-k stages (512-byte row slices), three deep (144 KB of
// LDS, one workgroup per CU), so each row has 1 KB in flight and each CU
// 64 KB of weights.  The eight waves split a stage's work as 2 row blocks x 4
// k slices of v_mfma_f32_32x32x16; the k slices meet in LDS at the end (four
// waves with k halves: 70B gate/up at 32 tokens 155.5 -> 154.0 us, step
// 380.5 -> 377.3 us).  Launches without a K split take a 128-row shape with
// 128-k stages four deep instead (see the shape constants below).
// Measured on the 70B gate/up at 32 tokens (four waves, 64 rows) against
// 64-k stages four deep with three workgroups per CU (128-byte slices, 384
// bytes per row in flight): 183 -> 173 us; 128-k stages six deep (one
// workgroup per CU) were slower (196 us), three deep with two workgroups per
// CU in between (176 us).
//
// The 16-byte chunks of a row slice are stored XOR-swizzled by (row & 15),
// which makes the fragment reads conflict-free: the 16 rows one ds_read_b128
// cycle serves land in 16 distinct 4-bank groups.
//
// Few row blocks (O, down, QKV at batch 32) leave CUs idle, so the K range is
// split over several workgroups; each split writes float32 partials and a
// small kernel sums them and applies the epilogue.  One split applies the
// epilogue directly: residual add, SwiGLU, RoPE + KV append, or logits.
#include "common.cuh"
#include "epilogue.cuh"

namespace ll {

// Two workgroup shapes: 64 weight rows in 256-k stages three deep (144 KB of
// LDS), and 128 rows in 128-k stages four deep (160 KB, 96 KB of weights in
// flight per CU).  The 128-row shape serves launches that need no K split
// (70B gate/up at 32 tokens: 153.0 -> 141.8 us); K-split launches keep 64
// rows (O, down and QKV were each ~1 us slower with 128).
constexpr int SK_BM = 64;                          // weight rows per workgroup
constexpr int SK_BK = 256;                         // k per stage
constexpr int SK_NST = 3;                          // stages in LDS
constexpr int SK_BM_W = 128;                       // the same, 128-row shape
constexpr int SK_BK_W = 128;
constexpr int SK_NST_W = 4;
constexpr int SK_BN = 32;                          // token slots
constexpr int SK_NW = 8;                           // waves per workgroup
constexpr int SK_TARGET_WG = 512;                  // workgroups wanted per launch
constexpr int SK_MAX_SPLIT = 8;

// Features covered by one workgroup of bm rows.
static int sk_features(int epi, int bm = SK_BM) { return epi == EPI_SWIGLU ? bm / 2 : bm; }

// Splits of K for a launch whose workgroups cover `feats` features each, to
// reach about `target` workgroups.
static int sk_split_f(int feats, int N, int K, int* kchunk, int target = SK_TARGET_WG) {
  const int nblk = (N + feats - 1) / feats;
  int ns = (target + nblk - 1) / nblk;
  ns = std::max(1, std::min(ns, SK_MAX_SPLIT));
  // A partly filled last round of 256 workgroups: one split fewer when that
  // still fills a round (70B QKV at 32 tokens: 640 -> 480 workgroups,
  // 40 -> 34 us).
  if (ns > 1 && (nblk * ns) % 256 != 0 && nblk * (ns - 1) >= 256) --ns;
  const int nkt = K / 64;
  ns = std::min(ns, nkt);
  const int kt_per = (nkt + ns - 1) / ns;
  *kchunk = kt_per * 64;
  return (nkt + kt_per - 1) / kt_per;
}

static int sk_split(int epi, int N, int K, int* kchunk, int bm = SK_BM) {
  return sk_split_f(sk_features(epi, bm), N, K, kchunk);
}

// Whether a launch takes the 128-row shape: when it needs no K split there.
static bool sk_wide(int epi, int N, int K) {
  int kchunk;
  return sk_split(epi, N, K, &kchunk, SK_BM_W) == 1;
}

// Code rows per workgroup of the int8 streaming kernel, its features, and the
// workgroups wanted per launch (one per CU at 144 KB of LDS).
constexpr int W8_BMW = 128;
constexpr int W8_TARGET_WG = 256;
static int w8_features(int epi) { return epi == EPI_SWIGLU ? W8_BMW / 2 : W8_BMW; }

// Weight rows of a launch: N (SwiGLU: gate rows then up rows, 2N).
static int sk_rows(int epi, int N) { return epi == EPI_SWIGLU ? 2 * N : N; }

// Deferred norm: each token has SK_SSQ_MAX partial-sum slots in a.ssq (16
// floats, 64 bytes); slots past a.ssq_parts hold zeros, so readers sum all of
// them in slot order (hidden sizes up to 16384).
constexpr int SK_SSQ_MAX = 16;

// 1 / rms of token m's input from the partial sums of squares that the
// residual projection before it left in a.ssq.
__device__ __forceinline__ float sk_rstd(const ProjArgs& a, int m) {
  const f32x4* p = reinterpret_cast<const f32x4*>(a.ssq + (size_t)m * SK_SSQ_MAX);
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < SK_SSQ_MAX / 4; ++i) {
    const f32x4 v = p[i];
    t += v[0]; t += v[1]; t += v[2]; t += v[3];
  }
  return 1.0f / sqrtf(t / (float)a.K + a.eps);
}

// A lane's slots for sk_rstd, loaded ahead (after a k loop's first loads are
// issued) so that their latency is not paid at the end of the workgroup.
struct SsqAhead {
  f32x4 v[SK_SSQ_MAX / 4];
  __device__ __forceinline__ void load(const ProjArgs& a, int m) {
    if (!a.ssq) return;
    const f32x4* p = reinterpret_cast<const f32x4*>(a.ssq + (size_t)(m < a.M ? m : 0) * SK_SSQ_MAX);
#pragma unroll
    for (int i = 0; i < SK_SSQ_MAX / 4; ++i) v[i] = p[i];
  }
  // Summed in the order sk_rstd uses.
  __device__ __forceinline__ float rstd(const ProjArgs& a) const {
    if (!a.ssq) return 1.0f;
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < SK_SSQ_MAX / 4; ++i) {
      t += v[i][0]; t += v[i][1]; t += v[i][2]; t += v[i][3];
    }
    return 1.0f / sqrtf(t / (float)a.K + a.eps);
  }
};

// Epilogue for four consecutive features f..f+3 of token m.  SwiGLU: r is
// the deferred norm's 1/rms of the token (1 without one).
template <int DT, int EPI>
__device__ __forceinline__ void sk_store4(const ProjArgs& a, int m, int f, const float* v,
                                          const float* up, float r = 1.0f) {
  typedef typename Elt<DT>::T T;
  if constexpr (EPI == EPI_LOGITS) {
    float* y = reinterpret_cast<float*>(a.y) + (size_t)m * a.N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (f + i < a.N) y[f + i] = v[i];
  } else if constexpr (EPI == EPI_RESID) {
    const T* r = reinterpret_cast<const T*>(a.resid) + (size_t)m * a.N + f;
    float rv[4];
    load4<DT>(r, rv);
    T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
    store4<DT>(y, rv[0] + v[0], rv[1] + v[1], rv[2] + v[2], rv[3] + v[3]);
  } else if constexpr (EPI == EPI_SWIGLU) {
    T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
    store4<DT>(y, silu(r * v[0]) * (r * up[0]), silu(r * v[1]) * (r * up[1]),
               silu(r * v[2]) * (r * up[2]), silu(r * v[3]) * (r * up[3]));
  } else {
    float w[4] = {v[0], v[1], v[2], v[3]};
    qkv_epilogue4<DT>(a, a.tok0 + m, m, f, w);
  }
}

// Stage geometry for BK (k per stage: 64, 128 or 256) and NST stages in LDS.  A
// row slice is BK*2 bytes = CPR 16-byte chunks; one global_load_lds (64 lanes
// x 16 bytes) fills RPI whole row slices, so a stage takes NI instructions,
// NIW per wave.  Chunk c of row r sits at physical chunk c ^ (r & 15): the 16
// rows that one ds_read_b128 cycle serves then land in 16 distinct 4-bank
// groups.
template <int BK, int NST, int NW, int BM>
struct SkGeom {
  static_assert(BK == 64 || BK == 128 || BK == 256, "stage width");
  static_assert(NW == 4 || NW == 8, "waves");
  static constexpr int ROWB = BK * 2;
  static constexpr int CPR = ROWB / 16;
  static constexpr int RPI = 64 / CPR;
  static constexpr int NI = (BM + SK_BN) / RPI;
  static constexpr int NIW = NI / NW;
  static constexpr int NIW_W = (BM / RPI) / NW;    // weight instructions per wave
  static constexpr int STAGE = (BM + SK_BN) * ROWB;
  static constexpr int RB = BM / 32;               // row blocks
  static constexpr int KSL = NW / RB;              // k slices of a stage
  static constexpr int KS2 = BK / 16 / KSL;        // 32x32x16 k-steps per wave per stage
  static_assert(NI % NW == 0 && (BM / RPI) % NW == 0 && NW % RB == 0, "work split");
  static constexpr int LDS = NST * STAGE;
  static_assert(NIW * (NST - 2) < 64, "vmcnt range");
  // Physical chunk = logical chunk ^ swz(row).  128-byte slices put two rows
  // in one 256-byte bank line, hence the shifted form for BK = 64.
  static __device__ __forceinline__ int swz(int r) { return CPR >= 16 ? (r & 15) : ((r >> 1) & 7); }
};

template <int DT, int EPI, bool SPLIT, int BK, int NST, int BM>
__global__ __launch_bounds__(SK_NW * 64) void gemv_dma_kernel(ProjArgs a, float* part, int kchunk,
                                                              int nsplit) {
  typedef typename Elt<DT>::T T;
  typedef SkGeom<BK, NST, SK_NW, BM> G;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int FB = SWI ? BM / 2 : BM;  // features per workgroup
  // One LDS object: the stage ring, reused at the end for the cross-wave sums.
  // (A second LDS variable gives the accesses alias scopes, and the wait-count
  // pass then waits for every outstanding DMA before each fragment read.)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[G::LDS];
  f32x16* red = reinterpret_cast<f32x16*>(lds);  // [KSL - 1][2][64] after the k loop

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K;
  // Grid x enumerates (row block, K split) with the split fastest, so the
  // workgroups resident together cover neighbouring K ranges of the same rows.
  const int blk = blockIdx.x / nsplit, ks = blockIdx.x - blk * nsplit;
  const int f0 = blk * FB;
  const int k0 = ks * kchunk;
  const int klen = min(K, k0 + kchunk) - k0;  // a multiple of 64
  const int nkt = (klen + BK - 1) / BK;

  // DMA: instruction i of a stage fills stage rows RPI*i .. RPI*i + RPI-1
  // (rows 0..BM-1 weights, then the 32 token slots); wave w issues i = w + NW j.  Lane
  // l: row RPI*i + l/CPR, physical chunk l%CPR, logical chunk phys ^ (row&15).
  // A chunk past the end of the K range (last stage of a range that is not a
  // multiple of BK) re-reads the range's first chunk instead; the k-steps that
  // would use it are skipped, and every wave still issues the same number of
  // loads per stage, which the wait counts rely on.
  const T* src[G::NIW];
  int kofs[G::NIW];
#pragma unroll
  for (int j = 0; j < G::NIW; ++j) {
    const int i = wave + SK_NW * j;
    const int r = G::RPI * i + lane / G::CPR;
    const int c = (lane % G::CPR) ^ G::swz(r);
    const T* row;
    if (r < BM) {
      if constexpr (SWI) {
        const int f = f0 + (r < FB ? r : r - FB);
        row = reinterpret_cast<const T*>(r < FB ? a.w[0] : a.w[1]) + (size_t)(f < a.N ? f : 0) * K;
      } else {
        const int f = f0 + r;
        row = seg_row<T>(a, f < a.N ? f : 0);
      }
    } else {
      const int m = r - BM;
      row = reinterpret_cast<const T*>(a.x) + (size_t)(m < a.M ? m : 0) * K;
    }
    src[j] = row + k0;
    kofs[j] = c * 8;
  }
  // Without a K split, workgroup blk walks the stages of K starting at stage
  // blk mod nkt and wraps around (when K is whole stages).  Otherwise every
  // resident workgroup reads the same 512-byte slot of its 16 KB rows at the
  // same moment: 70B gate/up at 32 tokens 167.6 -> 151.5 us.  Split launches
  // already put neighbouring workgroups on different K ranges.
  const int rot = (nsplit == 1 && klen % BK == 0) ? blk % nkt : 0;
  auto issue = [&](int st, int kt) {
    uint8_t* base = lds + st * G::STAGE;
    const int kr = kt + rot < nkt ? kt + rot : kt + rot - nkt;
    const int k = kr * BK;
#pragma unroll
    for (int j = 0; j < G::NIW; ++j) {
      const int kk = k + kofs[j];
      const T* g = src[j] + (kk < klen ? kk : 0);
      uint8_t* d = base + (wave + SK_NW * j) * 1024;
      if (j < G::NIW_W) dma16_stream(g, d);  // weights: instructions 0 .. 64/RPI - 1
      else dma16(g, d);                      // activations
    }
  };
  // This wave's part of stage kt has landed once at most `newer` later stages
  // (NIW loads each) are outstanding.
  auto wait_stage = [&](int newer) {
    static_for<0, NST - 1>([&](auto n) {
      if (newer == decltype(n)::value) wait_vmcnt<decltype(n)::value * G::NIW>();
    });
  };

  // Fragments: wave w multiplies row block rb = w % RB over the k-steps
  // kh*KS2 .. kh*KS2 + KS2-1 (k slice kh = w / RB) of every stage.
  const int rb = wave % G::RB, kh = wave / G::RB;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int swz = G::swz(l32);  // rows rb*32 + l32 and token row 64 + l32 share it
  const int aoff = (rb * 32 + l32) * G::ROWB;
  const int boff = BM * G::ROWB + l32 * G::ROWB;

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < nkt) issue(st, st);
  SsqAhead ssq;  // deferred norm of a SwiGLU launch without a K split
  if constexpr (SWI && !SPLIT) ssq.load(a, l32);
  // The barrier is a bare s_barrier: a full __syncthreads would also wait for
  // the stages still in flight.  Its explicit waits: this wave's loads of stage
  // kt (vmcnt) and its reads of stage kt-1, which the MFMAs consumed.  The
  // sched_barriers keep the fragment reads below it.
  for (int kt = 0; kt < nkt; ++kt) {
    wait_stage(min(nkt - 1, kt + NST - 2) - kt);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();  // stage kt complete everywhere; stage kt-1 no longer read
    __builtin_amdgcn_sched_barrier(0);
    if (kt + NST - 1 < nkt) issue((kt + NST - 1) % NST, kt + NST - 1);
    const uint8_t* base = lds + (kt % NST) * G::STAGE;
    const int nvalid = (klen - kt * BK) / 16 - kh * G::KS2;  // k-steps of this wave with data
    if (nvalid >= G::KS2) {
      u32x4 fa[G::KS2], fb[G::KS2];
#pragma unroll
      for (int t = 0; t < G::KS2; ++t) {
        const int ch = ((2 * (kh * G::KS2 + t) + h2) ^ swz) * 16;
        fa[t] = ld16(base + aoff + ch);
        fb[t] = ld16(base + boff + ch);
      }
#pragma unroll
      for (int t = 0; t < G::KS2; ++t) acc = mfma32<DT>(fa[t], fb[t], acc);
    } else {
      for (int t = 0; t < nvalid; ++t) {
        const int ch = ((2 * (kh * G::KS2 + t) + h2) ^ swz) * 16;
        acc = mfma32<DT>(ld16(base + aoff + ch), ld16(base + boff + ch), acc);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // k slices meet: the waves of slices 1.. hand their sums to those of slice 0
  // (once every wave is done with the last stage, whose buffer may be the one
  // reused).
  __syncthreads();
  if (kh > 0) red[((kh - 1) * G::RB + rb) * 64 + lane] = acc;
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int q = 0; q < G::KSL - 1; ++q) acc += red[(q * G::RB + rb) * 64 + lane];
  }
  if constexpr (!SPLIT && SWI) {
    // Gate rows are in row blocks 0 .. RB/2 - 1, the matching up rows RB/2 later.
    __syncthreads();
    if (kh == 0 && rb >= G::RB / 2) red[(rb - G::RB / 2) * 64 + lane] = acc;
    __syncthreads();
    if (rb >= G::RB / 2) return;
  }
  if (kh > 0) return;

  // Lane holds token l32 and rows rb*32 + g*8 + h2*4 + 0..3, g = 0..3.
  const int m = l32;
  if constexpr (SPLIT) {
    if (m < a.M) {
      const int nrows = SWI ? 2 * a.N : a.N;
      float* p = part + ((size_t)ks * a.M + m) * nrows;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = rb * 32 + g * 8 + h2 * 4;
        const int f = SWI ? (r < FB ? f0 + r : a.N + f0 + r - FB) : f0 + r;
        if ((SWI ? f0 + (r < FB ? r : r - FB) : f) < a.N) {
          f32x4 v = {acc[g * 4], acc[g * 4 + 1], acc[g * 4 + 2], acc[g * 4 + 3]};
          *reinterpret_cast<f32x4*>(p + f) = v;
        }
      }
    }
  } else if constexpr (SWI) {
    if (m >= a.M) return;
    const f32x16 up = red[rb * 64 + lane];
    const float r = ssq.rstd(a);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = f0 + rb * 32 + g * 8 + h2 * 4;
      if (f >= a.N) continue;
      float v[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = acc[g * 4 + i]; u[i] = up[g * 4 + i]; }
      sk_store4<DT, EPI>(a, m, f, v, u, r);
    }
  } else {
    if (m >= a.M) return;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = f0 + rb * 32 + g * 8 + h2 * 4;
      if (f >= a.N) continue;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc[g * 4 + i];
      sk_store4<DT, EPI>(a, m, f, v, nullptr);
    }
  }
}

// Weight-only int8 variant: rows of int8 codes (256-byte slices of a 256-k
// stage) and the token slots (512-byte slices, 16 KB) stream through LDS.
// The A fragment of a k-step is 8 codes (8 bytes),
// converted to the activation format (exact: |code| <= 127) before the MFMA;
// each row's float32 scale multiplies its sums after the k loop, so partials
// and results carry code x activation x scale as the row kernel computes.
// The 16-byte chunks of a weight slice are swizzled by (row & 15) like the
// activation slices; the 8-byte fragment reads then see 2-way bank conflicts.
// Eight waves with the stage's fragment reads issued before the conversions,
// 128 code rows per workgroup (4 row blocks x 2 k halves; 48 KB stages three
// deep, so a CU has 64 KB of codes in flight) and about one workgroup per CU
// per launch: at the 70B batch-32 decode gate/up took 153 us with four waves,
// 64 rows and the k-steps one after another, 143 us with the reads batched,
// 127 us with eight waves (sixteen: the same), 106 us with 128 rows and no K
// split (the step 381 -> 301 us).
constexpr int W8_BK = 256;
constexpr int W8_NW = 8;                         // waves per workgroup

// Geometry for BMW code rows per workgroup: RB row blocks of 32 x KSL k
// slices of each stage over the eight waves; NST stages of codes (BMW x 256
// bytes) and token slots (32 x 512 bytes).
template <int BMW>
struct W8Geom {
  static_assert(BMW == 64 || BMW == 128, "rows per workgroup");
  static constexpr int RB = BMW / 32;
  static constexpr int KSL = W8_NW / RB;
  static constexpr int KS2 = W8_BK / 16 / KSL;   // k-steps per wave and stage
  static constexpr int NST = BMW == 64 ? 4 : 3;
  static constexpr int WBYTES = BMW * W8_BK;
  static constexpr int ABYTES = SK_BN * W8_BK * 2;
  static constexpr int STAGE = WBYTES + ABYTES;
  static constexpr int NIW = STAGE / 1024 / W8_NW;    // DMA instructions per wave and stage
  static constexpr int NIW_W = WBYTES / 1024 / W8_NW;  // of them codes
  static constexpr int LDS = NST * STAGE;
  static_assert((KSL - 1) * RB * 64 * 64 <= LDS, "the k-slice sums reuse the ring");
};

// Scale of row r of the workgroup's block (SwiGLU: gate rows, then up rows).
__device__ __forceinline__ float w8_row_scale(const ProjArgs& a, int half, bool swi, int f0,
                                              int r) {
  if (swi) {
    const int f = f0 + (r < half ? r : r - half);
    return a.wscale[r < half ? 0 : 1][f < a.N ? f : 0];
  }
  int f = f0 + r;
  f = f < a.N ? f : 0;
  return f < a.seg1 ? a.wscale[0][f] : f < a.seg2 ? a.wscale[1][f - a.seg1] : a.wscale[2][f - a.seg2];
}

template <int DT, int EPI, bool SPLIT, int BMW>
__global__ __launch_bounds__(W8_NW * 64) void gemv_dma_w8_kernel(ProjArgs a, float* part,
                                                                  int kchunk, int nsplit) {
  typedef typename Elt<DT>::T T;
  typedef W8Geom<BMW> G;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int HALF = BMW / 2;
  constexpr int FB = SWI ? HALF : BMW;  // features per workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t lds[G::LDS];
  f32x16* red = reinterpret_cast<f32x16*>(lds);  // [KSL-1][RB][64] after the k loop

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K;
  const int blk = blockIdx.x / nsplit, ks = blockIdx.x - blk * nsplit;
  const int f0 = blk * FB;
  const int k0 = ks * kchunk;
  const int klen = min(K, k0 + kchunk) - k0;  // a multiple of 64
  const int nkt = (klen + W8_BK - 1) / W8_BK;

  // DMA: wave w issues instructions i = w + 8j.  i < BMW/4: code rows 4i + l/16,
  // physical chunk l%16 (16 codes); else token rows 2(i - BMW/4) + l/32,
  // physical chunk l%32 (8 elements).  Logical chunk = physical ^ (row & 15).
  // Chunks past the K range re-read the range's first one (their k-steps are
  // skipped), so every wave issues the same number of loads per stage.
  const uint8_t* src[G::NIW];
  int kofs[G::NIW];  // element (= byte for codes) offset of the chunk in a stage
  int esz[G::NIW];
#pragma unroll
  for (int j = 0; j < G::NIW; ++j) {
    const int i = wave + W8_NW * j;
    if (j < G::NIW_W) {
      const int r = 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      const int8_t* row;
      if constexpr (SWI) {
        const int f = f0 + (r < HALF ? r : r - HALF);
        row = reinterpret_cast<const int8_t*>(r < HALF ? a.w[0] : a.w[1]) + (size_t)(f < a.N ? f : 0) * K;
      } else {
        const int f = f0 + r;
        row = seg_row<int8_t>(a, f < a.N ? f : 0);
      }
      src[j] = reinterpret_cast<const uint8_t*>(row + k0);
      kofs[j] = c * 16;
      esz[j] = 1;
    } else {
      const int m = 2 * (i - BMW / 4) + (lane >> 5);
      const int c = (lane & 31) ^ (m & 15);
      const T* row = reinterpret_cast<const T*>(a.x) + (size_t)(m < a.M ? m : 0) * K;
      src[j] = reinterpret_cast<const uint8_t*>(row + k0);
      kofs[j] = c * 8;
      esz[j] = 2;
    }
  }
  // Stages in rotated order without a K split, as in the 16-bit kernel.
  const int rot = (nsplit == 1 && klen % W8_BK == 0) ? blk % nkt : 0;
  auto issue = [&](int st, int kt) {
    uint8_t* base = lds + st * G::STAGE;
    const int kr = kt + rot < nkt ? kt + rot : kt + rot - nkt;
    const int k = kr * W8_BK;
#pragma unroll
    for (int j = 0; j < G::NIW; ++j) {
      const int kk = k + kofs[j];
      const uint8_t* g = src[j] + (size_t)(kk < klen ? kk : 0) * esz[j];
      uint8_t* d = base + (wave + W8_NW * j) * 1024;
      if (j < G::NIW_W) dma16_stream(g, d);
      else dma16(g, d);
    }
  };
  auto wait_stage = [&](int newer) {
    static_for<0, G::NST - 1>([&](auto n) {
      if (newer == decltype(n)::value) wait_vmcnt<decltype(n)::value * G::NIW>();
    });
  };

  const int rb = wave % G::RB, kh = wave / G::RB;  // row block, k slice of each stage
  const int l32 = lane & 31, h2 = lane >> 5;
  const int swz = l32 & 15;
  const int aoff = (rb * 32 + l32) * W8_BK + 8 * h2;
  const int boff = G::WBYTES + l32 * W8_BK * 2;

  // 8 codes -> one fragment in the activation format.
  auto to_frag = [&](u32x2 raw) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * i + b] = (float)(int8_t)(raw[i] >> (8 * b));
    return pack16<DT>(f);
  };

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int st = 0; st < G::NST - 1; ++st)
    if (st < nkt) issue(st, st);
  SsqAhead ssq;  // deferred norm of a SwiGLU launch without a K split
  if constexpr (SWI && !SPLIT) ssq.load(a, l32);
  for (int kt = 0; kt < nkt; ++kt) {
    wait_stage(min(nkt - 1, kt + G::NST - 2) - kt);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (kt + G::NST - 1 < nkt) issue((kt + G::NST - 1) % G::NST, kt + G::NST - 1);
    const uint8_t* base = lds + (kt % G::NST) * G::STAGE;
    const int nvalid = (klen - kt * W8_BK) / 16 - kh * G::KS2;
    if (nvalid >= G::KS2) {
      // Every fragment read of the stage first, then conversions and MFMAs.
      u32x2 raw[G::KS2];
      u32x4 bfr[G::KS2];
#pragma unroll
      for (int t = 0; t < G::KS2; ++t) {
        const int ks16 = kh * G::KS2 + t;  // k-step: k = 16 ks16 .. +15
        raw[t] = *reinterpret_cast<const u32x2*>(base + aoff + ((ks16 ^ swz) << 4));
        bfr[t] = ld16(base + boff + (((2 * ks16 + h2) ^ swz) << 4));
      }
#pragma unroll
      for (int t = 0; t < G::KS2; ++t) acc = mfma32<DT>(to_frag(raw[t]), bfr[t], acc);
    } else {
      for (int t = 0; t < nvalid; ++t) {
        const int ks16 = kh * G::KS2 + t;
        const u32x2 r = *reinterpret_cast<const u32x2*>(base + aoff + ((ks16 ^ swz) << 4));
        const u32x4 b = ld16(base + boff + (((2 * ks16 + h2) ^ swz) << 4));
        acc = mfma32<DT>(to_frag(r), b, acc);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // k slices meet: waves with kh > 0 hand their sums to the kh = 0 waves,
  // which apply the row scales (lane: rows rb*32 + g*8 + h2*4 + i).  Every
  // wave passes every barrier before any returns.
  __syncthreads();
  if (kh > 0) red[((kh - 1) * G::RB + rb) * 64 + lane] = acc;
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int q = 0; q < G::KSL - 1; ++q) acc += red[(q * G::RB + rb) * 64 + lane];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[g * 4 + i] *= w8_row_scale(a, HALF, SWI, f0, rb * 32 + g * 8 + h2 * 4 + i);
  }
  if constexpr (!SPLIT && SWI) {
    // Gate rows are in row blocks 0 .. RB/2 - 1, the matching up rows RB/2 later.
    __syncthreads();  // every read of red is done
    if (kh == 0 && rb >= G::RB / 2) red[(rb - G::RB / 2) * 64 + lane] = acc;
    __syncthreads();
    if (rb >= G::RB / 2) return;
  }
  if (kh > 0) return;

  const int m = l32;
  if constexpr (SPLIT) {
    if (m < a.M) {
      const int nrows = SWI ? 2 * a.N : a.N;
      float* p = part + ((size_t)ks * a.M + m) * nrows;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = rb * 32 + g * 8 + h2 * 4;
        const int f = SWI ? (r < HALF ? f0 + r : a.N + f0 + r - HALF) : f0 + r;
        if ((SWI ? f0 + (r < HALF ? r : r - HALF) : f) < a.N) {
          f32x4 v = {acc[g * 4], acc[g * 4 + 1], acc[g * 4 + 2], acc[g * 4 + 3]};
          *reinterpret_cast<f32x4*>(p + f) = v;
        }
      }
    }
  } else if constexpr (SWI) {
    if (m >= a.M) return;
    const f32x16 up = red[rb * 64 + lane];
    const float r = ssq.rstd(a);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = f0 + rb * 32 + g * 8 + h2 * 4;
      if (f >= a.N) continue;
      float v[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = acc[g * 4 + i]; u[i] = up[g * 4 + i]; }
      sk_store4<DT, EPI>(a, m, f, v, u, r);
    }
  } else {
    if (m >= a.M) return;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = f0 + rb * 32 + g * 8 + h2 * 4;
      if (f >= a.N) continue;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc[g * 4 + i];
      sk_store4<DT, EPI>(a, m, f, v, nullptr);
    }
  }
}

// Sum of the K-split partials and the epilogue; one thread per (token, 4 features).
// With a.nout (EPI_RESID, N % 1024 == 0, so a workgroup is 1024 features of
// one token): y as stored, y * ngamma into nout, and the workgroup's sum of
// the stored y^2 into its slot of a.ssq.
template <int DT, int EPI>
__global__ __launch_bounds__(256) void gemv_split_reduce_kernel(ProjArgs a, const float* part,
                                                                int nsplit) {
  typedef typename Elt<DT>::T T;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  const int nf4 = (a.N + 3) / 4;
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id >= nf4 * a.M) return;
  const int m = id / nf4, f = (id - m * nf4) * 4;
  const int nrows = SWI ? 2 * a.N : a.N;
  f32x4 v = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float* p = part + ((size_t)s * a.M + m) * nrows;
    v += *reinterpret_cast<const f32x4*>(p + f);
    if constexpr (SWI) u += *reinterpret_cast<const f32x4*>(p + a.N + f);
  }
  float vv[4] = {v[0], v[1], v[2], v[3]}, uu[4] = {u[0], u[1], u[2], u[3]};
  if constexpr (SWI) {
    sk_store4<DT, EPI>(a, m, f, vv, uu, a.ssq ? sk_rstd(a, m) : 1.0f);
    return;
  }
  if constexpr (EPI == EPI_RESID) {
    if (a.nout) {
      float rv[4], yv[4], gv[4];
      load4<DT>(reinterpret_cast<const T*>(a.resid) + (size_t)m * a.N + f, rv);
      const u32x2 yp = {pack2<DT>(rv[0] + vv[0], rv[1] + vv[1]),
                        pack2<DT>(rv[2] + vv[2], rv[3] + vv[3])};
      *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f) = yp;
      // The stored values: what a norm pass would read.
      yv[0] = Elt<DT>::to_f32(yp[0] & 0xffffu);
      yv[1] = Elt<DT>::to_f32(yp[0] >> 16);
      yv[2] = Elt<DT>::to_f32(yp[1] & 0xffffu);
      yv[3] = Elt<DT>::to_f32(yp[1] >> 16);
      load4<DT>(reinterpret_cast<const T*>(a.ngamma) + f, gv);
      store4<DT>(reinterpret_cast<T*>(a.nout) + (size_t)m * a.N + f, yv[0] * gv[0],
                 yv[1] * gv[1], yv[2] * gv[2], yv[3] * gv[3]);
      float ss = yv[0] * yv[0] + yv[1] * yv[1] + yv[2] * yv[2] + yv[3] * yv[3];
      ss = wave_sum(ss);
      __shared__ float wsum[4];
      if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
      __syncthreads();
      float* slots = a.ssq + (size_t)m * SK_SSQ_MAX;
      if (threadIdx.x == 0) slots[f >> 10] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
      // The token's first workgroup zeroes the unused slots.
      if (f < 1024 && threadIdx.x >= a.ssq_parts && threadIdx.x < SK_SSQ_MAX)
        slots[threadIdx.x] = 0.f;
      return;
    }
  }
  sk_store4<DT, EPI>(a, m, f, vv, uu);
}

size_t gemv_dma_partial_floats(int epi, int N, int K, int M) {
  if (K % 64 != 0 || M < 1 || M > SK_BN) return 0;
  int kchunk;
  // Room for the splits of the 16-bit kernel and of the int8 one.
  const int ns = std::max(sk_split(epi, N, K, &kchunk),
                          sk_split_f(w8_features(epi), N, K, &kchunk, W8_TARGET_WG));
  return ns > 1 ? (size_t)ns * M * sk_rows(epi, N) : 0;
}

bool gemv_dma_supported(int dt, int M, int K, int N) {
  return dt != DT_F32 && M >= 1 && M <= SK_BN && K % 64 == 0 && N % 4 == 0;
}

int gemv_dma_norm_parts(int dt, bool w8, int M, int N_o, int K_o, int I) {
  if (dt != DT_BF16 || M <= 4 || N_o % 1024 != 0 || N_o / 1024 > SK_SSQ_MAX) return 0;
  if (!gemv_dma_supported(dt, M, K_o, N_o) || !gemv_dma_supported(dt, M, N_o, I)) return 0;
  if (!w8 && sk_wide(EPI_RESID, N_o, K_o)) return 0;  // no split, no reduction
  int kchunk;
  const int ns = w8 ? sk_split_f(w8_features(EPI_RESID), N_o, K_o, &kchunk, W8_TARGET_WG)
                    : sk_split(EPI_RESID, N_o, K_o, &kchunk);
  return ns > 1 ? N_o / 1024 : 0;
}

template <int DT, int EPI>
static hipError_t gemv_dma_epi(const ProjArgs& a, hipStream_t s) {
  if (sk_wide(EPI, a.N, a.K)) {
    const int nblk = (a.N + sk_features(EPI, SK_BM_W) - 1) / sk_features(EPI, SK_BM_W);
    LL_LAUNCH((gemv_dma_kernel<DT, EPI, false, SK_BK_W, SK_NST_W, SK_BM_W>), dim3(nblk),
              dim3(SK_NW * 64), 0, s, a, (float*)nullptr, a.K, 1);
    return hipGetLastError();
  }
  int kchunk;
  const int ns = sk_split(EPI, a.N, a.K, &kchunk);
  const int nblk = (a.N + sk_features(EPI) - 1) / sk_features(EPI);
  if (ns == 1) {
    LL_LAUNCH((gemv_dma_kernel<DT, EPI, false, SK_BK, SK_NST, SK_BM>), dim3(nblk), dim3(SK_NW * 64),
              0, s, a, (float*)nullptr, kchunk, 1);
    return hipGetLastError();
  }
  if (!a.part) return hipErrorInvalidValue;
  LL_LAUNCH((gemv_dma_kernel<DT, EPI, true, SK_BK, SK_NST, SK_BM>), dim3(nblk * ns), dim3(SK_NW * 64),
            0, s, a, a.part, kchunk, ns);
  const int n = ((a.N + 3) / 4) * a.M;
  LL_LAUNCH((gemv_split_reduce_kernel<DT, EPI>), dim3((n + 255) / 256), dim3(256), 0, s, a,
            (const float*)a.part, ns);
  return hipGetLastError();
}


template <int DT, int EPI>
static hipError_t gemv_dma_w8_epi(const ProjArgs& a, hipStream_t s) {
  int kchunk;
  const int ns = sk_split_f(w8_features(EPI), a.N, a.K, &kchunk, W8_TARGET_WG);
  const int nblk = (a.N + w8_features(EPI) - 1) / w8_features(EPI);
  if (ns == 1) {
    LL_LAUNCH((gemv_dma_w8_kernel<DT, EPI, false, W8_BMW>), dim3(nblk), dim3(W8_NW * 64), 0, s, a,
              (float*)nullptr, kchunk, 1);
    return hipGetLastError();
  }
  if (!a.part) return hipErrorInvalidValue;
  LL_LAUNCH((gemv_dma_w8_kernel<DT, EPI, true, W8_BMW>), dim3(nblk * ns), dim3(W8_NW * 64), 0, s,
            a, a.part, kchunk, ns);
  const int n = ((a.N + 3) / 4) * a.M;
  LL_LAUNCH((gemv_split_reduce_kernel<DT, EPI>), dim3((n + 255) / 256), dim3(256), 0, s, a,
            (const float*)a.part, ns);
  return hipGetLastError();
}

hipError_t launch_gemv_dma_w8(int dt, int epi, const ProjArgs& a, hipStream_t s) {
  if (!gemv_dma_supported(dt, a.M, a.K, a.N) || a.gamma || !a.wscale[0]) return hipErrorInvalidValue;
  if (dt == DT_BF16) {
    switch (epi) {
      case EPI_QKV: return gemv_dma_w8_epi<DT_BF16, EPI_QKV>(a, s);
      case EPI_RESID: return gemv_dma_w8_epi<DT_BF16, EPI_RESID>(a, s);
      case EPI_SWIGLU: return gemv_dma_w8_epi<DT_BF16, EPI_SWIGLU>(a, s);
    }
  } else if (dt == DT_F16) {
    switch (epi) {
      case EPI_QKV: return gemv_dma_w8_epi<DT_F16, EPI_QKV>(a, s);
      case EPI_RESID: return gemv_dma_w8_epi<DT_F16, EPI_RESID>(a, s);
      case EPI_SWIGLU: return gemv_dma_w8_epi<DT_F16, EPI_SWIGLU>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int DT>
static hipError_t gemv_dma_dt(int epi, const ProjArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_QKV: return gemv_dma_epi<DT, EPI_QKV>(a, s);
    case EPI_RESID: return gemv_dma_epi<DT, EPI_RESID>(a, s);
    case EPI_SWIGLU: return gemv_dma_epi<DT, EPI_SWIGLU>(a, s);
    case EPI_LOGITS: return gemv_dma_epi<DT, EPI_LOGITS>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_dma(int dt, int epi, const ProjArgs& a, hipStream_t s) {
  if (!gemv_dma_supported(dt, a.M, a.K, a.N) || a.gamma) return hipErrorInvalidValue;
  if (dt == DT_BF16) return gemv_dma_dt<DT_BF16>(epi, a, s);
  if (dt == DT_F16) return gemv_dma_dt<DT_F16>(epi, a, s);
  return hipErrorInvalidValue;
}

}  // namespace ll
