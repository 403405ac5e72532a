// Decode-sized projections: y[m, n] = sum_k act(x)[m, k] W[n, k] for up to 32
// tokens m, streaming every weight byte once from HBM.
//
// Weights sit on the MFMA "A" side (16 output features per tile) and tokens on
// the "B" side (16 per tile, padded with zeros), so the k-reduction is done by
// v_mfma_f32_16x16x32_{bf16,f16} (or four 16x16x4_f32 for float32) instead of
// cross-lane shuffles.  Lane l of a wave reads 64 contiguous bytes of weight
// row l%16 per k-block; the four lane groups l/16 cover 256 contiguous bytes,
// so each row segment is fetched whole.  The waves of a workgroup split K and
// meet in LDS.  Weight blocks stream through a register ring PF blocks ahead
// of the one being multiplied, so every wave keeps (PF+1) x 4 KB in flight.
//
// Four variants:
//  * gemv_row1 (1-4 tokens): each wave streams one row over the full K; see below.
//  * gemv_piece (one token, K a multiple of 2048: O, down, and QKV with its
//    norm): workgroups walk the matrix in 32 KB pieces of whole rows; see below.
//  * gemv_lds: the activations of the M tokens (M*K*size <= 48 KB) are staged
//    once per workgroup in LDS.  With a fused RMSNorm the staging pass also
//    multiplies by the gain and accumulates sum x^2, so 1/rms is known before
//    the weight loop and scales the results in the epilogue.
//  * gemv_glb: larger token counts; activation chunks come from global memory
//    (L2) one block ahead of use.  A fused norm is not available here: the
//    host normalises first.
// For 16-bit formats without a fused norm, the LDS-streaming kernel of
// gemv_dma.hip takes every case the row kernel does not.
// Epilogues: RoPE + KV-cache append (QKV), residual add (O, down), SwiGLU
// (gate/up, two weight matrices) or float32 logits (LM head).
#include "common.cuh"
#include "epilogue.cuh"

namespace ll {

constexpr int GEMV_LDS_BYTES = 48 * 1024;  // + static LDS stays within 64 KB
// For a single token the row kernel stages up to 64 KB of activations
// (dynamic LDS past 48 KB is enabled per kernel), so its 28672-wide down
// projection (56 KB) streams every row in one pass: no K split and no
// partial-sum launch (70B: 80.8 -> 76.9 us against the split streaming kernel
// plus its reduction).
constexpr int GEMV_ROW_LDS_BYTES = 64 * 1024;

// Cross-wave reduction of the accumulators and the epilogue (wave 0).
template <int DT, int EPI, int NA, int CT, int NW>
__device__ __forceinline__ void gemv_finish(const ProjArgs& a, f32x4 (&acc)[NA][CT],
                                            const float* scale_tok, int row0) {
  typedef typename Elt<DT>::T T;
  __shared__ f32x4 red[NW > 1 ? NW - 1 : 1][NA * CT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
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

  // Lane holds token r16 (+16 ct), features row0 + kg*4 + 0..3.
  const int f = row0 + kg * 4;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int m = ct * 16 + r16;
    if (m >= a.M) continue;
    const float scale = scale_tok ? scale_tok[m] : 1.f;
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
        for (int i = 0; i < 4; ++i) o[i] = silu(v[i]) * (acc[NA - 1][ct][i] * scale);
        T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
        store4<DT>(y, o[0], o[1], o[2], o[3]);
      } else {  // EPI_QKV
        qkv_epilogue4<DT>(a, a.tok0 + m, m, f, v);
      }
    }
  }
}

// Fused RMSNorm, f16: the staging pass stored the raw rows and the sums of
// squares; this second pass over LDS turns each into x * rstd * gain (the
// separate norm pass's arithmetic).  Staging x * gain and applying rstd after
// the dot products, as the 32-bit and bf16 paths do, could overflow f16's
// range (65504) where the normalised value cannot: |x * rstd| <= sqrt(K).
// Each thread rewrites the chunks it staged, so only the rstd needs a barrier.
template <int DT>
__device__ __forceinline__ void stage_prescaled(typename Elt<DT>::T* xs,
                                                const typename Elt<DT>::T* gg,
                                                const float* rstd_s, int M, int K, int tid,
                                                int nthreads) {
  constexpr int E = Elt<DT>::PER16;
  const int KC = K / E;
  for (int m = 0; m < M; ++m) {
    const float r = rstd_s[m];
    for (int c = tid; c < KC; c += nthreads) {
      float xf[E], gf[E];
      unpack16<DT>(ld16(xs + (size_t)m * K + c * E), xf);
      unpack16<DT>(ld16(gg + c * E), gf);
#pragma unroll
      for (int e = 0; e < E; ++e) xf[e] = xf[e] * r * gf[e];
      st16(xs + (size_t)m * K + c * E, pack16<DT>(xf));
    }
  }
}

// Weight row pointers of this lane (rows past N read row 0; dropped later).
template <int DT, int EPI, int NA>
__device__ __forceinline__ void gemv_rows(const ProjArgs& a, int row0,
                                          const typename Elt<DT>::T* (&wp)[NA]) {
  typedef typename Elt<DT>::T T;
  const int f_lane = row0 + (threadIdx.x & 15);
  const int f_safe = f_lane < a.N ? f_lane : 0;
  if constexpr (EPI == EPI_SWIGLU) {
    wp[0] = reinterpret_cast<const T*>(a.w[0]) + (size_t)f_safe * a.K;
    wp[NA - 1] = reinterpret_cast<const T*>(a.w[1]) + (size_t)f_safe * a.K;
  } else {
    wp[0] = seg_row<T>(a, f_safe);
  }
}

template <int DT, int EPI, bool NORM, int NW, int PF>
__global__ __launch_bounds__(NW * 64) void gemv_lds_kernel(ProjArgs a) {
  typedef typename Elt<DT>::T T;
  constexpr int E = Elt<DT>::PER16;   // elements per 16-byte chunk
  constexpr int KB = 16 * E;          // k per block: 4 lane groups x 4 chunks
  constexpr int NA = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int NS = PF + 1;          // ring slots
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  T* xs = reinterpret_cast<T*>(smem);  // [M][K]
  __shared__ float rstd_s[16];
  __shared__ float part_s[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int K = a.K, M = a.M;
  const int row0 = blockIdx.x * 16;

  const T* wp[NA];
  gemv_rows<DT, EPI, NA>(a, row0, wp);
  const int nkb = (K + KB - 1) / KB;
  const int kb0 = (nkb * wave) / NW;
  const int kb1 = (nkb * (wave + 1)) / NW;

  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 wa[NS][NA][4];
  auto load_w = [&](auto slot, int kb) {
    constexpr int S = decltype(slot)::value;
    const int kbase = kb * KB + kg * 4 * E;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kbase + s * E;
#pragma unroll
      for (int n = 0; n < NA; ++n) wa[S][n][s] = (k < K) ? ld16(wp[n] + k) : zero;
    }
  };
  // Start the weight stream before staging the activations.
  if (kb0 < kb1) load_w(ic<0>{}, kb0);
  if constexpr (PF >= 2) {
    if (kb0 + 1 < kb1) load_w(ic<1>{}, kb0 + 1);
  }

  // Stage activations (times the gain when the norm is fused; f16 stages the
  // normalised rows instead, see stage_prescaled).
  constexpr bool PRE = NORM && DT == DT_F16;
  const int KC = K / E;
  const T* xg = reinterpret_cast<const T*>(a.x);
  const T* gg = reinterpret_cast<const T*>(a.gamma);
  for (int m = 0; m < M; ++m) {
    float ss = 0.f;
    for (int c = tid; c < KC; c += NW * 64) {
      u32x4 xv = ld16(xg + (size_t)m * K + c * E);
      if constexpr (NORM) {
        float xf[E], gf[E];
        unpack16<DT>(xv, xf);
        if constexpr (!PRE) unpack16<DT>(ld16(gg + c * E), gf);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          ss += xf[e] * xf[e];
          if constexpr (!PRE) xf[e] *= gf[e];
        }
        if constexpr (!PRE) xv = pack16<DT>(xf);
      }
      st16(xs + (size_t)m * K + c * E, xv);
    }
    if constexpr (NORM) {
      ss = wave_sum(ss);
      if (lane == 0) part_s[wave] = ss;
      __syncthreads();
      if (tid == 0) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += part_s[w];
        rstd_s[m] = 1.0f / sqrtf(t / (float)K + a.eps);
      }
      __syncthreads();
    }
  }
  if constexpr (PRE) stage_prescaled<DT>(xs, gg, rstd_s, M, K, tid, NW * 64);
  __syncthreads();

  f32x4 acc[NA][1];
#pragma unroll
  for (int n = 0; n < NA; ++n) acc[n][0] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool tv = r16 < M;
  const T* xl = xs + (size_t)(tv ? r16 : 0) * K;

  auto step = [&](auto slot, int kb) {
    constexpr int S = decltype(slot)::value;
    if (kb + PF < kb1) load_w(ic<(S + PF) % NS>{}, kb + PF);
    const int kbase = kb * KB + kg * 4 * E;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kbase + s * E;
      const u32x4 xv = (tv && k < K) ? ld16(xl + k) : zero;
#pragma unroll
      for (int n = 0; n < NA; ++n) acc[n][0] = mfma16_chunk<DT>(wa[S][n][s], xv, acc[n][0]);
    }
  };
  for (int kb = kb0; kb < kb1; kb += NS) {
    step(ic<0>{}, kb);
    if (kb + 1 < kb1) step(ic<1 % NS>{}, kb + 1);
    if constexpr (NS > 2) {
      if (kb + 2 < kb1) step(ic<2 % NS>{}, kb + 2);
    }
  }
  gemv_finish<DT, EPI, NA, 1, NW>(a, acc, (NORM && !PRE) ? rstd_s : nullptr, row0);
}

template <int DT, int EPI, int CT, int NW, int PF>
__global__ __launch_bounds__(NW * 64) void gemv_glb_kernel(ProjArgs a) {
  typedef typename Elt<DT>::T T;
  constexpr int E = Elt<DT>::PER16;
  constexpr int KB = 16 * E;
  constexpr int NA = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int NS = PF + 1;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int K = a.K;
  const int row0 = blockIdx.x * 16;
  const T* wp[NA];
  gemv_rows<DT, EPI, NA>(a, row0, wp);
  const T* xp[CT];
  bool tv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int m = ct * 16 + r16;
    tv[ct] = m < a.M;
    xp[ct] = reinterpret_cast<const T*>(a.x) + (size_t)(tv[ct] ? m : 0) * K;
  }
  const int nkb = (K + KB - 1) / KB;
  const int kb0 = (nkb * wave) / NW;
  const int kb1 = (nkb * (wave + 1)) / NW;

  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 wa[NS][NA][4];
  u32x4 xa[NS][CT][4];
  auto load_w = [&](auto slot, int kb) {
    constexpr int S = decltype(slot)::value;
    const int kbase = kb * KB + kg * 4 * E;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kbase + s * E;
#pragma unroll
      for (int n = 0; n < NA; ++n) wa[S][n][s] = (k < K) ? ld16(wp[n] + k) : zero;
    }
  };
  auto load_x = [&](auto slot, int kb) {
    constexpr int S = decltype(slot)::value;
    const int kbase = kb * KB + kg * 4 * E;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kbase + s * E;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) xa[S][ct][s] = (k < K && tv[ct]) ? ld16(xp[ct] + k) : zero;
    }
  };
  if (kb0 < kb1) {
    load_x(ic<0>{}, kb0);
    load_w(ic<0>{}, kb0);
  }
  if constexpr (PF >= 2) {
    if (kb0 + 1 < kb1) load_w(ic<1>{}, kb0 + 1);
  }
  f32x4 acc[NA][CT];
#pragma unroll
  for (int n = 0; n < NA; ++n)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[n][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per step: activations of the next block, then weights PF blocks ahead
  // (issue order keeps the in-order load counter from waiting on the ring).
  auto step = [&](auto slot, int kb) {
    constexpr int S = decltype(slot)::value;
    if (kb + 1 < kb1) load_x(ic<(S + 1) % NS>{}, kb + 1);
    if (kb + PF < kb1) load_w(ic<(S + PF) % NS>{}, kb + PF);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int n = 0; n < NA; ++n)
          acc[n][ct] = mfma16_chunk<DT>(wa[S][n][s], xa[S][ct][s], acc[n][ct]);
  };
  for (int kb = kb0; kb < kb1; kb += NS) {
    step(ic<0>{}, kb);
    if (kb + 1 < kb1) step(ic<1 % NS>{}, kb + 1);
    if constexpr (NS > 2) {
      if (kb + 2 < kb1) step(ic<2 % NS>{}, kb + 2);
    }
  }
  gemv_finish<DT, EPI, NA, CT, NW>(a, acc, nullptr, blockIdx.x * 16);
}

size_t gemv_lds_bytes(int dt, int M, int K) { return (size_t)M * K * (dt == DT_F32 ? 4 : 2); }

bool gemv_fits_lds(int dt, int M, int K) {
  return M <= 16 && gemv_lds_bytes(dt, M, K) <= (size_t)GEMV_LDS_BYTES;
}

template <int DT, int EPI, bool NORM>
static hipError_t gemv_lds_launch(const ProjArgs& a, hipStream_t s) {
  const int grid = (a.N + 15) / 16;
  const size_t sh = gemv_lds_bytes(DT, a.M, a.K);
  if (grid <= 1024)  // few row tiles: split K over 8 waves
    LL_LAUNCH((gemv_lds_kernel<DT, EPI, NORM, 8, 2>), dim3(grid), dim3(512), sh, s, a);
  else
    LL_LAUNCH((gemv_lds_kernel<DT, EPI, NORM, 4, 2>), dim3(grid), dim3(256), sh, s, a);
  return hipGetLastError();
}

template <int DT, int EPI>
static hipError_t gemv_glb_launch(const ProjArgs& a, hipStream_t s) {
  const int grid = (a.N + 15) / 16;
  if (a.M <= 16)
    LL_LAUNCH((gemv_glb_kernel<DT, EPI, 1, 4, 2>), dim3(grid), dim3(256), 0, s, a);
  else
    LL_LAUNCH((gemv_glb_kernel<DT, EPI, 2, 4, 1>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One to four tokens, one weight row per wave: each wave streams a single
// contiguous row (measured on plain streaming reads: one stream per wave is
// 5-15% faster than two or four interleaved ones).  A workgroup of NWV waves
// takes NWV rows (SwiGLU: NWV/2 gate rows and the matching up rows), stages the
// activations (times the gain, with the sum of squares for a fused norm) once
// in LDS, and meets in LDS for the epilogue: RoPE pairs and the four
// consecutive features of the QKV epilogue, gate and up of SwiGLU.
// ---------------------------------------------------------------------------
// WQ: the weights are int8 codes (16 per 16-byte load) with one float32
// scale per row (a.wscale, by segment), applied after the reduction; the
// activations stay in format DT.  An int8 row is half as long in bytes, so
// each wave then streams two rows (RPW) to keep the same bytes in flight, and
// every activation chunk read from LDS serves both.  Only single-token
// launches with a fused norm (QKV, gate/up: many rows, and a norm pass per
// workgroup worth spreading over more rows) do that; O and down (4096 rows at
// 7B) keep one row per wave, or half the CUs would sit idle, and with four
// tokens the second row's registers spill.
// W4 (with WQ): 4-bit codes instead, two per byte (weight 2j in the low
// nibble of byte j), 32 per 16-byte load, sign-extended from the nibble.  A
// 4096-wide int4 row is 2 KB, so where the norm is fused each wave takes four
// rows, in batches of two 1 KB loads per row (QKV 14.2 -> 13.6 us, gate/up
// 18.6 -> 18.0 us at the 7B decode against two rows).
// W4 with bf16 activations and one token (D2) takes the products two at a
// time on v_dot2_f32_bf16: flipping a code's top bit gives q + 8 in 0..15,
// and that nibble ORed into the mantissa of bf16 128.0 is exactly 136 + q, so
// one AND-OR per pair of codes builds a bf16 pair without a conversion, and
// the row's sum is corrected by 136 * sum(x) (sum of the staged bf16 values,
// taken once per workgroup).  The mask picks the nibbles of bytes 0 and 2 (or,
// shifted, 1 and 3) of a word, i.e. codes (j, j+4), so the staging pass
// stores each chunk of eight activations in that pair order.  1.5 VALU ops per
// product instead of 3 (sign extension, conversion, FMA): 7B gate/up 19.0 ->
// 17.7 us, down 13.6 -> 12.2 us, QKV 14.1 -> 13.4 us.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
// Pairs (x0,x4),(x1,x5),(x2,x6),(x3,x7) from the chunk (x0,x1),(x2,x3),(x4,x5),(x6,x7).
__device__ __forceinline__ u32x4 pair_interleave(u32x4 d) {
  u32x4 p;
  p[0] = (d[0] & 0xffffu) | (d[2] << 16);
  p[1] = (d[0] >> 16) | (d[2] & 0xffff0000u);
  p[2] = (d[1] & 0xffffu) | (d[3] << 16);
  p[3] = (d[1] >> 16) | (d[3] & 0xffff0000u);
  return p;
}
template <bool WQ, int MT, bool NORM, bool W4 = false>
constexpr int row_rows_per_wave() { return (WQ && MT == 1 && NORM) ? (W4 ? 4 : 2) : 1; }

template <int DT, int EPI, bool NORM, int MT, int NWV, bool WQ = false, bool W4 = false>
__global__ __launch_bounds__(NWV * 64) void gemv_row1_kernel(ProjArgs a) {
  typedef typename Elt<DT>::T T;
  typedef typename std::conditional<WQ, int8_t, T>::type TW;
  static_assert(!W4 || WQ, "4-bit codes are a quantised format");
  constexpr int E = Elt<DT>::PER16;
  constexpr int EW = W4 ? 32 : WQ ? 16 : E;  // weights per 16-byte load
  constexpr int RPW = row_rows_per_wave<WQ, MT, NORM, W4>();  // rows per wave
  constexpr int NS = NWV * RPW;            // row slots per workgroup
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int FW = SWI ? NS / 2 : NS;    // output features per workgroup
  // 1 KB chunks per row and batch: 8 KB a wave, except int8 for several
  // tokens, which keeps 4 (more spill).
  constexpr int U = RPW == 4 ? 2 : (WQ && (RPW == 2 || MT > 1)) ? 4 : 8;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  T* xs = reinterpret_cast<T*>(smem);  // [M][K]
  __shared__ float rstd_s[MT];
  __shared__ float part_s[NWV];
  __shared__ float res_s[NS][MT];
  constexpr bool D2 = W4 && MT == 1 && DT == DT_BF16;  // dot2 path (above)
  __shared__ float psx_s[NWV];  // D2: per-wave sums of the staged activations
  float sx = 0.f;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = a.K, M = a.M;
  const int RS = W4 ? K / 2 : K;  // row stride in TW units
  const int f0 = blockIdx.x * FW;
  // Slot s (this wave's are wave, wave + NWV, ...): feature f0 + s (SwiGLU:
  // gate rows in the first FW slots, the matching up rows in the rest).  Rows
  // past N read row 0; their results are dropped.  int8 rows bring a scale.
  const TW* wp[RPW];
  float wscale[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int slot = wave + r * NWV;
    const int f = f0 + (SWI ? (slot % FW) : slot);
    const int fs = f < a.N ? f : 0;
    wscale[r] = 1.f;
    if constexpr (SWI) {
      wp[r] = reinterpret_cast<const TW*>(slot < FW ? a.w[0] : a.w[1]) + (size_t)fs * RS;
      if constexpr (WQ) wscale[r] = a.wscale[slot < FW ? 0 : 1][fs];
    } else {
      if constexpr (W4) {
        const int sg = fs < a.seg1 ? 0 : fs < a.seg2 ? 1 : 2;
        const int f_in = fs - (sg == 0 ? 0 : sg == 1 ? a.seg1 : a.seg2);
        wp[r] = reinterpret_cast<const TW*>(a.w[sg]) + (size_t)f_in * RS;
      } else {
        wp[r] = seg_row<TW>(a, fs);
      }
      if constexpr (WQ)
        wscale[r] = fs < a.seg1 ? a.wscale[0][fs]
                  : fs < a.seg2 ? a.wscale[1][fs - a.seg1] : a.wscale[2][fs - a.seg2];
    }
  }
  const int nch = (K + 64 * EW - 1) / (64 * EW);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 wv[RPW][U];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (c0 + u) * 64 * EW + lane * EW;
#pragma unroll
      for (int r = 0; r < RPW; ++r) wv[r][u] = (k < K) ? ld16_stream(wp[r] + (W4 ? k / 2 : k)) : zero;
    }
  };
  // Weight loads start before the activations are staged.
  load_batch(0);

  constexpr bool PRE = NORM && DT == DT_F16;  // see stage_prescaled
  const int KC = K / E;
  const T* xg = reinterpret_cast<const T*>(a.x);
  const T* gg = reinterpret_cast<const T*>(a.gamma);
  for (int m = 0; m < M; ++m) {
    float ss = 0.f;
    for (int c = tid; c < KC; c += NWV * 64) {
      u32x4 xv = ld16(xg + (size_t)m * K + c * E);
      if constexpr (NORM) {
        float xf[E], gf[E];
        unpack16<DT>(xv, xf);
        if constexpr (!PRE) unpack16<DT>(ld16(gg + c * E), gf);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          ss += xf[e] * xf[e];
          if constexpr (!PRE) xf[e] *= gf[e];
        }
        if constexpr (!PRE) xv = pack16<DT>(xf);
      }
      if constexpr (D2) {
        xv = pair_interleave(xv);
#pragma unroll
        for (int i = 0; i < 4; ++i) sx = dot2_bf16(xv[i], 0x3f803f80u, sx);
      }
      st16(xs + (size_t)m * K + c * E, xv);
    }
    if constexpr (D2) {
      sx = wave_sum(sx);
      if (lane == 0) psx_s[wave] = sx;
    }
    if constexpr (NORM) {
      ss = wave_sum(ss);
      if (lane == 0) part_s[wave] = ss;
      __syncthreads();
      if (tid == 0) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) t += part_s[w];
        rstd_s[m] = 1.0f / sqrtf(t / (float)K + a.eps);
      }
      __syncthreads();
    }
  }
  if constexpr (PRE) stage_prescaled<DT>(xs, gg, rstd_s, M, K, tid, NWV * 64);
  __syncthreads();

  float acc[RPW][MT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += U) {
    if (c0 > 0) load_batch(c0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (c0 + u) * 64 * EW + lane * EW;
      if (k >= K) break;
      if constexpr (W4) {
        // E activations at a time; their E codes come out of one or half a
        // 32-bit word of each row.
#pragma unroll
        for (int h = 0; h < EW / E; ++h) {
          if constexpr (D2) {
            // Activations staged in pair order: (x0,x4), (x1,x5), (x2,x6), (x3,x7).
            const u32x4 xp = ld16(xs + k + h * E);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
              const uint32_t uw = wv[r][u][h] ^ 0x88888888u;
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc[r][0] = dot2_bf16(((uw >> (4 * j)) & 0x000f000fu) | 0x43004300u, xp[j], acc[r][0]);
            }
            continue;
          } else if constexpr (MT == 1) {
            // One token: each code is used once, so convert it at its FMA
            // (fewer live registers, more waves per SIMD).
            float xf[E];
            unpack16<DT>(ld16(xs + k + h * E), xf);
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
              for (int e = 0; e < E; ++e) {
                const int idx = h * E + e;
                const uint32_t word = wv[r][u][idx >> 3];
                acc[r][0] += (float)((int32_t)(word << (28 - 4 * (idx & 7))) >> 28) * xf[e];
              }
            continue;
          }
          float wf4[RPW][E];
#pragma unroll
          for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const int idx = h * E + e;
              const uint32_t word = wv[r][u][idx >> 3];
              wf4[r][e] = (float)((int32_t)(word << (28 - 4 * (idx & 7))) >> 28);
            }
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m < M) {
              float xf[E];
              unpack16<DT>(ld16(xs + (size_t)m * K + k + h * E), xf);
#pragma unroll
              for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[r][m] += wf4[r][e] * xf[e];
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        float wf[RPW][EW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          if constexpr (WQ) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int b = 0; b < 4; ++b)
                wf[r][4 * i + b] = (float)(int8_t)(wv[r][u][i] >> (8 * b));
          } else {
            unpack16<DT>(wv[r][u], wf[r]);
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < M) {
#pragma unroll
            for (int h = 0; h < EW / E; ++h) {
              float xf[E];
              unpack16<DT>(ld16(xs + (size_t)m * K + k + h * E), xf);
#pragma unroll
              for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[r][m] += wf[r][h * E + e] * xf[e];
            }
          }
        }
        // int8: keep each chunk's conversions and activation reads next to
        // their use; hoisted across the batch they exhaust the registers.
        if constexpr (WQ) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]) * wscale[r];
  if constexpr (D2) {  // the codes entered as 136 + q
    float sxt = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) sxt += psx_s[w];
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[r][0] -= 136.f * sxt * wscale[r];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) res_s[wave + r * NWV][m] = acc[r][m];
  }
  __syncthreads();

  // Epilogue: thread t < FW * M (QKV: one thread per 4 features) takes
  // feature f0 + t % FW of token t / FW.
  if constexpr (EPI == EPI_QKV) {
    constexpr int G4 = FW / 4;
    if (tid >= G4 * M) return;
    const int m = tid / G4, g = tid - m * G4;
    const int f = f0 + 4 * g;
    if (f >= a.N) return;
    const float scale = (NORM && !PRE) ? rstd_s[m] : 1.f;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = res_s[4 * g + i][m] * scale;
    qkv_epilogue4<DT>(a, a.tok0 + m, m, f, v);
  } else {
    if (tid >= FW * M) return;
    const int m = tid / FW, i = tid - m * FW;
    const int f = f0 + i;
    if (f >= a.N) return;
    const float scale = (NORM && !PRE) ? rstd_s[m] : 1.f;
    const float v = res_s[i][m] * scale;
    if constexpr (EPI == EPI_LOGITS) {
      reinterpret_cast<float*>(a.y)[(size_t)m * a.N + f] = v;
    } else if constexpr (EPI == EPI_RESID) {
      const T* rp = reinterpret_cast<const T*>(a.resid) + (size_t)m * a.N + f;
      reinterpret_cast<T*>(a.y)[(size_t)m * a.N + f] = Elt<DT>::from_f32(Elt<DT>::to_f32(*rp) + v);
    } else {  // SwiGLU
      const float up = res_s[FW + i][m] * scale;
      reinterpret_cast<T*>(a.y)[(size_t)m * a.N + f] = Elt<DT>::from_f32(silu(v) * up);
    }
  }
}

template <int DT, int EPI, bool NORM>
static hipError_t gemv_row_launch(const ProjArgs& a, hipStream_t s) {
  // One row per wave; the QKV epilogue needs N % 4 == 0 (head_dim is a
  // multiple of 8).  Workgroup size: with a fused norm every workgroup also
  // reduces the activations, so small ones (4 waves) start sooner; without one
  // larger ones (16 waves) stage the activations fewer times.  Measured on
  // the 7B decode: QKV 20.3 -> 19.4 us, gate/up 30.1 -> 29.4, O 8.1 -> 7.6,
  // down 18.3 -> 17.8 against 8 waves throughout.
  constexpr int NWV = NORM ? 4 : 16;
  constexpr int FW = (EPI == EPI_SWIGLU) ? NWV / 2 : NWV;
  const int grid = (a.N + FW - 1) / FW;
  const size_t sh = gemv_lds_bytes(DT, a.M, a.K);
  auto go = [&](auto k) -> hipError_t {
    if (sh > (size_t)GEMV_LDS_BYTES) {
      const hipError_t e =
          hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
      if (e != hipSuccess) return e;
    }
    LL_LAUNCH(k, dim3(grid), dim3(NWV * 64), sh, s, a);
    return hipGetLastError();
  };
  if (a.M == 1) return go(gemv_row1_kernel<DT, EPI, NORM, 1, NWV>);
  return go(gemv_row1_kernel<DT, EPI, NORM, 4, NWV>);
}

// int8 (or, W4, int4) weights, 1-4 tokens: the row kernel with a larger
// activation stage.
template <int DT, int EPI, bool NORM, bool W4>
static hipError_t gemv_row_w8_launch(const ProjArgs& a, hipStream_t s) {
  constexpr int NWV = NORM ? 4 : 16;
  // Features per workgroup: NWV rows (two per wave for one token), halved for
  // SwiGLU's gate/up pairs.
  const int rows = NWV * (a.M == 1 ? row_rows_per_wave<true, 1, NORM, W4>()
                                    : row_rows_per_wave<true, 4, NORM, W4>());
  const int FW = (EPI == EPI_SWIGLU) ? rows / 2 : rows;
  const int grid = (a.N + FW - 1) / FW;
  const size_t sh = gemv_lds_bytes(DT, a.M, a.K);
  auto go = [&](auto k) -> hipError_t {
    // Dynamic LDS beyond 64 KB has to be allowed for the kernel first.
    if (sh > (size_t)GEMV_LDS_BYTES) {
      const hipError_t e =
          hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
      if (e != hipSuccess) return e;
    }
    LL_LAUNCH(k, dim3(grid), dim3(NWV * 64), sh, s, a);
    return hipGetLastError();
  };
  if (a.M == 1) return go(gemv_row1_kernel<DT, EPI, NORM, 1, NWV, true, W4>);
  return go(gemv_row1_kernel<DT, EPI, NORM, 4, NWV, true, W4>);
}

template <int DT, bool W4>
static hipError_t gemv_w8_dt(int epi, const ProjArgs& a, hipStream_t s) {
  const bool norm = a.gamma != nullptr;
  switch (epi) {
    case EPI_QKV: return norm ? gemv_row_w8_launch<DT, EPI_QKV, true, W4>(a, s)
                              : gemv_row_w8_launch<DT, EPI_QKV, false, W4>(a, s);
    case EPI_RESID: return gemv_row_w8_launch<DT, EPI_RESID, false, W4>(a, s);
    case EPI_SWIGLU: return norm ? gemv_row_w8_launch<DT, EPI_SWIGLU, true, W4>(a, s)
                                 : gemv_row_w8_launch<DT, EPI_SWIGLU, false, W4>(a, s);
  }
  return hipErrorInvalidValue;
}

bool gemv_w8_fits(int dt, int M, int K) {
  return M >= 1 && M <= 4 && K % 16 == 0 && gemv_lds_bytes(dt, M, K) <= (size_t)GEMV_W8_LDS_BYTES;
}

hipError_t launch_gemv_w8(int dt, int epi, const ProjArgs& a, hipStream_t s) {
  if (!a.wscale[0]) return hipErrorInvalidValue;
  if (a.wbits == 4) {
    // int4: the row kernel only (1-4 tokens, K a multiple of 32).
    if (!gemv_w8_fits(dt, a.M, a.K) || a.K % 32) return hipErrorInvalidValue;
    switch (dt) {
      case DT_F32: return gemv_w8_dt<DT_F32, true>(epi, a, s);
      case DT_BF16: return gemv_w8_dt<DT_BF16, true>(epi, a, s);
      case DT_F16: return gemv_w8_dt<DT_F16, true>(epi, a, s);
    }
    return hipErrorInvalidValue;
  }
  // More tokens (or a stage that does not fit) go through the LDS-streaming
  // kernel, which reads every weight once for up to 32 tokens.
  if (!gemv_w8_fits(dt, a.M, a.K)) return launch_gemv_dma_w8(dt, epi, a, s);
  switch (dt) {
    case DT_F32: return gemv_w8_dt<DT_F32, false>(epi, a, s);
    case DT_BF16: return gemv_w8_dt<DT_BF16, false>(epi, a, s);
    case DT_F16: return gemv_w8_dt<DT_F16, false>(epi, a, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// One token, 16-bit formats, K a multiple of 2048: the residual projections
// (O, down) and the QKV projection with its fused norm.  Workgroups walk the
// weight matrix in pieces of R whole rows (R K 2 bytes = 32 KB, or one longer
// row) with a grid-stride loop, the next piece's loads in flight during the
// current piece's products.  The requests in flight then cover a compact
// stretch of memory, where one row per wave has every row of the matrix open
// at once: a copy of the row kernel stripped of its activation stage,
// products and epilogue ran no faster than the whole kernel (70B O 27.0
// against 27.4 us, against 23.5 for a plain read), so the access pattern is
// the difference.  70B O 27.4 -> 25.4 us, down (one 56 KB row per piece)
// 75.7 -> 74.0 us over cold weight copies; QKV 31.4 -> 30.2 us in the
// 80-layer stack.
// Thread t takes chunks t + 256 i of a piece: chunk i is in row i / KCB at
// k = 8 (t + 256 (i % KCB)), so each thread's KCB activation chunks serve
// every row of every piece and stay in registers; the row sums meet in LDS.
// ---------------------------------------------------------------------------
constexpr int PIECE_WG_PER_CU = 8;

template <int DT, int EPI, bool NORM, int KCB, int R>
__global__ __launch_bounds__(256) void gemv_piece_kernel(ProjArgs a, int npieces) {
  typedef typename Elt<DT>::T T;
  constexpr int E = Elt<DT>::PER16, CPT = KCB * R;
  static_assert(E == 8, "16-bit formats");
  static_assert(EPI != EPI_QKV || R % 2 == 0, "the QKV epilogue takes whole RoPE pairs");
  constexpr bool PRE = NORM && DT == DT_F16;  // as in the row kernel (stage_prescaled)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  __shared__ float red[2][4][R];  // by piece parity: one barrier per piece
  // Piece p: features [p R, p R + R), inside one segment (segment starts are
  // multiples of R).
  auto piece_base = [&](int p) {
    const int f = p * R;
    const int sg = f < a.seg1 ? 0 : f < a.seg2 ? 1 : 2;
    const int f_in = f - (sg == 0 ? 0 : sg == 1 ? a.seg1 : a.seg2);
    return reinterpret_cast<const T*>(a.w[sg]) + (size_t)f_in * K + tid * E;
  };
  u32x4 wa[CPT], wb[CPT];
  auto load = [&](u32x4 (&w)[CPT], int p) {
    const T* base = p < npieces ? piece_base(p) : nullptr;
#pragma unroll
    for (int i = 0; i < CPT; ++i) w[i] = p < npieces ? ld16_stream(base + (size_t)i * 256 * E) : zero;
  };
  int p = blockIdx.x;
  load(wa, p);

  // Activation chunks k = 8 (tid + 256 j); with a fused norm, sum x^2 over the
  // row (one barrier), then x * gain (bf16, 1/rms scales the results) or
  // x / rms * gain (f16, whose range the unscaled product could exceed).
  u32x4 xv[KCB];
  const T* xg = reinterpret_cast<const T*>(a.x) + tid * E;
#pragma unroll
  for (int j = 0; j < KCB; ++j) xv[j] = ld16(xg + j * 256 * E);
  float scale = 1.f;
  if constexpr (NORM) {
    const T* gg = reinterpret_cast<const T*>(a.gamma) + tid * E;
    u32x4 gv[KCB];
#pragma unroll
    for (int j = 0; j < KCB; ++j) gv[j] = ld16(gg + j * 256 * E);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < KCB; ++j) {
      float f[E];
      unpack16<DT>(xv[j], f);
#pragma unroll
      for (int e = 0; e < E; ++e) ss += f[e] * f[e];
    }
    ss = wave_sum(ss);
    __shared__ float ss_s[4];
    if (lane == 0) ss_s[wave] = ss;
    __syncthreads();
    const float rstd = 1.0f / sqrtf((ss_s[0] + ss_s[1] + ss_s[2] + ss_s[3]) / (float)K + a.eps);
#pragma unroll
    for (int j = 0; j < KCB; ++j) {
      float f[E], g[E];
      unpack16<DT>(xv[j], f);
      unpack16<DT>(gv[j], g);
#pragma unroll
      for (int e = 0; e < E; ++e) f[e] = PRE ? f[e] * rstd * g[e] : f[e] * g[e];
      xv[j] = pack16<DT>(f);
    }
    if constexpr (!PRE) scale = rstd;
  }

  int par = 0;
  auto piece = [&](u32x4 (&w)[CPT], int pc) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      float wf[E], xf[E];
      unpack16<DT>(w[i], wf);
      unpack16<DT>(xv[i % KCB], xf);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[i / KCB] += wf[e] * xf[e];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = wave_sum(acc[r]);
      if (lane == 0) red[par][wave][r] = v;
    }
    __syncthreads();
    auto row_sum = [&](int r) {
      return (red[par][0][r] + red[par][1][r] + red[par][2][r] + red[par][3][r]) * scale;
    };
    if constexpr (EPI == EPI_QKV) {
      constexpr int G = (R % 4 == 0) ? 4 : 2;  // features per epilogue call
      if (tid < R / G) {
        float v[G];
#pragma unroll
        for (int i = 0; i < G; ++i) v[i] = row_sum(G * tid + i);
        if constexpr (G == 4) qkv_epilogue4<DT>(a, a.tok0, 0, pc * R + 4 * tid, v);
        else qkv_epilogue2<DT>(a, a.tok0, 0, pc * R + 2 * tid, v);
      }
    } else if (tid < R) {
      const int f = pc * R + tid;
      const float v = row_sum(tid);
      if constexpr (EPI == EPI_LOGITS) {
        reinterpret_cast<float*>(a.y)[f] = v;
      } else {
        const T* rp = reinterpret_cast<const T*>(a.resid) + f;
        reinterpret_cast<T*>(a.y)[f] = Elt<DT>::from_f32(Elt<DT>::to_f32(*rp) + v);
      }
    }
    par ^= 1;
  };
  // Buffers alternate with explicit code paths, so the wait for a piece's
  // loads leaves the next piece's in flight.
  while (p < npieces) {
    load(wb, p + gridDim.x);
    piece(wa, p);
    p += gridDim.x;
    if (p >= npieces) break;
    load(wa, p + gridDim.x);
    piece(wb, p);
    p += gridDim.x;
  }
}

template <int DT, int EPI, bool NORM, int KCB, int R>
static hipError_t gemv_piece_launch(const ProjArgs& a, hipStream_t s) {
  const int npieces = a.N / R;
  const int grid = std::min(npieces, 256 * PIECE_WG_PER_CU);
  LL_LAUNCH((gemv_piece_kernel<DT, EPI, NORM, KCB, R>), dim3(grid), dim3(256), 0, s, a, npieces);
  return hipGetLastError();
}

template <int DT, int EPI, bool NORM>
static hipError_t gemv_piece_k(const ProjArgs& a, hipStream_t s, bool& taken) {
  // Rows per piece: 32 KB of them (the QKV epilogue takes RoPE pairs).
  taken = true;
  switch (a.K / 2048) {
    case 1: return gemv_piece_launch<DT, EPI, NORM, 1, 8>(a, s);
    case 2: return gemv_piece_launch<DT, EPI, NORM, 2, 4>(a, s);
    case 4: return gemv_piece_launch<DT, EPI, NORM, 4, 2>(a, s);
  }
  if constexpr (EPI != EPI_QKV) {
    switch (a.K / 2048) {
      case 8: return gemv_piece_launch<DT, EPI, NORM, 8, 1>(a, s);
      case 14: return gemv_piece_launch<DT, EPI, NORM, 14, 1>(a, s);
    }
  }
  taken = false;
  return hipSuccess;
}

// The piece kernel for this launch, if it has one (sets `taken`): one token,
// 16-bit formats, K a multiple of 2048, QKV or residual epilogue.  (The LM
// head, 32000 rows with the norm, measured 82.0 -> 86.4 us in the stack's
// trace, so it keeps the row kernel.)
template <int DT>
static hipError_t gemv_piece_dispatch(int epi, const ProjArgs& a, hipStream_t s, bool& taken) {
  taken = false;
  if constexpr (DT == DT_F32) {
    return hipSuccess;
  } else {
    if (a.M != 1 || a.K % 2048 != 0 || a.N % 8 != 0) return hipSuccess;
    if (epi == EPI_QKV && (a.seg1 % 8 != 0 || a.seg2 % 8 != 0)) return hipSuccess;
    const bool norm = a.gamma != nullptr;
    switch (epi) {
      case EPI_RESID: return norm ? hipSuccess : gemv_piece_k<DT, EPI_RESID, false>(a, s, taken);
      case EPI_QKV: return norm ? gemv_piece_k<DT, EPI_QKV, true>(a, s, taken)
                                : gemv_piece_k<DT, EPI_QKV, false>(a, s, taken);
    }
    return hipSuccess;
  }
}

template <int DT>
static hipError_t gemv_dt(int epi, const ProjArgs& a, hipStream_t s) {
  const bool norm = a.gamma != nullptr;
  {
    bool taken;
    const hipError_t e = gemv_piece_dispatch<DT>(epi, a, s, taken);
    if (taken) return e;
  }
  if (a.M <= 4 && (gemv_fits_lds(DT, a.M, a.K) ||
                   (a.M == 1 && gemv_lds_bytes(DT, 1, a.K) <= (size_t)GEMV_ROW_LDS_BYTES))) {
    switch (epi) {
      case EPI_QKV: return norm ? gemv_row_launch<DT, EPI_QKV, true>(a, s)
                                : gemv_row_launch<DT, EPI_QKV, false>(a, s);
      case EPI_RESID: return gemv_row_launch<DT, EPI_RESID, false>(a, s);
      case EPI_SWIGLU: return norm ? gemv_row_launch<DT, EPI_SWIGLU, true>(a, s)
                                   : gemv_row_launch<DT, EPI_SWIGLU, false>(a, s);
      case EPI_LOGITS: return norm ? gemv_row_launch<DT, EPI_LOGITS, true>(a, s)
                                   : gemv_row_launch<DT, EPI_LOGITS, false>(a, s);
    }
    return hipErrorInvalidValue;
  }
  if (!norm && gemv_dma_supported(DT, a.M, a.K, a.N)) return launch_gemv_dma(DT, epi, a, s);
  if (gemv_fits_lds(DT, a.M, a.K)) {
    switch (epi) {
      case EPI_QKV: return norm ? gemv_lds_launch<DT, EPI_QKV, true>(a, s)
                                : gemv_lds_launch<DT, EPI_QKV, false>(a, s);
      case EPI_RESID: return gemv_lds_launch<DT, EPI_RESID, false>(a, s);
      case EPI_SWIGLU: return norm ? gemv_lds_launch<DT, EPI_SWIGLU, true>(a, s)
                                   : gemv_lds_launch<DT, EPI_SWIGLU, false>(a, s);
      case EPI_LOGITS: return norm ? gemv_lds_launch<DT, EPI_LOGITS, true>(a, s)
                                   : gemv_lds_launch<DT, EPI_LOGITS, false>(a, s);
    }
    return hipErrorInvalidValue;
  }
  if (norm) return hipErrorInvalidValue;  // the caller normalises first
  switch (epi) {
    case EPI_QKV: return gemv_glb_launch<DT, EPI_QKV>(a, s);
    case EPI_RESID: return gemv_glb_launch<DT, EPI_RESID>(a, s);
    case EPI_SWIGLU: return gemv_glb_launch<DT, EPI_SWIGLU>(a, s);
    case EPI_LOGITS: return gemv_glb_launch<DT, EPI_LOGITS>(a, s);
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
