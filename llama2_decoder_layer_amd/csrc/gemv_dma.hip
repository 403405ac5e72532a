// Weight-streaming projection for up to 32 tokens in a 16-bit format:
// D[f, m] = sum_k W[f, k] x[m, k], every weight byte read once from HBM.
//
// A workgroup owns 64 weight rows (SwiGLU: 32 gate + the 32 matching up rows)
// and all token slots (32, the missing ones read token 0 and are dropped), over
// one K range.  Weights and activations move global -> LDS by
// global_load_lds in 64-k stages (128-byte row slices), NST stages deep, so
// each workgroup keeps up to (NST-1) x 12 KB in flight without holding any of
// it in registers.  The four waves split a stage's work as 2 row blocks x 2
// k halves of v_mfma_f32_32x32x16; the k halves meet in LDS at the end.
//
// The 16-byte chunks of a 128-byte row slice are stored XOR-swizzled by
// (row >> 1) & 7, which makes the fragment reads conflict-free: the 16 rows one
// ds_read_b128 cycle serves land in 16 distinct 4-bank groups.
//
// Few row blocks (O, down, QKV at batch 32) leave CUs idle, so the K range is
// split over several workgroups; each split writes float32 partials and a
// small kernel sums them and applies the epilogue.  One split applies the
// epilogue directly: residual add, SwiGLU, RoPE + KV append, or logits.
#include "common.cuh"
#include "epilogue.cuh"

namespace ll {

constexpr int SK_BM = 64;                          // weight rows per workgroup
constexpr int SK_BN = 32;                          // token slots
constexpr int SK_BK = 64;                          // k per stage
constexpr int SK_NST = 4;                          // stages in LDS
constexpr int SK_ROWB = SK_BK * 2;                 // bytes per row slice
constexpr int SK_STAGE = (SK_BM + SK_BN) * SK_ROWB;  // 12 KB
constexpr int SK_TARGET_WG = 512;                  // workgroups wanted per launch
constexpr int SK_MAX_SPLIT = 8;

// Features covered by one workgroup and the number of K splits used.
static int sk_features(int epi) { return epi == EPI_SWIGLU ? SK_BM / 2 : SK_BM; }

static int sk_split(int epi, int N, int K, int* kchunk) {
  const int nblk = (N + sk_features(epi) - 1) / sk_features(epi);
  int ns = (SK_TARGET_WG + nblk - 1) / nblk;
  ns = std::max(1, std::min(ns, SK_MAX_SPLIT));
  const int nkt = K / SK_BK;
  ns = std::min(ns, nkt);
  const int kt_per = (nkt + ns - 1) / ns;
  *kchunk = kt_per * SK_BK;
  return (nkt + kt_per - 1) / kt_per;
}

// Weight rows of a launch: N (SwiGLU: gate rows then up rows, 2N).
static int sk_rows(int epi, int N) { return epi == EPI_SWIGLU ? 2 * N : N; }

// Epilogue for four consecutive features f..f+3 of token m.
template <int DT, int EPI>
__device__ __forceinline__ void sk_store4(const ProjArgs& a, int m, int f, const float* v,
                                          const float* up) {
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
    store4<DT>(y, silu(v[0]) * up[0], silu(v[1]) * up[1], silu(v[2]) * up[2],
               silu(v[3]) * up[3]);
  } else {
    float w[4] = {v[0], v[1], v[2], v[3]};
    qkv_epilogue4<DT>(a, a.tok0 + m, m, f, w);
  }
}

template <int DT, int EPI, bool SPLIT>
__global__ __launch_bounds__(256) void gemv_dma_kernel(ProjArgs a, float* part, int kchunk, int nsplit) {
  typedef typename Elt<DT>::T T;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int FB = SWI ? SK_BM / 2 : SK_BM;  // features per workgroup
  // One LDS object: the stage ring, reused at the end for the cross-wave sums.
  // (A second LDS variable gives the accesses alias scopes, and the wait-count
  // pass then waits for every outstanding DMA before each fragment read.)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[SK_NST * SK_STAGE];
  f32x16* red = reinterpret_cast<f32x16*>(lds);  // [2][64] after the k loop

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K;
  // Grid x enumerates (row block, K split) with the split fastest, so the
  // workgroups resident together cover neighbouring K ranges of the same rows.
  const int blk = blockIdx.x / nsplit, ks = blockIdx.x - blk * nsplit;
  const int f0 = blk * FB;
  const int k0 = ks * kchunk;
  const int nkt = (min(K, k0 + kchunk) - k0) / SK_BK;

  // DMA: instruction i of a stage fills rows 8i..8i+7 (i < 8: weights, else
  // tokens 8(i-8)..); wave w issues i = w, w+4 (weights) and w+8 (tokens).
  // Lane l: row 8i + l/8, physical chunk l%8 = logical chunk ^ ((row>>1)&7).
  const int rr = lane >> 3, pc = lane & 7;
  const T* src[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int i = wave + 4 * j;
    const int r = 8 * (i & 7) + rr;
    const int c = pc ^ ((r >> 1) & 7);
    const T* row;
    if (j < 2) {
      if constexpr (SWI) {
        const int f = f0 + (r & 31);
        row = reinterpret_cast<const T*>(r < 32 ? a.w[0] : a.w[1]) + (size_t)(f < a.N ? f : 0) * K;
      } else {
        const int f = f0 + r;
        row = seg_row<T>(a, f < a.N ? f : 0);
      }
    } else {
      row = reinterpret_cast<const T*>(a.x) + (size_t)(r < a.M ? r : 0) * K;
    }
    src[j] = row + k0 + c * 8;
  }
  auto issue = [&](int st, int kt) {
    uint8_t* base = lds + st * SK_STAGE;
    const int k = kt * SK_BK;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (j < 2) dma16_stream(src[j] + k, base + (wave + 4 * j) * 1024);  // weights
      else dma16(src[j] + k, base + (wave + 4 * j) * 1024);               // activations
    }
  };
  // This wave's part of a stage has landed once at most `newer` later stages
  // (3 loads each) are outstanding.
  auto wait_stage = [&](int newer) {
    if (newer >= 2) wait_vmcnt<6>();
    else if (newer == 1) wait_vmcnt<3>();
    else wait_vmcnt<0>();
  };

  // Fragments: wave w multiplies row block rb = w & 1 over k-steps 2(w>>1)
  // and 2(w>>1)+1 of every stage.
  const int rb = wave & 1, kh = wave >> 1;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int swz = (l32 >> 1) & 7;
  const int aoff = (rb * 32 + l32) * SK_ROWB;
  const int boff = SK_BM * SK_ROWB + l32 * SK_ROWB;
  const int ch0 = (((4 * kh + 0 + h2) ^ swz) * 16);  // k-step 2kh: logical chunk 2(2kh)+h2
  const int ch1 = (((4 * kh + 2 + h2) ^ swz) * 16);  // k-step 2kh+1

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

#pragma unroll
  for (int st = 0; st < SK_NST - 1; ++st)
    if (st < nkt) issue(st, st);
  // The barrier is a bare s_barrier: a full __syncthreads would also wait for
  // the stages still in flight.  Its explicit waits: this wave's loads of stage
  // kt (vmcnt) and its reads of stage kt-1, which the MFMAs consumed.  The
  // sched_barriers keep the fragment reads below it.
  for (int kt = 0; kt < nkt; ++kt) {
    wait_stage(min(nkt - 1, kt + SK_NST - 2) - kt);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();  // stage kt complete everywhere; stage kt-1 no longer read
    __builtin_amdgcn_sched_barrier(0);
    if (kt + SK_NST - 1 < nkt) issue((kt + SK_NST - 1) % SK_NST, kt + SK_NST - 1);
    const uint8_t* base = lds + (kt % SK_NST) * SK_STAGE;
    const u32x4 a0 = ld16(base + aoff + ch0), b0 = ld16(base + boff + ch0);
    const u32x4 a1 = ld16(base + aoff + ch1), b1 = ld16(base + boff + ch1);
    acc = mfma32<DT>(a0, b0, acc);
    acc = mfma32<DT>(a1, b1, acc);
    __builtin_amdgcn_sched_barrier(0);
  }

  // k halves meet: waves 2, 3 hand their sums to waves 0, 1 (once every wave
  // is done with the last stage, whose buffer may be the one reused).
  __syncthreads();
  if (kh == 1) red[rb * 64 + lane] = acc;
  __syncthreads();
  if (kh == 0) acc += red[rb * 64 + lane];
  if constexpr (!SPLIT && SWI) {
    // Gate rows are in wave 0, the matching up rows in wave 1.
    __syncthreads();
    if (wave == 1) red[lane] = acc;
    __syncthreads();
    if (wave != 0) return;
  }
  if (kh == 1) return;

  // Lane holds token l32 and rows rb*32 + g*8 + h2*4 + 0..3, g = 0..3.
  const int m = l32;
  if constexpr (SPLIT) {
    if (m < a.M) {
      const int nrows = SWI ? 2 * a.N : a.N;
      float* p = part + ((size_t)ks * a.M + m) * nrows;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = rb * 32 + g * 8 + h2 * 4;
        const int f = SWI ? (r < 32 ? f0 + r : a.N + f0 + r - 32) : f0 + r;
        if ((SWI ? f0 + (r & 31) : f) < a.N) {
          f32x4 v = {acc[g * 4], acc[g * 4 + 1], acc[g * 4 + 2], acc[g * 4 + 3]};
          *reinterpret_cast<f32x4*>(p + f) = v;
        }
      }
    }
  } else if constexpr (SWI) {
    if (m >= a.M) return;
    const f32x16 up = red[lane];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = f0 + g * 8 + h2 * 4;
      if (f >= a.N) continue;
      float v[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = acc[g * 4 + i]; u[i] = up[g * 4 + i]; }
      sk_store4<DT, EPI>(a, m, f, v, u);
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
template <int DT, int EPI>
__global__ __launch_bounds__(256) void gemv_split_reduce_kernel(ProjArgs a, const float* part,
                                                                int nsplit) {
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
  sk_store4<DT, EPI>(a, m, f, vv, uu);
}

size_t gemv_dma_partial_floats(int epi, int N, int K, int M) {
  if (K % SK_BK != 0 || M < 1 || M > SK_BN) return 0;
  int kchunk;
  const int ns = sk_split(epi, N, K, &kchunk);
  return ns > 1 ? (size_t)ns * M * sk_rows(epi, N) : 0;
}

bool gemv_dma_supported(int dt, int M, int K, int N) {
  return dt != DT_F32 && M >= 1 && M <= SK_BN && K % SK_BK == 0 && N % 4 == 0;
}

template <int DT, int EPI>
static hipError_t gemv_dma_epi(const ProjArgs& a, hipStream_t s) {
  int kchunk;
  const int ns = sk_split(EPI, a.N, a.K, &kchunk);
  const int nblk = (a.N + sk_features(EPI) - 1) / sk_features(EPI);
  if (ns == 1) {
    LL_LAUNCH((gemv_dma_kernel<DT, EPI, false>), dim3(nblk), dim3(256), 0, s, a,
              (float*)nullptr, kchunk, 1);
    return hipGetLastError();
  }
  if (!a.part) return hipErrorInvalidValue;
  LL_LAUNCH((gemv_dma_kernel<DT, EPI, true>), dim3(nblk * ns), dim3(256), 0, s, a, a.part, kchunk,
            ns);
  const int n = ((a.N + 3) / 4) * a.M;
  LL_LAUNCH((gemv_split_reduce_kernel<DT, EPI>), dim3((n + 255) / 256), dim3(256), 0, s, a,
            (const float*)a.part, ns);
  return hipGetLastError();
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
