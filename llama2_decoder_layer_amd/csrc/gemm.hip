// Prefill projections: y[m, n] = sum_k u[m, k] W[n, k] for many tokens m.
//
// The tile is computed transposed, D[feature, token] = W u^T, so that the four
// consecutive output features a lane holds (v_mfma_f32_32x32x16 result layout)
// give lane-local RoPE pairs, lane-local SwiGLU (gate and up land in the same
// lane) and 8-byte stores.  Workgroup tile: 128 weight rows x 128 tokens x 64 k,
// four waves; both operands are staged through LDS (double buffered, 16-byte
// chunks XOR-swizzled by row so the ds_read_b128 of an MFMA fragment spreads
// over the banks).  Tiles are numbered so that each XCD gets a contiguous run
// and, within it, groups of 4 weight panels x 8 token panels share L2.
#include "common.cuh"
#include "epilogue.cuh"

namespace ll {

constexpr int GBM = 128;  // weight rows (features) per tile
constexpr int GBN = 128;  // tokens per tile
constexpr int GBK = 64;   // k per stage
constexpr int GROUP_M = 4;

template <int DT, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(ProjArgs a) {
  typedef typename Elt<DT>::T T;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int FM = SWI ? GBM / 2 : GBM;  // output features per tile
  constexpr int RB = SWI ? 4 : 2;          // 32-row blocks per wave
  constexpr int CB = SWI ? 1 : 2;          // 32-token blocks per wave

  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][GBM * GBK];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][GBN * GBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const int ntm = (a.N + FM - 1) / FM;
  const int ntn = (a.M + GBN - 1) / GBN;

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
  const int n0 = tile_n * GBN;

  // Global -> LDS assignment: 128 rows x 8 chunks per operand, 4 chunks per thread.
  const int lc = tid & 7;          // chunk within the 128-byte row slice
  const int lr = tid >> 3;         // rows lr + 32 i
  const T* arow[4];
  const T* brow[4];
  bool av[4], bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lr + 32 * i;
    int f;
    if constexpr (SWI) {
      f = f0 + (r & 63);
      av[i] = f < a.N;
      const T* base = reinterpret_cast<const T*>(r < 64 ? a.w[0] : a.w[1]);
      arow[i] = base + (size_t)(av[i] ? f : 0) * K;
    } else {
      f = f0 + r;
      av[i] = f < a.N;
      arow[i] = seg_row<T>(a, av[i] ? f : 0);
    }
    const int m = n0 + r;
    bv[i] = m < a.M;
    brow[i] = reinterpret_cast<const T*>(a.x) + (size_t)(bv[i] ? m : 0) * K;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k = kt * GBK + lc * 8;
    const bool kin = k < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = (kin && av[i]) ? ld16(arow[i] + k) : zero;
      rb[i] = (kin && bv[i]) ? ld16(brow[i] + k) : zero;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lr + 32 * i;
      const int off = r * GBK + ((lc ^ (r & 7)) << 3);
      st16(&lds_a[buf][off], ra[i]);
      st16(&lds_b[buf][off], rb[i]);
    }
  };

  // Wave placement inside the tile.
  int row_base[RB], col_base[CB];
  if constexpr (SWI) {
#pragma unroll
    for (int r = 0; r < RB; ++r) row_base[r] = r * 32;
    col_base[0] = wave * 32;
  } else {
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int r = 0; r < RB; ++r) row_base[r] = wm * 64 + r * 32;
#pragma unroll
    for (int c = 0; c < CB; ++c) col_base[c] = wn * 64 + c * 32;
  }
  const int l32 = lane & 31, h2 = lane >> 5;

  f32x16 acc[RB][CB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.f;

  const int nkt = (K + GBK - 1) / GBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < GBK / 16; ++s) {
      const int ch = s * 2 + h2;
      u32x4 fa[RB], fb[CB];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int row = row_base[r] + l32;
        fa[r] = ld16(&lds_a[cur][row * GBK + ((ch ^ (row & 7)) << 3)]);
      }
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int col = col_base[c] + l32;
        fb[c] = ld16(&lds_b[cur][col * GBK + ((ch ^ (col & 7)) << 3)]);
      }
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c) acc[r][c] = mfma32<DT>(fa[r], fb[c], acc[r][c]);
    }
    if (kt + 1 < nkt) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  acc[r][c][i]: feature row_base[r] + (i/4)*8 + h2*4 + i%4,
  // token col_base[c] + l32.
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int m = n0 + col_base[c] + l32;
    if (m >= a.M) continue;
#pragma unroll
    for (int r = 0; r < (SWI ? 2 : RB); ++r) {
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
          for (int i = 0; i < 4; ++i) o[i] = silu(v[i]) * acc[r + 2][c][g4 * 4 + i];
          T* y = reinterpret_cast<T*>(a.y) + (size_t)m * a.N + f;
          store4<DT>(y, o[0], o[1], o[2], o[3]);
        } else {
          qkv_epilogue4<DT>(a, a.tok0 + m, m, f, v);
        }
      }
    }
  }
}

template <int DT>
static hipError_t gemm_dt(int epi, const ProjArgs& a, hipStream_t s) {
  const int fm = (epi == EPI_SWIGLU) ? GBM / 2 : GBM;
  const int ntiles = ((a.N + fm - 1) / fm) * ((a.M + GBN - 1) / GBN);
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<DT, EPI_QKV>), dim3(ntiles), dim3(256), 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_kernel<DT, EPI_RESID>), dim3(ntiles), dim3(256), 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<DT, EPI_SWIGLU>), dim3(ntiles), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int dt, int epi, const ProjArgs& a, hipStream_t s) {
  if (dt == DT_BF16) return gemm_dt<DT_BF16>(epi, a, s);
  if (dt == DT_F16) return gemm_dt<DT_F16>(epi, a, s);
  return hipErrorInvalidValue;
}

}  // namespace ll
