// Causal prefill attention on MFMA (bf16 / f16 inputs, float32 softmax).
//
// Workgroup: 128 queries of one head (32 per wave) against 64-key tiles of the
// head's cache, online softmax across tiles (exact: same result as one softmax
// over all visible keys).  Scores are computed transposed, S^T = K Q^T with
// v_mfma_f32_32x32x16: a lane then owns one query column, so the running max
// and sum of each query are lane-local (plus one exchange with lane l^32), and
// the probabilities it holds are already the B operand of O^T = V^T P^T -- the
// MFMA k order is chosen to match the keys each lane holds.  K is staged in LDS
// row-major (16-byte chunks XOR-swizzled); V is staged transposed, [d][key], so
// the A operand of the second product is two 8-byte LDS reads (its padded row
// of 68 elements puts the 32 rows of one read on distinct banks).  Tiles entirely
// above a wave's last query are skipped; only diagonal tiles are masked.  The
// latest (most expensive) query blocks are launched first.
#include "common.cuh"
#include "epilogue.cuh"

namespace ll {

constexpr int PQ = 128;   // queries per workgroup
constexpr int PKV = 64;   // keys per tile
constexpr int VT_STRIDE = PKV + 4;  // padded row of the transposed V tile (elements)

template <int DT, int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnPrefillArgs a) {
  typedef typename Elt<DT>::T ET;
  constexpr int CPR = HD / 8;          // 16-byte chunks per key row
  constexpr int KPT = HD / 32;         // keys per thread in the V transpose
  // K rows are HD*2 bytes; XOR the 16-byte chunk index with bits of the row so
  // the 16 rows of one ds_read_b128 cycle hit distinct bank groups (256-byte
  // rows: the low four bits; 128-byte rows, two per bank sweep: bits 1..3).
  auto ksw = [](int kr) { return HD == 128 ? (kr & 15) : ((kr >> 1) & 7); };
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[PKV * HD];
  __shared__ __attribute__((aligned(16))) uint16_t lds_vt[HD * VT_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int nqb = gridDim.x;
  const int qb = nqb - 1 - blockIdx.x;  // heavy blocks first
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int j = h / (a.nh / a.nkv);
  const int T = a.T;

  const int q_first = qb * PQ;                       // token index of the block's first query
  const int q_last = min(q_first + PQ, T) - 1;
  const int kv_end = a.start_pos + q_last + 1;       // keys [0, kv_end) are needed
  const int ntiles = (kv_end + PKV - 1) / PKV;

  const int wq0 = q_first + wave * 32;               // this wave's first query
  const int w_last_pos = a.start_pos + min(wq0 + 31, T - 1);
  const int my_t = wq0 + l32;
  const int my_pos = a.start_pos + my_t;

  // Q fragments (B operand of S^T = K Q^T): query my_t, k-chunk s*2 + h2.
  const ET* qp = reinterpret_cast<const ET*>(a.q) + (((size_t)b * a.nh + h) * T + (my_t < T ? my_t : 0)) * HD;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 qf[HD / 16];
#pragma unroll
  for (int s = 0; s < HD / 16; ++s) qf[s] = (my_t < T) ? ld16(qp + s * 16 + h2 * 8) : zero;

  const size_t head_off = ((size_t)b * a.nkv + j) * a.s_max * HD;
  const ET* kbase = reinterpret_cast<const ET*>(a.kc) + head_off;
  const ET* vbase = reinterpret_cast<const ET*>(a.vc) + head_off;

  f32x16 oacc[HD / 32];
#pragma unroll
  for (int d = 0; d < HD / 32; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float qk_scale = 1.44269504088896341f / sqrtf((float)HD);

  for (int tile = 0; tile < ntiles; ++tile) {
    const int key0 = tile * PKV;
    __syncthreads();
    // K tile -> LDS (row-major, swizzled).  Keys >= kv_end are zero.
#pragma unroll
    for (int i = 0; i < (PKV * CPR) / 256; ++i) {
      const int idx = tid + i * 256;
      const int kr = idx / CPR, c = idx - kr * CPR;
      const int key = key0 + kr;
      const u32x4 v = (key < kv_end) ? ld16(kbase + (size_t)key * HD + c * 8) : zero;
      st16(&lds_k[kr * HD + ((c ^ ksw(kr)) << 3)], v);
    }
    // V tile -> LDS transposed: thread takes KPT keys x 8 dims.
    {
      const int dc = tid % CPR;
      const int kg = tid / CPR;
      uint32_t e16[KPT][4];
#pragma unroll
      for (int kk = 0; kk < KPT; ++kk) {
        const int key = key0 + kg * KPT + kk;
        const u32x4 v = (key < kv_end) ? ld16(vbase + (size_t)key * HD + dc * 8) : zero;
#pragma unroll
        for (int w = 0; w < 4; ++w) e16[kk][w] = v[w];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = dc * 8 + e;
        uint16_t* dst = &lds_vt[d * VT_STRIDE + kg * KPT];
        if constexpr (KPT == 4) {
          u32x2 pk;
          const int sh = (e & 1) * 16;
          pk[0] = ((e16[0][e >> 1] >> sh) & 0xffffu) | (((e16[1][e >> 1] >> sh) & 0xffffu) << 16);
          pk[1] = ((e16[2][e >> 1] >> sh) & 0xffffu) | (((e16[3][e >> 1] >> sh) & 0xffffu) << 16);
          *reinterpret_cast<u32x2*>(dst) = pk;
        } else {
          const int sh = (e & 1) * 16;
          const uint32_t pk = ((e16[0][e >> 1] >> sh) & 0xffffu) | (((e16[1][e >> 1] >> sh) & 0xffffu) << 16);
          *reinterpret_cast<uint32_t*>(dst) = pk;
        }
      }
    }
    __syncthreads();
    if (key0 > w_last_pos) continue;  // every key of this tile is in this wave's future

    // S^T = K Q^T for the tile's two 32-key blocks.
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) {
      const int ch = s * 2 + h2;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kr = kb * 32 + l32;
        const u32x4 kf = ld16(&lds_k[kr * HD + ((ch ^ ksw(kr)) << 3)]);
        sacc[kb] = mfma32<DT>(kf, qf[s], sacc[kb]);
      }
    }
    // Scale, mask, online softmax (log2 domain).
    const bool need_mask = key0 + PKV - 1 > a.start_pos + wq0;
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float sv = sacc[kb][i] * qk_scale;
        if (need_mask) {
          const int key = key0 + kb * 32 + (i >> 2) * 8 + h2 * 4 + (i & 3);
          if (key > my_pos) sv = -INFINITY;
        }
        sacc[kb][i] = sv;
        mt = fmaxf(mt, sv);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2f(sacc[kb][i] - m_use);
        sacc[kb][i] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < HD / 32; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;

    // O^T += V^T P^T.  MFMA (kb, hf) covers keys kb*32 + hf*16 + (e/4)*8 + h2*4 + e%4.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = sacc[kb][hf * 8 + e];
        const u32x4 pb = pack16<DT>(pf);
        const int kofs = kb * 32 + hf * 16 + h2 * 4;
#pragma unroll
        for (int d = 0; d < HD / 32; ++d) {
          const uint16_t* vr = &lds_vt[(d * 32 + l32) * VT_STRIDE + kofs];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
          const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
          oacc[d] = mfma32<DT>(va, pb, oacc[d]);
        }
      }
    }
  }

  // Normalise and write o[b, t, h*HD + d].
  if (my_t < T) {
    const float inv = 1.0f / l_run;
    const size_t obase = ((size_t)b * T + my_t) * (size_t)(a.nh * HD) + h * HD;
#pragma unroll
    for (int d = 0; d < HD / 32; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dd = d * 32 + g4 * 8 + h2 * 4;
        store4_rt(a.o, obase + dd, a.out_dt, oacc[d][g4 * 4] * inv, oacc[d][g4 * 4 + 1] * inv,
                  oacc[d][g4 * 4 + 2] * inv, oacc[d][g4 * 4 + 3] * inv);
      }
  }
}

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s) {
  dim3 grid((a.T + PQ - 1) / PQ, a.nh, a.B);
  if (a.dt == DT_BF16) {
    if (a.hd == 128) LL_LAUNCH((attn_prefill_kernel<DT_BF16, 128>), grid, dim3(256), 0, s, a);
    else LL_LAUNCH((attn_prefill_kernel<DT_BF16, 64>), grid, dim3(256), 0, s, a);
  } else if (a.dt == DT_F16) {
    if (a.hd == 128) LL_LAUNCH((attn_prefill_kernel<DT_F16, 128>), grid, dim3(256), 0, s, a);
    else LL_LAUNCH((attn_prefill_kernel<DT_F16, 64>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ll
