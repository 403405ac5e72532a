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
// K/V tile stages in LDS (head_dim 128 kernel).  Two keep two workgroups per
// CU; three or four (one workgroup per CU) measured 1.6-1.8x slower.
constexpr int PF_STAGES = 2;
static_assert(PF_STAGES == 2, "the head_dim 128 loop alternates two buffers");

// The work item (query block, head, sequence) of this workgroup; grid
// (query blocks, heads, sequences).  Workgroup i of a launch runs on XCD
// i % 8.  When the (sequence, head) units split evenly over the 8 XCDs, each
// XCD takes a contiguous run of units, so the query blocks of a head (and the
// heads of one KV group) read their K and V through one L2, and walks its
// units heaviest (latest) query block first.  Otherwise the grid order, also
// heaviest first.
struct PrefillItem {
  int qb, h, b;
};
__device__ __forceinline__ PrefillItem prefill_item() {
  const int nqb = gridDim.x, nh = gridDim.y;
  const int units = nh * gridDim.z;
  if (units % 8 != 0) return {nqb - 1 - (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
  const int lin = blockIdx.x + nqb * (blockIdx.y + nh * blockIdx.z);
  const int xcd = lin & 7, r = lin >> 3;  // r < nqb * units / 8
  const int per = units / 8;
  const int qi = r / per;
  const int u = xcd * per + (r - qi * per);
  return {nqb - 1 - qi, u % nh, u / nh};
}

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
  const PrefillItem it = prefill_item();
  const int qb = it.qb, h = it.h, b = it.b;
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

  const ET* kbase = reinterpret_cast<const ET*>(a.kc);
  const ET* vbase = reinterpret_cast<const ET*>(a.vc);

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
      const u32x4 v = (key < kv_end)
          ? ld16(kbase + kv_row(a.pages, b, j, key, a.nkv, a.s_max, HD) + c * 8) : zero;
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
        const u32x4 v = (key < kv_end)
            ? ld16(vbase + kv_row(a.pages, b, j, key, a.nkv, a.s_max, HD) + dc * 8) : zero;
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

// head_dim 128: the same blocking, but K and V tiles move global -> LDS by
// global_load_lds into a two-stage ring (tile t+1 loads while tile t is used)
// and V stays in its [key][dim] layout.  The A operand of O^T = V^T P^T is read
// with ds_read_b64_tr_b16, which transposes 16-bit data across each group of 16
// lanes: when lane i = 4e + q of a group reads the 4 elements at (row R + e,
// col C + 4q), lane j of the group receives rows R..R+3 of col C + j.  Two
// such reads give a lane the 8 keys its MFMA k-group needs for one dim.
// Swizzles (16-byte chunk c of row r stored at chunk c ^ f(r)): K uses
// f = r & 15 (16 rows of one b128 read on distinct banks); V uses
// f = 4 (r & 3) (the 4 rows x 64 bytes of 32 lanes' transposed reads cover all
// 64 banks once).  The DMA writes the swizzled layout by permuting each lane's
// global address.
template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_prefill_tr_kernel(AttnPrefillArgs a) {
  typedef typename Elt<DT>::T ET;
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  constexpr int HD = 128;
  constexpr int ROWB = HD * 2;                   // bytes per key row
  constexpr int TILE_B = PKV * ROWB;             // one K or V tile: 16 KB
  constexpr int STAGE_B = 2 * TILE_B;            // K then V
  // One LDS object (a second one gives the accesses alias scopes, and the
  // wait-count pass then waits for every outstanding DMA before each read).
  __shared__ __attribute__((aligned(1024))) uint8_t lds[PF_STAGES * STAGE_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;
  const PrefillItem it = prefill_item();
  const int qb = it.qb, h = it.h, b = it.b;
  const int j = h / (a.nh / a.nkv);
  const int T = a.T;

  const int q_first = qb * PQ;
  const int q_last = min(q_first + PQ, T) - 1;
  const int kv_end = a.start_pos + q_last + 1;       // keys [0, kv_end) are needed
  const int ntiles = (kv_end + PKV - 1) / PKV;

  const int wq0 = q_first + wave * 32;
  const int w_last_pos = a.start_pos + min(wq0 + 31, T - 1);
  const int my_t = wq0 + l32;
  const int my_pos = a.start_pos + my_t;

  const ET* qp = reinterpret_cast<const ET*>(a.q) + (((size_t)b * a.nh + h) * T + (my_t < T ? my_t : 0)) * HD;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 qf[HD / 16];
#pragma unroll
  for (int s = 0; s < HD / 16; ++s) qf[s] = (my_t < T) ? ld16(qp + s * 16 + h2 * 8) : zero;

  const ET* kbase = reinterpret_cast<const ET*>(a.kc);
  const ET* vbase = reinterpret_cast<const ET*>(a.vc);

  // DMA: instruction i of wave w fills rows 16w + 4i + (lane >> 4), physical
  // chunk lane & 15.  Rows past kv_end read the last needed row (finite; those
  // keys are masked).  Contiguous caches: a uniform (scalar) base pointer per
  // tile plus fixed per-lane offsets, so issuing a tile costs no vector
  // arithmetic; only the last tile clamps its rows.  A paged cache: the
  // wave's 16 rows are 16-aligned keys (or all the clamped last key) inside
  // one block of at least 16 positions, so the block index is wave-uniform
  // and comes from a scalar load, which leaves the DMA wait counts alone.
  const int rsub = lane >> 4, pch = lane & 15;
  const int vcol = (pch ^ (4 * rsub)) * 8;  // (16w + 4i + rsub) & 3 == rsub
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int koff[4], voff[4];  // element offsets of this lane's rows at key0 = 0
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wave + 4 * i + rsub;
    koff[i] = r * HD + (pch ^ (r & 15)) * 8;
    voff[i] = r * HD + vcol;
  }
  const size_t head_base = ((size_t)b * a.nkv + j) * a.s_max * HD;
  auto issue = [&](int buf, int key0) {
    uint8_t* kb = lds + buf * STAGE_B + 16 * wave_u * ROWB;
    uint8_t* vb = kb + TILE_B;
    if (!a.pages.table && key0 + PKV <= kv_end) {
      const ET* ks = kbase + head_base + (size_t)key0 * HD;
      const ET* vs = vbase + head_base + (size_t)key0 * HD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dma16(ks + koff[i], kb + 4 * i * ROWB);
        dma16(vs + voff[i], vb + 4 * i * ROWB);
      }
      return;
    }
    size_t base;
    int kmask;
    if (a.pages.table) {
      const int blk = kv_block_uniform(a.pages, b, min(key0 + 16 * wave, kv_end - 1));
      base = (((size_t)blk * a.nkv + j) << a.pages.log2_bs) * HD;
      kmask = (1 << a.pages.log2_bs) - 1;
    } else {
      base = head_base;
      kmask = -1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + rsub;
      const int key = min(key0 + r, kv_end - 1);
      const int kcol = (pch ^ (r & 15)) * 8;
      const size_t row = base + (size_t)(key & kmask) * HD;
      dma16(kbase + row + kcol, kb + 4 * i * ROWB);
      dma16(vbase + row + vcol, vb + 4 * i * ROWB);
    }
  };

  f32x16 oacc[HD / 32];
#pragma unroll
  for (int d = 0; d < HD / 32; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float qk_scale = 1.44269504088896341f / sqrtf((float)HD);

  // LDS byte offsets of this lane's fragment reads within a tile, fixed for
  // the whole loop (the buffer, key block and half-tile offsets are
  // immediates):
  //  K, MFMA step s: row l32 (+32 kb), chunk (2s + h2) ^ (l32 & 15).
  //  V transposed reads for dims d*32 + [0, 32): group gi = lane >> 4 covers
  //  dims (gi & 1)*16 + [0, 16) and keys (gi >> 1)*4 + 4 rows (+ kb*32 +
  //  hf*16, + 8 for the second read); the swizzle is 4 (row & 3) = 4 e with
  //  e = ii >> 2 for every read, so chunk (d*4 + c0) ^ 4e = 4 (d ^ e) + c0.
  int kaddr[HD / 16];
#pragma unroll
  for (int st = 0; st < HD / 16; ++st) kaddr[st] = l32 * ROWB + (((st * 2 + h2) ^ (l32 & 15)) << 4);
  const int gi = lane >> 4, ii = lane & 15;
  const int tr_row = (gi >> 1) * 4 + (ii >> 2);
  const int tr_col = (gi & 1) * 16 + 4 * (ii & 3);
  const int e4 = ii >> 2, c0 = tr_col >> 3;
  int vaddr[HD / 32];
#pragma unroll
  for (int d = 0; d < HD / 32; ++d)
    vaddr[d] = TILE_B + tr_row * ROWB + ((4 * (d ^ e4) + c0) << 4) + ((tr_col >> 2) & 1) * 8;

  // Tile t+1 loads while tile t is used (8 DMA loads per wave and tile); the
  // loop is unrolled by the two buffers so every LDS offset is constant.
  if (ntiles > 0) issue(0, 0);
  auto process = [&](auto BUF, int tile) {
    constexpr int buf = decltype(BUF)::value;
    const int key0 = tile * PKV;
    if (tile + 1 < ntiles) wait_vmcnt<0>();  // this wave's part of the tile has landed
    else wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();  // tile landed everywhere; tile-1's buffer is free
    __builtin_amdgcn_sched_barrier(0);
    if (tile + 1 < ntiles) issue(buf ^ 1, key0 + PKV);
    if (key0 > w_last_pos) return;  // every key of this tile is in this wave's future
    const uint8_t* tb = lds + buf * STAGE_B;

    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
    // K fragments one step ahead of their MFMAs (the scheduler would otherwise
    // wait for each pair of reads right before its MFMAs).
    u32x4 kf[2][2];
    auto kread = [&](int st, int slot) {
      kf[slot][0] = ld16(tb + kaddr[st]);
      kf[slot][1] = ld16(tb + kaddr[st] + 32 * ROWB);
    };
    kread(0, 0);
    static_for<0, HD / 16>([&](auto STI) {
      constexpr int st = decltype(STI)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (st + 1 < HD / 16) kread(st + 1, (st + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32<DT>(kf[st & 1][kb], qf[st], sacc[kb]);
    });
    __builtin_amdgcn_sched_barrier(0);
    // Online softmax on unscaled scores; the scale folds into the exponent,
    // p = 2^(s c - m c) with c = log2(e)/sqrt(hd).  The reference max m_run is
    // only raised when a score exceeds it by more than 8 (log2 units), so the
    // running sums are rarely rescaled and p stays <= 2^8.
    if (key0 + PKV - 1 > a.start_pos + wq0) {  // diagonal tile: causal mask
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + (i >> 2) * 8 + h2 * 4 + (i & 3);
          if (key > my_pos) sacc[kb][i] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * qk_scale;
    const bool raise = mt > m_run + 8.f;  // also true on a lane's first visible key
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;  // 0 when m_run = -inf
      const float m_new = raise ? mt : m_run;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < HD / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      m_run = m_new;
    }
    // A lane with no visible key yet keeps m_run = -inf: its p are 0.
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], qk_scale, -m_use));
        sacc[kb][i] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32, 64);
    l_run += rs;

    // O^T += V^T P^T.  MFMA (kb, hf) covers keys kb*32 + hf*16 + (e/4)*8 + h2*4 + e%4.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = sacc[kb][hf * 8 + e];
        const u32x4 pb = pack16<DT>(pf);
#pragma unroll
        for (int d = 0; d < HD / 32; ++d) {
          const int rb = (kb * 32 + hf * 16) * ROWB;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(tb + vaddr[d] + rb));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(tb + vaddr[d] + rb + 8 * ROWB));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2v = __builtin_bit_cast(u32x2, hi);
          const u32x4 va = {l2[0], l2[1], h2v[0], h2v[1]};
          oacc[d] = mfma32<DT>(va, pb, oacc[d]);
        }
      }
    }
  };
  for (int tile = 0; tile < ntiles; tile += 2) {
    process(ic<0>{}, tile);
    if (tile + 1 < ntiles) process(ic<1>{}, tile + 1);
  }

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
    if (a.hd == 128) LL_LAUNCH((attn_prefill_tr_kernel<DT_BF16>), grid, dim3(256), 0, s, a);
    else LL_LAUNCH((attn_prefill_kernel<DT_BF16, 64>), grid, dim3(256), 0, s, a);
  } else if (a.dt == DT_F16) {
    if (a.hd == 128) LL_LAUNCH((attn_prefill_tr_kernel<DT_F16>), grid, dim3(256), 0, s, a);
    else LL_LAUNCH((attn_prefill_kernel<DT_F16, 64>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ll
