// Token sampling after the LM head: repetition penalty, temperature, top-k,
// softmax, top-p and the draw ("Llama2架构与推理全解析" §2.5 names the steps,
// §3.3 gives typical settings; "Llama2架构全景解析" §2.2, step 3, draws from
// softmax(logits / T)).
//
// One 1024-thread workgroup per row.  Each thread keeps EPT = 32 logits of the
// row in registers (vocabularies up to 32768; 64 per thread would spill at
// 1024 threads) as order-preserving 32-bit keys (a larger float gives a larger
// key).  Appending the inverted vocabulary index (16 bits) makes every
// element's 48-bit composite distinct and orders equal logits by lower index,
// so a 6-pass radix select (8 bits per pass, histograms in LDS) finds the k-th
// largest composite exactly and exactly k elements lie at or above it.  Those
// k (<= 1024) are sorted in LDS by a bitonic network, and one block scan of
// exp(z - z_max) in that order gives the softmax mass, the top-p cut (the
// smallest leading set whose mass reaches top_p) and the inverse-CDF draw at
// the caller's uniform u.  Temperature 0 is the greedy limit: k = 1.
#include "common.cuh"
#include "kernels.h"

namespace ll {

constexpr int SM_THREADS = 1024;
constexpr int SM_WAVES = SM_THREADS / 64;

__device__ __forceinline__ uint32_t float_key(float z) {
  const uint32_t f = __float_as_uint(z);
  return (f & 0x80000000u) ? ~f : (f | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Inclusive sum over the workgroup in thread order; `tot` gets the total.
__device__ __forceinline__ float block_scan(float v, float* wsum, float* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    float w = lane < SM_WAVES ? wsum[lane] : 0.f;
#pragma unroll
    for (int o = 1; o < SM_WAVES; o <<= 1) {
      const float t = __shfl_up(w, o, 64);
      if (lane >= o) w += t;
    }
    if (lane < SM_WAVES) wsum[SM_WAVES + lane] = w;  // inclusive wave prefix
  }
  __syncthreads();
  if (wave > 0) v += wsum[SM_WAVES + wave - 1];
  *tot = wsum[2 * SM_WAVES - 1];
  return v;
}

template <int EPT>
__global__ __launch_bounds__(SM_THREADS) void sample_kernel(SampleArgs a) {
  __shared__ uint32_t seen[SAMPLE_MAX_VOCAB / 32];
  // 16 copies of the 256-bin histogram (lane & 15 picks one), 257 words
  // apart so that one digit's copies sit in 16 different banks: lanes of a
  // wave that share a digit then collide 4 at a time instead of 64.
  __shared__ uint32_t hist[16 * 257];
  __shared__ uint64_t cand[SM_THREADS];
  __shared__ float wsum[2 * SM_WAVES];
  __shared__ uint64_t sel[3];  // selected prefix, remaining count, bin taken whole
  __shared__ uint32_t ncand;

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int V = a.vocab;
  const bool greedy = !(a.temperature > 0.f);
  const int k = greedy ? 1 : min(a.top_k, V);

  // Ids already seen in this row's history (each penalised once).
  for (int i = tid; i < (V + 31) / 32; i += SM_THREADS) seen[i] = 0u;
  if (tid < 1024) cand[tid] = 0ull;
  if (tid == 0) ncand = 0u;
  __syncthreads();
  if (a.history) {
    const int32_t* h = a.history + (size_t)row * a.n_hist;
    for (int i = tid; i < a.n_hist; i += SM_THREADS) {
      const int id = h[i];
      if (id >= 0 && id < V) atomicOr(&seen[id >> 5], 1u << (id & 31));
    }
  }
  __syncthreads();

  // Penalised, tempered logits as keys; 0 marks a slot past the vocabulary
  // (no float maps to key 0 except a NaN pattern).
  const float* lg = a.logits + (size_t)row * V;
  uint32_t key[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int v = j * SM_THREADS + tid;
    uint32_t kk = 0u;
    if (v < V) {
      float z = lg[v];
      if ((seen[v >> 5] >> (v & 31)) & 1u) z = z > 0.f ? z / a.penalty : z * a.penalty;
      if (!greedy) z = z / a.temperature;
      kk = float_key(z);
    }
    key[j] = kk;
  }

  // Radix select of the k-th largest composite (key << 16 | (0xffff - v)).
  // Once the chosen digit's bin holds exactly the elements still wanted,
  // every element of it is selected and the lower digits need no pass.
  uint64_t prefix = 0ull, mask = 0ull;
  uint32_t remaining = (uint32_t)k;
  const int copy = (tid & 15) * 257;
  for (int pass = 0; pass < 6; ++pass) {
    const int shift = 40 - 8 * pass;
    for (int i = tid; i < 16 * 257; i += SM_THREADS) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int v = j * SM_THREADS + tid;
      if (v < V) {
        const uint64_t c = ((uint64_t)key[j] << 16) | (uint64_t)(0xffff - v);
        if ((c & mask) == prefix) atomicAdd(&hist[copy + (int)((c >> shift) & 255u)], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // Lane l owns bins 252-4l .. 255-4l (high digits in low lanes); an
      // inclusive scan over lanes counts everything at or above a lane's bins.
      const int lane = tid;
      uint32_t b[4], s = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bin = 255 - 4 * lane - i;
        uint32_t t = 0u;
#pragma unroll
        for (int c = 0; c < 16; ++c) t += hist[c * 257 + bin];
        b[i] = t;
        s += b[i];
      }
      uint32_t incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const uint32_t excl = incl - s;
      if (excl < remaining && incl >= remaining) {
        uint32_t above = excl, in_bin = 0u;
        int d = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (above + b[i] >= remaining) {
            d = 255 - 4 * lane - i;
            in_bin = b[i];
            break;
          }
          above += b[i];
        }
        sel[0] = prefix | ((uint64_t)d << shift);
        sel[1] = remaining - above;
        sel[2] = (above + in_bin == remaining) ? 1ull : 0ull;
      }
    }
    __syncthreads();
    prefix = sel[0];
    remaining = (uint32_t)sel[1];
    mask |= 255ull << shift;
    const bool whole_bin = sel[2] != 0ull;
    __syncthreads();
    if (whole_bin) break;
  }

  // The k composites at or above the k-th largest, sorted ascending (the
  // unused slots stay 0 and sort first).
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int v = j * SM_THREADS + tid;
    if (v < V) {
      const uint64_t c = ((uint64_t)key[j] << 16) | (uint64_t)(0xffff - v);
      if (c >= prefix) {
        const uint32_t slot = atomicAdd(&ncand, 1u);
        if (slot < SM_THREADS) cand[slot] = c;
      }
    }
  }
  __syncthreads();
  // Ascending bitonic sort of the first SZ slots (SZ = k rounded up to a
  // power of two; the unused ones hold 0 and sort first).
  int sz = 1;
  while (sz < k) sz <<= 1;
  for (int size = 2; size <= sz; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int other = tid ^ stride;
      if (tid < sz && other > tid) {
        const uint64_t x = cand[tid], y = cand[other];
        const bool up = (tid & size) == 0;
        if (up ? x > y : x < y) {
          cand[tid] = y;
          cand[other] = x;
        }
      }
      __syncthreads();
    }
  }

  // Candidate i (the i-th largest) sits at cand[sz - 1 - i].
  const int i = tid;
  const uint64_t ci = cand[sz - 1 - (i < k ? i : 0)];
  const float z0 = key_float((uint32_t)(cand[sz - 1] >> 16));
  const float e = i < k ? expf(key_float((uint32_t)(ci >> 16)) - z0) : 0.f;
  float total;
  const float cum = block_scan(e, wsum, &total);
  // Top-p: keep candidate i while the mass before it is below top_p.
  const int n = __syncthreads_count(i < k && (cum - e) < a.top_p * total);
  // Mass of the kept set, then the first kept candidate whose cumulative mass
  // exceeds u times it.
  if (i == n - 1) wsum[0] = cum;
  __syncthreads();
  const float target = a.u[row] * wsum[0];
  const int below = __syncthreads_count(i < n && cum <= target);
  const int pick = below < n ? below : n - 1;
  if (i == pick) a.ids_out[row] = 0xffff - (int)(ci & 0xffffull);
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
  if (a.vocab < 1 || a.vocab > SAMPLE_MAX_VOCAB) return hipErrorInvalidValue;
  LL_LAUNCH(sample_kernel<SAMPLE_MAX_VOCAB / SM_THREADS>, dim3(a.n), dim3(SM_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace ll
