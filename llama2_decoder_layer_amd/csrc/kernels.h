// Host-side launch interface between the C ABI (layer.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ll {

enum Epi {
  EPI_QKV = 0,     // RoPE on q/k, q to the workspace, k/v appended to the caches
  EPI_RESID = 1,   // y = resid + acc
  EPI_SWIGLU = 2,  // y = silu(acc_gate) * acc_up   (two weight matrices)
  EPI_LOGITS = 3,  // y (float32) = acc
};

// Arguments of one projection y[m, n] = sum_k act(x)[m, k] * W[n, k].
// A paged KV cache: k/v pools [n_blocks, nkv, 1 << log2_bs, hd]; table[b *
// stride + i] is the pool block holding positions [i << log2_bs, (i+1) <<
// log2_bs) of sequence b (entries are clamped into [0, n_blocks)).
struct KvPages {
  const int32_t* table;
  int stride, log2_bs, n_blocks;
};

// Element offset of the row of position `pos` of KV head j of sequence b:
// contiguous caches [B, nkv, s_max, hd], or through the block table.
__device__ __forceinline__ size_t kv_row(const KvPages& pg, int b, int j, int pos, int nkv,
                                         int s_max, int hd) {
  if (!pg.table) return (((size_t)b * nkv + j) * s_max + pos) * hd;
  int blk = pg.table[(size_t)b * pg.stride + (pos >> pg.log2_bs)];
  blk = blk < 0 ? 0 : (blk >= pg.n_blocks ? pg.n_blocks - 1 : blk);
  return ((((size_t)blk * nkv + j) << pg.log2_bs) + (pos & ((1 << pg.log2_bs) - 1))) * hd;
}

// Pool block of position `key` of sequence b when both are the same in every
// lane of the wave: a scalar load (constant address space), which waits on
// lgkmcnt, so it leaves the vector-memory counts of the DMA pipelines alone.
__device__ __forceinline__ int kv_block_uniform(const KvPages& pg, int b, int key) {
  typedef __attribute__((address_space(4))) const int32_t* cptr;
  const int idx = __builtin_amdgcn_readfirstlane(b * pg.stride + (key >> pg.log2_bs));
  int blk = ((cptr)pg.table)[idx];
  return blk < 0 ? 0 : (blk >= pg.n_blocks ? pg.n_blocks - 1 : blk);
}

struct ProjArgs {
  const void* w[3];   // row segments: [0,seg1) w[0]; [seg1,seg2) w[1]; [seg2,N) w[2]
  int seg1, seg2;     // (EPI_SWIGLU: w[0] = gate, w[1] = up, both N rows)
  int N, K, M;        // out features, in features, tokens in this launch
  int tok0;           // global index of this launch's first token
  const void* x;      // [M, K] activations (raw hidden state when `gamma` is set)
  const void* gamma;  // RMSNorm gain [K] (fused norm) or nullptr
  float eps;
  const void* resid;  // [M, N] (EPI_RESID)
  void* y;            // [M, N]
  // EPI_QKV
  float* q32;         // [M, nh*hd] float32, rows of this launch (decode-style attention)
  void* q16;          // [B, nh, T, hd] in the KV-cache format (prefill attention)
  void* kc;
  void* vc;
  const int32_t* ctx_len;  // decode: position of token n is ctx_len[n]; else start_pos + n%T
  int start_pos, T, max_ctx;
  int nh, nkv, hd, s_max, kv_dt;
  const float* rcos;
  const float* rsin;
  float* part;        // float32 K-split partials of the streaming projection (workspace)
  const float* wscale[3];  // int8 / int4 weights: float32 scale per row of each segment
  int wbits;               // quantised weights: 8 (int8 codes) or 4 (packed int4 codes)
  KvPages pages;           // paged caches (pages.table == nullptr: contiguous)
  // RMSNorm of the next projection's input, deferred into the streaming
  // kernels (bf16 activations).  An EPI_RESID K-split launch with nout set
  // also writes nout = y * ngamma [M, N] and, for token m, the sum of y^2 over
  // features 1024 g .. 1024 g + 1023 into ssq[16 m + g] (g < ssq_parts =
  // N / 1024 <= 16; the other slots of the 16 get zeros).  An EPI_SWIGLU
  // launch with ssq set multiplies both of its sums by
  // 1 / sqrt(sum of the 16 slots / K + eps) before the SwiGLU.
  void* nout;
  const void* ngamma;
  float* ssq;
  int ssq_parts;
};

// Decode-sized projection (M <= 32 tokens).  A fused norm (gamma != nullptr)
// needs the M activation rows to fit the LDS stage: gemv_fits_lds(dt, M, K).
hipError_t launch_gemv(int dt, int epi, const ProjArgs& a, hipStream_t s);
bool gemv_fits_lds(int dt, int M, int K);
// Weight-only int8 projection for 1-4 tokens (a.w int8 [N][K] per segment,
// a.wscale float32 per row; K % 16 == 0; activations of the M tokens within
// GEMV_W8_LDS_BYTES).
constexpr int GEMV_W8_LDS_BYTES = 128 * 1024;
bool gemv_w8_fits(int dt, int M, int K);
hipError_t launch_gemv_w8(int dt, int epi, const ProjArgs& a, hipStream_t s);
// a.wbits == 4: packed int4 codes (weight 2j in the low nibble of byte j,
// rows of K/2 bytes), K % 32 == 0, and only what gemv_w8_fits admits.
// Weight-only int8 through the LDS-streaming kernel (16-bit activations, M <= 32,
// K % 64 == 0, no fused norm; partials as gemv_dma_partial_floats).
hipError_t launch_gemv_dma_w8(int dt, int epi, const ProjArgs& a, hipStream_t s);
// Partial sums per token (N_o / 1024) with which the residual projection
// [N_o x K_o] at M tokens can defer the norm of its output into the gate/up
// projection [2 I x N_o] (int8 weights when w8), or 0 when the two launches
// do not take the streaming paths that implement it.
int gemv_dma_norm_parts(int dt, bool w8, int M, int N_o, int K_o, int I);
// Positions [start, start + count) of every (sequence, KV head) of contiguous
// caches [B, nkv, s_max, hd] copied into the pools of a paged cache.
hipError_t launch_kv_pages_write(const void* k_src, const void* v_src, int s_max, int start,
                                 int count, void* k_pool, void* v_pool, const KvPages& pg,
                                 int batch, int nkv, int hd, int kv_dt, hipStream_t s);
// Per-row symmetric int8 codes and float32 scales of a [rows, cols] matrix.
hipError_t launch_quantize_w8(int dt, const void* w, int8_t* q, float* scale, int rows, int cols,
                              hipStream_t s);
hipError_t launch_quantize_w4(int dt, const void* w, uint8_t* q, float* scale, int rows, int cols,
                              hipStream_t s);
// Prefill projection (M tokens): MFMA tiles with fused epilogues.  When the
// last round of 256 x 256 tiles would leave CUs idle, its tiles are split
// along K; the partials go to a.part, which must hold gemm_partial_bytes.
hipError_t launch_gemm(int dt, int epi, const ProjArgs& a, hipStream_t s);
size_t gemm_partial_bytes(int epi, int N, int M, int K);

// Weight-streaming projection through LDS for 16-bit formats (K % 64 == 0,
// N % 4 == 0, M <= 32, no fused norm); launch_gemv picks it when the row
// kernel does not apply.  Few row blocks split K; the splits' partials go to
// a.part, which must hold gemv_dma_partial_floats(epi, N, K, M) floats.
bool gemv_dma_supported(int dt, int M, int K, int N);
size_t gemv_dma_partial_floats(int epi, int N, int K, int M);
hipError_t launch_gemv_dma(int dt, int epi, const ProjArgs& a, hipStream_t s);

// RMSNorm of `rows` rows of width H: u = x / sqrt(mean(x^2) + eps) * gamma.
hipError_t launch_rmsnorm(int dt, const void* x, const void* gamma, void* u, int rows, int H,
                          float eps, hipStream_t s);

// Split-over-context attention for single queries.  Query n (of B*T) belongs
// to sequence n/T at position ctx_len[n/T] (decode) or start_pos + n%T
// (prefill); it attends over cache positions 0..pos.
struct AttnDecodeArgs {
  const float* q;        // [nq, nh, hd] float32
  const void* kc;        // [B, nkv, s_max, hd]
  const void* vc;
  const int32_t* ctx_len;
  int start_pos, T, max_ctx;
  int nq, nh, nkv, hd, s_max, kv_dt, act_dt;
  int chunk, nsplit;     // keys per split, splits per query
  float* part_m;         // [nq, nh, nsplit]
  float* part_l;         // [nq, nh, nsplit]
  float* part_acc;       // [nq, nh, nsplit, hd]
  void* o;               // [nq, nh*hd] act dtype
  KvPages pages;         // paged caches: kc/vc are the pools, rows of query n's sequence n / T
};
hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t s);
// Query heads served per workgroup for a GQA group of g heads.
int attn_heads_per_group(int g);
// Keys per split for the launch (one of 2, 4 or 8 x 256/(hd/8); 256 to 2048
// for the GQA kernel), or -1 when
// the context needs more than ATTN_MAX_SPLITS splits of the largest chunk.
constexpr int ATTN_MAX_SPLITS = 1024;
int attn_pick_chunk(int hd, int max_keys, int queries, int nkv, int g, int kv_dt);
// 16-bit caches with 4 or 8 query heads per group take the MFMA-score kernel
// (chunks of 256 to 2048 keys).
bool attn_uses_gqa_kernel(int kv_dt, int g);
// Smallest chunk attn_pick_chunk returns (sizes the workspace).
inline int attn_min_chunk(int hd) { return 2 * (256 / (hd / 8)); }

// Causal prefill attention with MFMA (16-bit formats).
struct AttnPrefillArgs {
  const void* q;   // [B, nh, T, hd] in format dt
  const void* kc;  // [B, nkv, s_max, hd] in format dt (bf16 or f16)
  const void* vc;
  void* o;         // [B, T, nh*hd] in format out_dt
  int B, T, start_pos, nh, nkv, hd, s_max, dt, out_dt;
  KvPages pages;   // paged caches: kc/vc are the pools (block_size >= 16)
};
hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s);

hipError_t launch_rope_table(float* c, float* sn, int max_pos, int hd, double theta, hipStream_t s);
hipError_t launch_embed(const void* table, const int32_t* ids, void* h, int n, int H, int vocab,
                        int dt, hipStream_t s);
hipError_t launch_argmax(const float* logits, int32_t* ids, int n, int vocab, hipStream_t s);

// Kernel ids for the timing hooks (order matches kernel_names in layer.hip).
enum KernelId {
  KID_RMSNORM = 0,
  KID_GEMV_QKV,
  KID_GEMV_O,
  KID_GEMV_GATEUP,
  KID_GEMV_DOWN,
  KID_GEMM_QKV,
  KID_GEMM_O,
  KID_GEMM_GATEUP,
  KID_GEMM_DOWN,
  KID_ATTN_DECODE,
  KID_ATTN_PREFILL,
  KID_SAMPLE,
  KID_COUNT
};
// Benchmark timer.  timer_before arms an event pair for the next launch when
// kernel `kid` is the one being timed; the launch itself (LL_LAUNCH) hands the
// pair to the dispatch, which records its own start and end, so the pair
// brackets that kernel's execution and nothing else.  timer_after disarms.
struct ArmedEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
void timer_before(int kid, hipStream_t s);
void timer_after(int kid, hipStream_t s);
ArmedEvents take_armed_events();

// Every kernel of the library is launched through this macro.
// Token sampling, one workgroup per row (vocab <= SAMPLE_MAX_VOCAB, top_k <= 1024).
constexpr int SAMPLE_MAX_VOCAB = 32768;
struct SampleArgs {
  const float* logits;     // [n, vocab]
  const int32_t* history;  // [n, n_hist] or nullptr
  int n_hist;
  const float* u;          // [n]
  int32_t* ids_out;        // [n]
  int n, vocab;
  float temperature;       // 0: greedy
  int top_k;
  float top_p, penalty;
};
hipError_t launch_sample(const SampleArgs& a, hipStream_t s);

#define LL_LAUNCH(kernel, grid, block, shm, stream, ...)                                      \
  do {                                                                                        \
    const ::ll::ArmedEvents ev_ = ::ll::take_armed_events();                                  \
    if (ev_.start)                                                                            \
      hipExtLaunchKernelGGL(kernel, grid, block, shm, stream, ev_.start, ev_.stop, 0,         \
                            __VA_ARGS__);                                                     \
    else                                                                                      \
      hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__);                      \
  } while (0)

}  // namespace ll
