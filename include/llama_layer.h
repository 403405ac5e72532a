/*
 * llama_layer.h -- C ABI of the MI355X (gfx950) Llama-2 decoder layer.
 *
 * One call runs one pre-norm decoder layer for a batch of sequences:
 *
 *   u   = RMSNorm(x; attn_norm, eps)                 per token, eps inside the root
 *   q,k,v = u W_q^T, u W_k^T, u W_v^T                split into heads of head_dim
 *   q,k = RoPE(q,k; position)                        adjacent pairs (2i, 2i+1) turned
 *                                                    by position * rope_theta^(-2i/head_dim)
 *   K/V cache[b, j, position, :] = k, v              append (k after RoPE)
 *   o_h = softmax(q_h K_j^T / sqrt(head_dim) + causal mask) V_j,  j = h / (n_heads/n_kv_heads)
 *   h1  = x + o W_o^T
 *   out = h1 + (silu(u2 W_gate^T) * (u2 W_up^T)) W_down^T,   u2 = RMSNorm(h1; ffn_norm, eps)
 *
 * Definitions: "Llama2架构与推理全解析：从原理到KV Cache与量化部署" §1.2 (RMSNorm),
 * §1.3 (SwiGLU), §1.4 (RoPE), §1.5 (GQA), §2.1 (prefill / decode), §2.3 (the
 * per-layer recipe and residual stream), §2.4 (KV cache); "Llama2架构全景解析"
 * §1.1 (pre-norm, RoPE as multiplication by e^{i m theta}), §1.2 (query heads
 * sharing one K/V head); "LLM架构全景解析：从基础模块到工程实践" §2.2 (the cache
 * object written at the current position).
 *
 * Around the layer: the same layer over a paged KV cache (decode and chunked
 * prefill), with weight-only INT8 or INT4 projections (decode), RoPE tables (also
 * NTK-scaled for longer contexts), embedding lookup, the LM head with a
 * greedy pick, and a fused sampler (penalty, temperature, top-k, top-p).
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are DEVICE pointers unless stated otherwise, dense,
 *    row-major, 16-byte aligned (int32 id/length arrays and float32 logits:
 *    4-byte aligned).  The caller owns every buffer; the library
 *    never allocates or frees device memory and never synchronises.
 *  - Work is enqueued on `stream` (a hipStream_t of the calling process's HIP
 *    runtime; NULL = the null stream) and runs asynchronously.
 *  - Weights are stored [out_features, in_features] (y = x W^T).
 *  - Return 0 on success, a negative LL_E* code otherwise.  Arguments are
 *    validated on the host before anything is enqueued, so a call that fails
 *    validation has no side effect.  Faults inside kernels surface at the
 *    caller's next synchronisation, as with any asynchronous API.
 *  - Calls are stateless; distinct buffers may be used from several host
 *    threads at once.  Calls that share a workspace must be ordered (same
 *    stream, or synchronised).
 */
#ifndef LLAMA_LAYER_H
#define LLAMA_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats. */
typedef enum { LL_F32 = 0, LL_BF16 = 1, LL_F16 = 2 } ll_dtype;

/* Error codes. */
enum {
  LL_OK = 0,
  LL_EINVAL = -1,       /* bad configuration or size                         */
  LL_ENULL = -2,        /* a required pointer is NULL                        */
  LL_EALIGN = -3,       /* a pointer is not 16-byte aligned                  */
  LL_ECACHE_FULL = -4,  /* positions would run past the cache capacity s_max */
  LL_EWORKSPACE = -5,   /* workspace missing or smaller than required        */
  LL_EHIP = -6,         /* the HIP runtime reported an error at launch       */
  LL_EUNSUPPORTED = -7, /* valid but not implemented (e.g. head_dim 96)      */
  LL_ESCRATCH = -8      /* llama_layer_decode_noalloc: call exceeds its scratch */
};

/*
 * Layer hyper-parameters, named as in the size table of
 * "Llama2架构与推理全解析" §1.6.
 *   hidden        model width H (multiple of 8)
 *   n_heads       query heads
 *   n_kv_heads    key/value heads; n_heads % n_kv_heads == 0 (GQA; == MHA when equal)
 *   head_dim      64 or 128; n_heads * head_dim must be a multiple of 8
 *   intermediate  SwiGLU width I (multiple of 8)
 *   eps           RMSNorm epsilon (> 0)
 *   rope_theta    RoPE base (> 1)
 *   act_dtype     format of weights, gains, x and y: LL_F32 or LL_BF16 (or LL_F16)
 *   kv_dtype      format of the K/V caches: LL_F32, LL_BF16 or LL_F16
 *                 (LL_F32 caches require act_dtype LL_F32)
 *   max_pos       rows of rope_cos / rope_sin; every position used must be < max_pos
 */
typedef struct {
  int32_t hidden, n_heads, n_kv_heads, head_dim, intermediate;
  float eps, rope_theta;
  int32_t act_dtype, kv_dtype;
  int32_t max_pos;
} ll_config;

/*
 * One layer's parameters (device pointers, act_dtype unless noted).
 *   attn_norm [H]                  gain of the attention RMSNorm
 *   w_q [n_heads*head_dim, H]      w_k, w_v [n_kv_heads*head_dim, H]
 *   w_o [H, n_heads*head_dim]
 *   ffn_norm [H]                   gain of the FFN RMSNorm
 *   w_gate, w_up [I, H]            w_down [H, I]
 *   rope_cos, rope_sin  float32 [max_pos, head_dim/2]: cos/sin(m * theta_i),
 *                       as written by llama_rope_table().
 */
typedef struct {
  const void *attn_norm, *w_q, *w_k, *w_v, *w_o, *ffn_norm, *w_gate, *w_up, *w_down;
  const float *rope_cos, *rope_sin;
} ll_weights;

/*
 * Bytes of device workspace a prefill (tokens = T) or decode (tokens = 1)
 * call with this configuration needs; 0 if the configuration is invalid.  With
 * tokens = 1 the size covers both a decode of `batch` sequences and a
 * one-token prefill.
 */
size_t llama_layer_workspace_size(const ll_config* cfg, int32_t batch, int32_t tokens,
                                  int32_t s_max);

/*
 * Prefill ("Llama2架构与推理全解析" §2.1): all `tokens` new tokens of each of
 * `batch` sequences at positions start_pos .. start_pos+tokens-1.
 *   x        [batch, tokens, H] act_dtype, read only
 *   y        [batch, tokens, H] act_dtype, written; must not overlap x
 *   k_cache, v_cache  [batch, n_kv_heads, s_max, head_dim] kv_dtype: positions
 *            < start_pos are read as they are, the new positions are written
 *   ws       workspace of at least llama_layer_workspace_size(cfg, batch, tokens, s_max) bytes
 * Errors: LL_ECACHE_FULL if start_pos + tokens > s_max or > max_pos.
 */
int llama_layer_prefill(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                        void* k_cache, void* v_cache, int32_t batch, int32_t tokens,
                        int32_t start_pos, int32_t s_max, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * Decode ("Llama2架构与推理全解析" §2.1, §2.4): one new token per sequence.
 *   x        [batch, H] act_dtype;  y [batch, H] act_dtype (no overlap with x)
 *   ctx_len  DEVICE int32 [batch]: tokens already cached for each sequence; the
 *            new token sits at position ctx_len[b], its K/V are written there and
 *            its query attends over positions 0..ctx_len[b].  Read only: the
 *            caller advances it (the cache owner's cur_pos += 1).
 *   max_ctx  HOST int: an upper bound of every ctx_len[b]; sizes the launch.
 *            Device values outside [0, max_ctx] are clamped into it (no fault,
 *            result undefined).
 * Errors: LL_ECACHE_FULL if max_ctx + 1 > s_max or > max_pos.
 */
int llama_layer_decode(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                       void* k_cache, void* v_cache, const int32_t* ctx_len, int32_t batch,
                       int32_t max_ctx, int32_t s_max, void* ws, size_t ws_bytes, void* stream);

/*
 * llama_layer_decode without a workspace argument and without allocating, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments, caches,
 * results and errors as llama_layer_decode (the same kernels, bit-identical
 * outputs).  The workspace is a built-in device array of 64 MiB, one per
 * device, held from the library's first use on that device until the process
 * ends; its address is looked up on the first call on each device.  A call
 * whose workspace, sized for its batch and max_ctx, exceeds 64 MiB returns
 * LL_ESCRATCH before enqueueing anything (e.g. 7B-shaped layers: batch 1 up to
 * 32K contexts; 70B-shaped: batch 32 at 4K).  Every call on a device shares
 * that device's array, so calls that can overlap on one device (different
 * streams, several host threads) race: order them.  The array keeps the last
 * call's contents; the decode needs none of it to start at zero.  Never
 * allocates, frees or synchronises.
 */
int llama_layer_decode_noalloc(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                               void* k_cache, void* v_cache, const int32_t* ctx_len,
                               int32_t batch, int32_t max_ctx, int32_t s_max, void* stream);

/*
 * Paged KV cache ("Llama2架构全景解析" §2.3 and §3.1: paging the KV cache ends
 * fragmentation and lets batch 32 fit where batch 4 ran out of memory;
 * "LLM架构全景解析" §2.2: a memory pool instead of per-request allocation).
 * The cache of every sequence lives in fixed-size blocks of a shared pool:
 *   k_pool, v_pool  DEVICE [n_blocks, n_kv_heads, block_size, head_dim] in
 *                   kv_dtype (one block holds block_size positions of every
 *                   KV head), 16-byte aligned
 *   block_table     DEVICE int32 [batch, max_blocks]: block_table[b][i] is the
 *                   pool block holding positions [i*block_size,
 *                   (i+1)*block_size) of sequence b; entries outside
 *                   [0, n_blocks) are clamped into it (the caller owns the
 *                   table and keeps it valid; the library never reads past
 *                   the pool)
 *   block_size      a power of two in [16, 1024]
 * llama_layer_decode_paged is llama_layer_decode over such a cache: the same
 * arithmetic in the same order, so its results equal the contiguous cache's
 * bit for bit.  A sequence can address max_blocks * block_size positions
 * (max_ctx + 1 must fit; else LL_ECACHE_FULL); the workspace is
 * llama_layer_workspace_size(cfg, batch, 1, max_blocks * block_size).
 */
int llama_layer_decode_paged(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                             void* k_pool, void* v_pool, int32_t n_blocks, int32_t block_size,
                             const int32_t* block_table, int32_t max_blocks,
                             const int32_t* ctx_len, int32_t batch, int32_t max_ctx, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * llama_layer_prefill over a paged cache (arguments as llama_layer_decode_paged
 * and llama_layer_prefill): positions start_pos .. start_pos + tokens - 1 of
 * every sequence are appended through its block table, and attention reads
 * the earlier positions from the pages, so a prompt can be prefilled in
 * chunks.  Results equal llama_layer_prefill's on a contiguous cache bit for
 * bit; the workspace is llama_layer_workspace_size(cfg, batch, tokens,
 * max_blocks * block_size).
 */
int llama_layer_prefill_paged(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                              void* k_pool, void* v_pool, int32_t n_blocks, int32_t block_size,
                              const int32_t* block_table, int32_t max_blocks, int32_t batch,
                              int32_t tokens, int32_t start_pos, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * Copies positions [start, start + count) of every sequence and KV head of
 * contiguous caches k_src, v_src [batch, n_kv_heads, s_max, head_dim] into a
 * paged cache (arguments as above), e.g. after llama_layer_prefill on a
 * contiguous scratch cache.  head_dim * element size must be a multiple of
 * 16 bytes.  Errors: LL_ENULL, LL_EALIGN, LL_EINVAL, LL_ECACHE_FULL
 * (start + count beyond s_max or max_blocks * block_size), LL_EHIP.
 */
int llama_kv_pages_write(const void* k_src, const void* v_src, int32_t s_max, int32_t start,
                         int32_t count, void* k_pool, void* v_pool, int32_t n_blocks,
                         int32_t block_size, const int32_t* block_table, int32_t max_blocks,
                         int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t kv_dtype,
                         void* stream);

/*
 * Weight-only INT8 ("Llama2架构与推理全解析" §3.2: one byte per weight instead
 * of two halves the weight memory at a small loss of precision).  Symmetric
 * round-to-nearest per output row:
 *   scale[r] = max_c |w[r, c]| / 127          (float32)
 *   q[r, c]  = rint(w[r, c] / scale[r])       (float32 division correctly
 *              rounded, ties to even, in [-127, 127]; a zero row: scale 0, q 0)
 *   w        DEVICE [rows, cols] in dtype, 16-byte aligned
 *   q        DEVICE int8 [rows, cols], 16-byte aligned; scale DEVICE float32 [rows]
 * Errors: LL_ENULL, LL_EALIGN, LL_EINVAL (rows or cols <= 0, cols % 16 != 0,
 * bad dtype), LL_EHIP.
 */
int llama_quantize_w8(const void* w, int8_t* q, float* scale, int32_t rows, int32_t cols,
                      int32_t dtype, void* stream);

/*
 * A layer whose seven projection matrices are llama_quantize_w8 codes and
 * scales; the norms and RoPE tables are as in ll_weights.  The layer computes
 * with the weights q[r, c] * scale[r].
 */
typedef struct ll_weights_w8 {
  const void* attn_norm;                       /* [hidden], act_dtype */
  const int8_t *w_q, *w_k, *w_v, *w_o;         /* shapes as in ll_weights */
  const void* ffn_norm;                        /* [hidden], act_dtype */
  const int8_t *w_gate, *w_up, *w_down;
  const float *s_q, *s_k, *s_v, *s_o;          /* float32, one per row of each */
  const float *s_gate, *s_up, *s_down;
  const float *rope_cos, *rope_sin;            /* float32 [max_pos, head_dim/2] */
} ll_weights_w8;

/*
 * llama_layer_decode with INT8 weights: the same arguments, workspace size
 * (llama_layer_workspace_size with tokens = 1), caches and results, the
 * projections reading one byte per weight.  Sequences go through in groups
 * that read every weight once: up to 32 with bf16/f16 activations when
 * hidden, intermediate and n_heads * head_dim are multiples of 64, else up
 * to 4 (fewer when 4 rows of the longest reduction would not fit the 128 KB
 * activation stage).  hidden, intermediate and n_heads * head_dim must be
 * multiples of 16.
 * Errors: as llama_layer_decode; LL_EUNSUPPORTED when a single row of the
 * longest reduction does not fit the stage.
 */
int llama_layer_decode_w8(const ll_config* cfg, const ll_weights_w8* w, const void* x, void* y,
                          void* k_cache, void* v_cache, const int32_t* ctx_len, int32_t batch,
                          int32_t max_ctx, int32_t s_max, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Weight-only INT4 ("Llama2架构与推理全解析" §3.2: about half a byte per
 * weight, a 7B model in roughly 4 GB, at a larger loss of precision than
 * INT8).  The INT8 scheme with 4-bit codes:
 *   scale[r] = max_c |w[r, c]| / 7            (float32)
 *   code     = rint(w[r, c] / scale[r])       (float32 division correctly
 *              rounded, ties to even, in [-7, 7]; a zero row: scale 0, codes 0)
 * packed two to a byte in two's complement nibbles: byte j of a row holds
 * the code of column 2j in its low nibble and of column 2j + 1 in its high one.
 *   w        DEVICE [rows, cols] in dtype, 16-byte aligned
 *   q        DEVICE uint8 [rows, cols / 2], 16-byte aligned; scale DEVICE float32 [rows]
 * Errors: LL_ENULL, LL_EALIGN, LL_EINVAL (rows or cols <= 0, cols % 32 != 0,
 * bad dtype), LL_EHIP.
 */
int llama_quantize_w4(const void* w, uint8_t* q, float* scale, int32_t rows, int32_t cols,
                      int32_t dtype, void* stream);

/*
 * A layer whose seven projection matrices are llama_quantize_w4 codes and
 * scales (rows of cols / 2 bytes); the rest as in ll_weights_w8.  The layer
 * computes with the weights code[r, c] * scale[r].
 */
typedef struct ll_weights_w4 {
  const void* attn_norm;                       /* [hidden], act_dtype */
  const uint8_t *w_q, *w_k, *w_v, *w_o;        /* [rows, cols / 2] packed codes */
  const void* ffn_norm;                        /* [hidden], act_dtype */
  const uint8_t *w_gate, *w_up, *w_down;
  const float *s_q, *s_k, *s_v, *s_o;          /* float32, one per row of each */
  const float *s_gate, *s_up, *s_down;
  const float *rope_cos, *rope_sin;            /* float32 [max_pos, head_dim/2] */
} ll_weights_w4;

/*
 * llama_layer_decode with INT4 weights: the same arguments, workspace size
 * (llama_layer_workspace_size with tokens = 1), caches and results, the
 * projections reading half a byte per weight.  Sequences go through in groups
 * of up to 4 (fewer when 4 rows of the longest reduction would not fit the
 * 128 KB activation stage), each group reading every weight once, so beyond
 * 8 sequences llama_layer_decode_w8 (up to 32 per weight pass) reads fewer
 * bytes.  hidden, intermediate and n_heads * head_dim must be multiples of 32.
 * Errors: as llama_layer_decode; LL_EUNSUPPORTED when a single row of the
 * longest reduction does not fit the stage.
 */
int llama_layer_decode_w4(const ll_config* cfg, const ll_weights_w4* w, const void* x, void* y,
                          void* k_cache, void* v_cache, const int32_t* ctx_len, int32_t batch,
                          int32_t max_ctx, int32_t s_max, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * RoPE angle tables: cos/sin[m, i] = cos/sin(m * rope_theta^(-2i/head_dim)) for
 * m < max_pos, i < head_dim/2, evaluated in float64 on the device and rounded
 * to float32 ("Llama2架构与推理全解析" §1.4).  cos_out, sin_out: device float32
 * [max_pos, head_dim/2].
 */
int llama_rope_table(float* cos_out, float* sin_out, int32_t max_pos, int32_t head_dim,
                     float rope_theta, void* stream);

/*
 * NTK-aware RoPE tables for contexts beyond the trained length
 * ("LLM架构全景解析" §3.1, position-encoding extension): the same tables as
 * llama_rope_table with the base raised to
 *   base' = rope_theta * ntk_scale^(head_dim / (head_dim - 2)),
 * i.e. theta_i' = theta_i * ntk_scale^(-2i/(head_dim - 2)): the fastest pair
 * (i = 0) keeps its frequency and the slowest (i = head_dim/2 - 1) turns
 * ntk_scale times slower, so a context ntk_scale times longer spans the
 * angles the slow pairs covered before.  The layer entry points take these
 * tables unchanged.  ntk_scale = 1 gives llama_rope_table's tables.
 * Errors: LL_ENULL, LL_EINVAL (max_pos <= 0, head_dim odd or < 4,
 * rope_theta <= 1, ntk_scale < 1 or not finite), LL_EHIP.
 */
int llama_rope_table_ntk(float* cos_out, float* sin_out, int32_t max_pos, int32_t head_dim,
                         float rope_theta, float ntk_scale, void* stream);

/*
 * Embedding lookup ("Llama2架构与推理全解析" §2.3): h[i, :] = table[ids[i], :].
 *   table [vocab, hidden] dtype; ids DEVICE int32 [n] (clamped into [0, vocab));
 *   h [n, hidden] dtype.
 */
int llama_embed(const void* table, const int32_t* ids, void* h, int32_t n, int32_t hidden,
                int32_t vocab, int32_t dtype, void* stream);

/*
 * Output head and greedy pick ("Llama2架构与推理全解析" §2.3, §2.5):
 * logits = RMSNorm(h; final_norm, eps) W_lm^T, ids_out[i] = argmax_v logits[i, v]
 * with ties going to the lowest index.
 *   final_norm [hidden], w_lm [vocab, hidden], h [n, hidden]: dtype
 *   ids_out DEVICE int32 [n]; logits DEVICE float32 [n, vocab] (required: it is
 *   also the scratch of the argmax)
 * Errors: LL_EUNSUPPORTED if one row of h does not fit the projection's 48 KB
 * LDS stage (hidden > 24576 for 16-bit formats, > 12288 for float32).
 */
int llama_head_argmax(const void* final_norm, const void* w_lm, const void* h,
                      int32_t* ids_out, float* logits, int32_t n, int32_t hidden,
                      int32_t vocab, float eps, int32_t dtype, void* stream);

/*
 * Token sampling after the LM head ("Llama2架构与推理全解析" §2.5 for the
 * steps, §3.3 for typical settings -- temperature 0.7, top-p 0.9, top-k 50,
 * repetition penalty 1.1; "Llama2架构全景解析" §2.2, step 3, draws from
 * softmax(logits / T)).  For each row r:
 *   1. every distinct id of history[r] lowers its logit: divided by
 *      `penalty` if positive, multiplied by it otherwise (penalty 1: off);
 *   2. z = logit / temperature;
 *   3. top-k keeps the top_k largest z (equal z: lower index first);
 *   4. p = softmax over those;
 *   5. top-p keeps the smallest leading set, in that order, whose mass
 *      reaches top_p (top_p 1: all);
 *   6. ids_out[r] = the first kept token whose cumulative mass exceeds
 *      u[r] times the kept mass (inverse-CDF draw at the caller's uniform).
 * temperature 0 is the greedy limit: the highest penalised logit, lowest
 * index on ties.  Mass sums run in float32.
 *   logits   DEVICE float32 [n, vocab], 4-byte aligned
 *   history  DEVICE int32 [n, n_hist]; ids outside [0, vocab) (e.g. -1
 *            padding) are ignored; may be NULL when n_hist == 0
 *   u        DEVICE float32 [n], uniforms in [0, 1)
 *   ids_out  DEVICE int32 [n]
 * One workgroup per row; nothing is allocated.  n == 0 does nothing.
 * Errors: LL_ENULL, LL_EALIGN, LL_EINVAL (vocab not in [1, 32768], top_k not
 * in [1, 1024], top_p not in (0, 1], temperature < 0 or not finite,
 * penalty <= 0 or not finite, n < 0, n_hist < 0), LL_EHIP.
 */
int llama_sample(const float* logits, const int32_t* history, int32_t n_hist, const float* u,
                 int32_t* ids_out, int32_t n, int32_t vocab, float temperature, int32_t top_k,
                 float top_p, float penalty, void* stream);

/* Static description of an error code. */
const char* llama_layer_strerror(int code);

/*
 * Kernel timing (benchmark instrumentation).  llama_layer_timer_start arms
 * HIP-event pairs for up to max_launches future launches of kernel
 * `kernel_id` (see llama_layer_kernel_name) on whatever stream they are
 * enqueued.  Each pair is handed to the kernel's dispatch (hipExtLaunchKernel),
 * which records its own start and end, so a pair measures that kernel's
 * execution only; where an id covers two kernels (attn_decode: split pass and
 * merge) the first one is timed.  llama_layer_timer_stop waits for those
 * events, writes the summed milliseconds and the number of timed launches, and
 * disarms.  Not thread-safe; creates and destroys HIP events (host-side
 * objects, no device memory).
 */
int llama_layer_timer_start(int32_t kernel_id, int32_t max_launches);
int llama_layer_timer_stop(double* total_ms, int32_t* launches);
/* Name of a kernel id, or NULL past the last one. */
const char* llama_layer_kernel_name(int32_t kernel_id);

/*
 * Measured peaks (benchmark instrumentation, not part of the layer): the rates
 * the layer's roofline fractions are read against, taken on the GPU in use,
 * beside the published 8 TB/s HBM and 2.5 PFLOP/s dense bf16 MFMA.
 *   llama_peak_read       streams `bytes` of src (DEVICE, 16-byte aligned,
 *                         bytes a multiple of 16) once, non-temporal 16-byte
 *                         loads; sink DEVICE uint32 [1024] is written only in
 *                         the practically impossible case that the XOR of all
 *                         the data equals a fixed constant (it keeps the loads
 *                         live).
 *   llama_peak_copy       copies `bytes` from src to dst (DEVICE, 16-byte
 *                         aligned, not overlapping): bytes read + bytes written.
 *   llama_peak_mfma_bf16  back-to-back v_mfma_f32_32x32x16_bf16 on register
 *                         operands, no memory traffic; *flops (HOST) receives
 *                         the work enqueued (iters * 2^28 FLOPs); out
 *                         DEVICE float32 [131072] receives the sums.
 * Time them with events on `stream`.  Errors: LL_ENULL, LL_EALIGN, LL_EINVAL,
 * LL_EHIP.
 */
int llama_peak_read(const void* src, size_t bytes, uint32_t* sink, void* stream);
int llama_peak_copy(void* dst, const void* src, size_t bytes, void* stream);
int llama_peak_mfma_bf16(float* out, int32_t iters, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_LAYER_H */
