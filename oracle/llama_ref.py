"""fp64 CPU oracle of the Llama-2 decoder layer (prefill and KV-cached decode).

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, calls or links this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may use it.  It shares no code, constant or helper with the
HIP path; it consumes plain float64 NumPy arrays (the exact values the GPU sees,
widened without modification) and returns float64 arrays.

Sources (four web pages, cited by title and section):
  * "Llama2架构全景解析" -- devpress.csdn.net; its §1.1 gives pre-norm RMSNorm,
    the RoPE complex form f(q, m) = (W_q x_m) * e^{i m theta} and SwiGLU; its
    §1.2 the GQA grouping (8 query heads share one K/V head for 70B).
  * "Llama2架构与推理全解析：从原理到KV Cache与量化部署" -- sheratonhq.com; §1.2
    RMSNorm, §1.3 SwiGLU, §1.4 RoPE, §1.5 GQA, §1.6 the size table, §2.1
    prefill/decode, §2.3 the per-layer recipe and residual stream, §2.4 the KV
    cache and its size formula, §2.5 greedy decoding, §3.1 weight memory.
  * "LLM架构全景解析：从基础模块到工程实践" -- intelliparadigm.com; §2.2 the
    append-only cache object, §3.2 max subtraction before softmax.

Readings taken where the pages are silent or garbled (each is listed, with the
reason, in the design notes): eps sits inside the square root; theta_i =
rope_theta^(-2i/head_dim); RoPE rotates adjacent pairs (2i, 2i+1); positions are
0-based; V is not rotated and the cache stores K after RoPE; scores are scaled by
1/sqrt(head_dim); query head h reads KV head floor(h / (n_heads/n_kv_heads));
key tau is visible to a query at position m iff tau <= m; greedy ties go to the
lowest index; the LM head is applied to the last position only.

Pins (tests/test_oracle_*.py, all CPU):
  rmsnorm         closed form rms(u) = sqrt(ms/(ms+eps)) with gamma = 1, scale
                  invariance, row independence, torch.nn.functional.rms_norm.
  rope            norm preservation, identity at m = 0, dot products depend only
                  on m - n, head_dim = 2 equals complex multiplication by
                  e^{i m theta_0}, an independent complex-number evaluation.
  attention       brute-force double loop with an explicit mask, single key gives
                  v_0, future perturbation leaves earlier rows unchanged, constant
                  V gives that constant, torch scaled_dot_product_attention
                  (is_causal, enable_gqa), MHA equivalences for GQA/MQA.
  swiglu_ffn      silu closed forms, W_gate = 0 gives zero, torch silu.
  layer_prefill   transformers' LlamaDecoderLayer in float64 (RoPE layouts
                  related by a fixed row permutation of W_q/W_k).
  layer_decode    prefill(T) then k decodes equals prefill(T + k).
  embed           one-hot rows times the table.
  lm_head         a hand-worked two-row example (final gain, eps inside the
                  root, untied W_lm), torch rms_norm followed by a linear layer.
  greedy/stack    argmax lowest-index tie break; with no layers, generation is
                  the head alone on the prompt's last token and then on each
                  previous id (torch); cached generation equals
                  full-recompute generation.
  quantize_w8     the round-to-nearest bound |w - q s| <= s/2, the largest
                  magnitude on +-127, sign symmetry, exact re-quantisation of
                  dequantised rows, zero rows.
  sample          a hand-worked 4-token example (temperature, top-k, top-p,
                  penalty), inverse-CDF counts over a grid of u, the greedy
                  limits (T -> 0, top-k = 1), transformers' logits processors.
  sizes           the pages' KV-cache formula and printed sizes (tests/golden).
No function here is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F64 = np.float64


@dataclass(frozen=True)
class LayerConfig:
    """Hyper-parameter names as the size table of "Llama2架构与推理全解析" §1.6
    and the hidden/intermediate discussion of §1.3 use them."""

    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    eps: float
    rope_theta: float

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads


@dataclass
class LayerWeights:
    """One layer's parameters, float64, stored [out, in] (y = x @ W.T).

    The pages write the products as x·W with W as [in, out]; storing the
    transpose is the same mathematics.
    """

    attn_norm: np.ndarray  # [hidden]
    w_q: np.ndarray        # [n_heads*head_dim, hidden]
    w_k: np.ndarray        # [n_kv_heads*head_dim, hidden]
    w_v: np.ndarray        # [n_kv_heads*head_dim, hidden]
    w_o: np.ndarray        # [hidden, n_heads*head_dim]
    ffn_norm: np.ndarray   # [hidden]
    w_gate: np.ndarray     # [intermediate, hidden]
    w_up: np.ndarray       # [intermediate, hidden]
    w_down: np.ndarray     # [hidden, intermediate]


# --------------------------------------------------------------------------
# Step definitions
# --------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each token vector ("Llama2架构与推理全解析" §1.2).

    The mean of squares is taken over the last (hidden) axis of each token on
    its own -- never across tokens or the batch -- eps is added inside the
    square root, and the result is scaled by the learned gain gamma.
    """
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=F64)


def rope_inv_freq(head_dim: int, rope_theta: float) -> np.ndarray:
    """theta_i = rope_theta^(-2i/head_dim), i = 0 .. head_dim/2 - 1.

    The pages only say each dimension pair turns at its own preset frequency,
    fast for some and slow for others ("Llama2架构与推理全解析" §1.4); this is
    the standard family that the NTK base-scaling rule of "LLM架构全景解析"
    §3.1 presupposes.
    """
    i = np.arange(head_dim // 2, dtype=F64)
    return np.power(F64(rope_theta), -2.0 * i / head_dim)


def ntk_rope_base(rope_theta: float, ntk_scale: float, head_dim: int) -> float:
    """RoPE base for a context ntk_scale times the trained one, by the
    NTK-aware rule of "LLM架构全景解析" §3.1 (position-encoding extension): the
    base is multiplied by ntk_scale^(dim/(dim-2)), dim being the rotated
    dimension of a head.  With this base, rope() and every layer function
    apply the extended encoding unchanged.
    """
    d = F64(head_dim)
    return F64(rope_theta) * np.power(F64(ntk_scale), d / (d - 2.0))


def rope(z: np.ndarray, positions: np.ndarray, rope_theta: float) -> np.ndarray:
    """Rotate adjacent pairs (2i, 2i+1) of every head by angle m * theta_i.

    "Llama2架构全景解析" §1.1 writes the encoding as multiplication by
    e^{i m theta}; "Llama2架构与推理全解析" §1.4 groups the dimensions two by two
    as points in a plane and rotates each by a position-dependent angle.

    z: [T, heads, head_dim]; positions: [T] absolute (0-based) positions.
    """
    z = np.asarray(z, dtype=F64)
    hd = z.shape[-1]
    ang = np.asarray(positions, dtype=F64)[:, None] * rope_inv_freq(hd, rope_theta)[None, :]
    c = np.cos(ang)[:, None, :]  # [T, 1, hd/2]
    s = np.sin(ang)[:, None, :]
    a = z[..., 0::2]
    b = z[..., 1::2]
    out = np.empty_like(z)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """Softmax with the row maximum subtracted first ("LLM架构全景解析" §3.2)."""
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def causal_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         q_pos: np.ndarray) -> np.ndarray:
    """Scaled dot-product causal attention with grouped K/V heads.

    q: [T, n_heads, hd] at absolute positions q_pos[T]; k, v: [S, n_kv_heads, hd]
    holding keys/values for positions 0 .. S-1.  Scores are q.k / sqrt(hd);
    keys later than the query's own position get -inf; softmax; weighted sum of
    V ("Llama2架构与推理全解析" §2.3).  Query head h uses KV head
    floor(h / group): consecutive query heads share one K/V head
    ("Llama2架构全景解析" §1.2, "Llama2架构与推理全解析" §1.5).
    Returns o: [T, n_heads, hd].
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    T, nh, hd = q.shape
    S, nkv, _ = k.shape
    g = nh // nkv
    key_pos = np.arange(S)
    visible = key_pos[None, :] <= np.asarray(q_pos)[:, None]  # [T, S]
    o = np.empty((T, nh, hd), dtype=F64)
    for h in range(nh):
        j = h // g
        s = (q[:, h, :] @ k[:, j, :].T) / np.sqrt(F64(hd))
        s = np.where(visible, s, -np.inf)
        o[:, h, :] = softmax(s, axis=-1) @ v[:, j, :]
    return o


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) ("Llama2架构与推理全解析" §1.3)."""
    z = np.asarray(z, dtype=F64)
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(u: np.ndarray, w: LayerWeights) -> np.ndarray:
    """(silu(u W_gate) * (u W_up)) W_down ("Llama2架构与推理全解析" §1.3)."""
    a = silu(u @ w.w_gate.T) * (u @ w.w_up.T)
    return a @ w.w_down.T


# --------------------------------------------------------------------------
# The layer
# --------------------------------------------------------------------------

def _layer_one_sequence(cfg: LayerConfig, w: LayerWeights, x: np.ndarray,
                        k_cache: np.ndarray, v_cache: np.ndarray, start_pos: int,
                        out_rows=None) -> np.ndarray:
    """One pre-norm decoder layer for one sequence of T new tokens.

    x: [T, hidden] at positions start_pos .. start_pos+T-1.  k_cache / v_cache:
    [n_kv_heads, S_max, head_dim], updated in place: the new K (after RoPE) and
    V are appended at their positions, earlier entries are read as they are
    ("Llama2架构与推理全解析" §2.4; the cache object of "LLM架构全景解析" §2.2).
    Steps follow "Llama2架构与推理全解析" §2.3: h = x + attn(rmsnorm(x)), then
    out = h + ffn(rmsnorm(h)).  If out_rows is given only those rows of the
    output are computed (the K/V of every row are still appended).
    """
    x = np.asarray(x, dtype=F64)
    T = x.shape[0]
    nh, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    pos = start_pos + np.arange(T)

    u = rmsnorm(x, w.attn_norm, cfg.eps)
    q = (u @ w.w_q.T).reshape(T, nh, hd)
    k = (u @ w.w_k.T).reshape(T, nkv, hd)
    v = (u @ w.w_v.T).reshape(T, nkv, hd)
    q = rope(q, pos, cfg.rope_theta)
    k = rope(k, pos, cfg.rope_theta)
    k_cache[:, pos, :] = k.transpose(1, 0, 2)
    v_cache[:, pos, :] = v.transpose(1, 0, 2)

    rows = np.arange(T) if out_rows is None else np.asarray(out_rows)
    S = start_pos + T
    keys = k_cache[:, :S, :].transpose(1, 0, 2)
    vals = v_cache[:, :S, :].transpose(1, 0, 2)
    o = causal_gqa_attention(q[rows], keys, vals, pos[rows])
    h1 = x[rows] + o.reshape(len(rows), nh * hd) @ w.w_o.T
    u2 = rmsnorm(h1, w.ffn_norm, cfg.eps)
    return h1 + swiglu_ffn(u2, w)


def layer_prefill(cfg: LayerConfig, w: LayerWeights, x: np.ndarray,
                  k_cache: np.ndarray, v_cache: np.ndarray, start_pos: int,
                  out_rows=None) -> np.ndarray:
    """Prefill: all T prompt tokens of each sequence at once
    ("Llama2架构与推理全解析" §2.1).

    x: [B, T, hidden]; caches [B, n_kv_heads, S_max, head_dim] (updated in
    place).  Returns out [B, T, hidden] (or [B, len(out_rows), hidden]).
    """
    x = np.asarray(x, dtype=F64)
    return np.stack([
        _layer_one_sequence(cfg, w, x[b], k_cache[b], v_cache[b], start_pos, out_rows)
        for b in range(x.shape[0])
    ])


def layer_decode(cfg: LayerConfig, w: LayerWeights, x: np.ndarray,
                 k_cache: np.ndarray, v_cache: np.ndarray,
                 ctx_len: np.ndarray) -> np.ndarray:
    """Decode: one new token per sequence at position ctx_len[b]; only its K/V
    are computed and appended, and its query attends over the whole cache
    ("Llama2架构与推理全解析" §2.1, §2.4; "Llama2架构全景解析" §2.2).

    x: [B, hidden]; ctx_len[B] = tokens already cached for sequence b.
    Returns out [B, hidden].
    """
    x = np.asarray(x, dtype=F64)
    return np.stack([
        _layer_one_sequence(cfg, w, x[b:b + 1], k_cache[b], v_cache[b], int(ctx_len[b]))[0]
        for b in range(x.shape[0])
    ])


# --------------------------------------------------------------------------
# Stack glue: embedding, output head, greedy decoding
# --------------------------------------------------------------------------

def embed(table: np.ndarray, ids) -> np.ndarray:
    """Row lookup in the vocab x hidden table ("Llama2架构与推理全解析" §2.3)."""
    return np.asarray(table, dtype=F64)[np.asarray(ids, dtype=np.int64)]


def lm_head(h: np.ndarray, final_norm: np.ndarray, w_lm: np.ndarray, eps: float) -> np.ndarray:
    """logits = rmsnorm(h) @ W_lm.T with W_lm separate from the embedding table
    ("Llama2架构与推理全解析" §2.3)."""
    return rmsnorm(h, final_norm, eps) @ np.asarray(w_lm, dtype=F64).T


def greedy(logits: np.ndarray) -> np.ndarray:
    """Pick the highest-scoring token; ties go to the lowest index
    ("Llama2架构与推理全解析" §2.5)."""
    return np.argmax(np.asarray(logits), axis=-1)


def quantize_w8_rows(w):
    """Weight-only INT8 by rows ("Llama2架构与推理全解析" §3.2: one byte per
    weight instead of two, with a small loss of precision).

    Reading: symmetric round-to-nearest per output row, the scale being the
    row's largest magnitude over 127; codes = rint(w / scale) clipped to
    [-127, 127] (ties to even), an all-zero row gets scale 0 and codes 0.  The
    scale and the division are taken in float32, the precision of the kernel,
    so that both sides pick the same integer codes.

    w: [rows, cols] (values exactly representable in float32).
    Returns (codes int8 [rows, cols], scales float32 [rows]).
    """
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(w32 / safe[:, None])
    q = np.where(scale[:, None] > 0, np.clip(q, -127, 127), 0)
    return q.astype(np.int8), scale


def dequantize_w8(codes, scales) -> np.ndarray:
    """The weights an INT8 layer computes with: codes times the row scale, in
    float64 (exact: an 8-bit integer times a float32 scale)."""
    return np.asarray(codes, dtype=F64) * np.asarray(scales, dtype=F64)[:, None]


def quantize_w4_rows(w):
    """Weight-only INT4 by rows ("Llama2架构与推理全解析" §3.2: about half a byte
    per weight, so a 7B model in roughly 4 GB, at a larger loss of precision
    than INT8).

    Reading: the INT8 scheme with 4-bit codes.  Symmetric round-to-nearest per
    output row, the scale being the row's largest magnitude over 7; codes =
    rint(w / scale) clipped to [-7, 7] (ties to even); an all-zero row gets
    scale 0 and codes 0.  Scale and division in float32, as for INT8.  How the
    codes are packed two to a byte is a storage layout, not part of this
    definition.

    w: [rows, cols] (values exactly representable in float32).
    Returns (codes int8 [rows, cols] in [-7, 7], scales float32 [rows]).
    """
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    scale = (amax / np.float32(7.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(w32 / safe[:, None])
    q = np.where(scale[:, None] > 0, np.clip(q, -7, 7), 0)
    return q.astype(np.int8), scale


def dequantize_w4(codes, scales) -> np.ndarray:
    """The weights an INT4 layer computes with: codes times the row scale, in
    float64 (exact)."""
    return np.asarray(codes, dtype=F64) * np.asarray(scales, dtype=F64)[:, None]


def sampling_distribution(logits, history, temperature: float, top_k: int, top_p: float,
                          penalty: float):
    """The distribution one token is drawn from ("Llama2架构与推理全解析" §2.5;
    "Llama2架构全景解析" §2.2, step 3, draws from softmax(logits / T)).

    Steps in the pages' order: the repetition penalty lowers every token that
    already occurred (a positive logit is divided by `penalty`, a negative
    one multiplied, once per distinct id); the logits are divided by the
    temperature; top-k keeps the k largest; softmax over those; top-p keeps
    the smallest leading set, in decreasing probability, whose mass reaches
    top_p.  Equal values are ordered by lower index first.

    logits: [V]; history: ids already seen (entries < 0 ignored).
    Returns (ids, probs): the kept tokens in that order and their
    renormalised probabilities.
    """
    z = np.array(logits, dtype=F64)
    seen = np.unique([int(t) for t in np.asarray(history).ravel() if 0 <= int(t) < z.shape[0]])
    for t in seen:
        z[t] = z[t] / penalty if z[t] > 0 else z[t] * penalty
    z = z / temperature
    order = np.lexsort((np.arange(z.shape[0]), -z))  # decreasing z, then increasing index
    order = order[:top_k]
    e = np.exp(z[order] - z[order[0]])
    p = e / np.sum(e)
    cum_before = np.concatenate(([0.0], np.cumsum(p)[:-1]))
    keep = cum_before < top_p  # stop after the token whose mass reaches top_p
    ids, p = order[keep], p[keep]
    return ids, p / np.sum(p)


def sample(logits, history, u, temperature: float, top_k: int, top_p: float,
           penalty: float) -> np.ndarray:
    """One token per row: draw from sampling_distribution by the inverse of its
    cumulative distribution at the given uniform u in [0, 1) (multinomial
    sampling with the random number passed in).  temperature 0 is the greedy
    limit: the highest penalised logit, lowest index on ties.

    logits: [n, V]; history: [n, n_hist]; u: [n].
    """
    logits = np.asarray(logits, dtype=F64)
    out = np.empty(logits.shape[0], dtype=np.int64)
    for r in range(logits.shape[0]):
        hist = history[r] if history is not None else []
        if temperature == 0:
            ids, _ = sampling_distribution(logits[r], hist, 1.0, 1, 1.0, penalty)
            out[r] = ids[0]
            continue
        ids, p = sampling_distribution(logits[r], hist, temperature, top_k, top_p, penalty)
        c = np.cumsum(p)
        i = int(np.searchsorted(c, float(u[r]), side="right"))  # first i with c[i] > u
        out[r] = ids[min(i, len(ids) - 1)]
    return out


def generate_greedy(cfg: LayerConfig, layers, embed_table, final_norm, w_lm,
                    prompt_ids, n_new: int, s_max: int):
    """Prefill the prompt once, then n_new single-token decode steps
    ("Llama2架构与推理全解析" §3.4 and §2.6).

    Batch 1.  Returns (ids, logits): 1 + n_new greedy ids (the first comes from
    the prefill's last position) and the logits that chose each.
    """
    prompt_ids = np.asarray(prompt_ids, dtype=np.int64)
    T = prompt_ids.shape[0]
    caches = [(np.zeros((1, cfg.n_kv_heads, s_max, cfg.head_dim)),
               np.zeros((1, cfg.n_kv_heads, s_max, cfg.head_dim))) for _ in layers]
    h = embed(embed_table, prompt_ids)[None]  # [1, T, H]
    for w, (kc, vc) in zip(layers, caches):
        h = layer_prefill(cfg, w, h, kc, vc, 0)
    logits = [lm_head(h[0, -1], final_norm, w_lm, cfg.eps)]
    ids = [int(greedy(logits[-1]))]
    for step in range(n_new):
        h = embed(embed_table, [ids[-1]])  # [1, H]
        ctx = np.array([T + step])
        for w, (kc, vc) in zip(layers, caches):
            h = layer_decode(cfg, w, h, kc, vc, ctx)
        logits.append(lm_head(h[0], final_norm, w_lm, cfg.eps))
        ids.append(int(greedy(logits[-1])))
    return np.array(ids), np.stack(logits)


# --------------------------------------------------------------------------
# Sizes
# --------------------------------------------------------------------------

def kv_cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int, seq_len: int,
                   bytes_per_elem: int) -> int:
    """K and V copies x layers x KV heads x head_dim x positions x element size
    ("Llama2架构与推理全解析" §2.4)."""
    return 2 * n_layers * n_kv_heads * head_dim * seq_len * bytes_per_elem


def layer_param_count(cfg: LayerConfig) -> int:
    """Parameters of one layer: Q/K/V/O projections, gate/up/down, two gains."""
    H, nh, nkv, hd, I = cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate
    return H * nh * hd + 2 * H * nkv * hd + nh * hd * H + 3 * H * I + 2 * H


def model_param_count(cfg: LayerConfig, n_layers: int, vocab: int) -> int:
    """Layers plus an untied embedding table and LM head plus the final gain
    ("Llama2架构与推理全解析" §2.3 notes the head is not tied to the table)."""
    return n_layers * layer_param_count(cfg) + 2 * vocab * cfg.hidden + cfg.hidden
