"""Seeded synthetic workloads (weights, hidden states, caches, lengths).

This module holds no arithmetic of the decoder layer: it only draws seeded
random numbers, rounds them to a storage format and widens stored values back
to float64.  Both the HIP path's tests/benchmark and the fp64 oracle's tests take
their inputs from here, so the two sides see bit-identical values.

Storage forms: float32 arrays for ``f32``; uint16 bit patterns for ``bf16`` and
``f16`` (round-to-nearest-even from float32).

Recipes (the workloads the pages describe, made synthetic):
  * weights ~ N(0, 0.02) drawn in float32 then rounded; RMSNorm gains = 1;
  * prefill / decode hidden states ~ N(0, 1);
  * KV caches of decode workloads pre-filled with N(0, 1) values, read as keys
    that are already rotated;
  * batched-decode context lengths ~ U{lo .. hi} inclusive;
  * prompt ids ~ U{0 .. vocab-1}.
Seeds: weights of workload k use PCG64(1000 + k), inputs PCG64(2000 + k).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "bf16", "f16")
DTYPE_BYTES = {"f32": 4, "bf16": 2, "f16": 2}


# --------------------------------------------------------------------------
# Storage rounding and widening (format conversion only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_storage(a_f32, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a_f32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a_f32)
    if dtype == "f16":
        return f32_to_f16_bits(a_f32)
    raise ValueError(dtype)


def to_f64(stored, dtype: str) -> np.ndarray:
    """Widen stored values to float64 exactly."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    if dtype == "f16":
        return np.asarray(stored, dtype=np.uint16).view(np.float16).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Shape:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    eps: float = 1e-5
    rope_theta: float = 10000.0

    def as_dict(self):
        return dict(hidden=self.hidden, n_heads=self.n_heads, n_kv_heads=self.n_kv_heads,
                    head_dim=self.head_dim, intermediate=self.intermediate,
                    eps=self.eps, rope_theta=self.rope_theta)


TINY = Shape(256, 4, 2, 64, 688)                 # tiny stack: 2 layers, vocab 512
L7B = Shape(4096, 32, 32, 128, 11008)            # 7B-shaped layer
L13B = Shape(5120, 40, 40, 128, 13824)           # 13B-shaped layer
L70B = Shape(8192, 64, 8, 128, 28672)            # 70B-shaped GQA layer


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: a layer shape, dtypes, a phase and its sizes."""

    name: str
    index: int                 # seed index k: weights PCG64(1000+k), inputs PCG64(2000+k)
    shape: Shape
    act_dtype: str
    kv_dtype: str
    phase: str                 # "prefill" | "decode" | "stack"
    batch: int = 1
    tokens: int = 1            # prefill tokens per sequence
    ctx: int = 0               # decode: tokens already cached (fixed)
    ctx_range: tuple = ()      # decode: (lo, hi) inclusive, drawn per sequence
    s_max: int = 0
    n_layers: int = 1
    vocab: int = 0
    prompt: int = 0
    new_tokens: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny_stack_f32": Workload("tiny_stack_f32", 0, TINY, "f32", "f32", "stack",
                               batch=1, s_max=24, n_layers=2, vocab=512, prompt=16,
                               new_tokens=8),
    "decode_7b_b1_ctx4096": Workload("decode_7b_b1_ctx4096", 1, L7B, "bf16", "bf16", "decode",
                                     batch=1, ctx=4096, s_max=4097),
    "prefill_13b_t4096": Workload("prefill_13b_t4096", 2, L13B, "bf16", "bf16", "prefill",
                                  batch=1, tokens=4096, s_max=4096),
    "decode_70b_b32_ragged": Workload("decode_70b_b32_ragged", 3, L70B, "bf16", "f16", "decode",
                                      batch=32, ctx_range=(512, 4096), s_max=4097),
    "stack_70b_80l": Workload("stack_70b_80l", 4, L70B, "bf16", "bf16", "stack",
                              batch=1, s_max=1152, n_layers=80, vocab=32000, prompt=1024,
                              new_tokens=128),
}


# --------------------------------------------------------------------------
# Draws
# --------------------------------------------------------------------------

WEIGHT_STD = 0.02
LAYER_TENSORS = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")


def layer_tensor_shapes(s: Shape) -> dict:
    H, nh, nkv, hd, I = s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate
    return {"w_q": (nh * hd, H), "w_k": (nkv * hd, H), "w_v": (nkv * hd, H),
            "w_o": (H, nh * hd), "w_gate": (I, H), "w_up": (I, H), "w_down": (H, I)}


def normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def draw_layer(rng: np.random.Generator, s: Shape, dtype: str) -> dict:
    """One layer's weights in storage form; gains are ones."""
    out = {}
    for name, shp in layer_tensor_shapes(s).items():
        out[name] = to_storage(normal(rng, shp, WEIGHT_STD), dtype)
    ones = np.ones(s.hidden, dtype=np.float32)
    out["attn_norm"] = to_storage(ones, dtype)
    out["ffn_norm"] = to_storage(ones, dtype)
    return out


def weights_rng(k: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 + k))


def inputs_rng(k: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(2000 + k))


def draw_stack(w: Workload) -> dict:
    """Tiny/large stack: layers, embedding table, final gain, LM head, prompt."""
    rng = weights_rng(w.index)
    layers = [draw_layer(rng, w.shape, w.act_dtype) for _ in range(w.n_layers)]
    embed = to_storage(normal(rng, (w.vocab, w.shape.hidden), WEIGHT_STD), w.act_dtype)
    w_lm = to_storage(normal(rng, (w.vocab, w.shape.hidden), WEIGHT_STD), w.act_dtype)
    final_norm = to_storage(np.ones(w.shape.hidden, np.float32), w.act_dtype)
    prompt = inputs_rng(w.index).integers(0, w.vocab, size=w.prompt, dtype=np.int64)
    return dict(layers=layers, embed=embed, w_lm=w_lm, final_norm=final_norm,
                prompt=prompt.astype(np.int32))


def draw_decode_inputs(rng: np.random.Generator, s: Shape, batch: int, s_max: int,
                       act_dtype: str, kv_dtype: str, ctx=None, ctx_range=None) -> dict:
    """Hidden states x[B, H], per-sequence lengths and pre-filled caches."""
    if ctx_range:
        lo, hi = ctx_range
        ctx_len = rng.integers(lo, hi + 1, size=batch, dtype=np.int64).astype(np.int32)
    else:
        ctx_len = np.full(batch, ctx, dtype=np.int32)
    x = to_storage(normal(rng, (batch, s.hidden)), act_dtype)
    cshape = (batch, s.n_kv_heads, s_max, s.head_dim)
    k_cache = to_storage(normal(rng, cshape), kv_dtype)
    v_cache = to_storage(normal(rng, cshape), kv_dtype)
    return dict(x=x, ctx_len=ctx_len, k_cache=k_cache, v_cache=v_cache)


def draw_prefill_inputs(rng: np.random.Generator, s: Shape, batch: int, tokens: int,
                        s_max: int, act_dtype: str, kv_dtype: str, start_pos: int = 0) -> dict:
    """Hidden states x[B, T, H]; caches pre-filled with N(0,1) before start_pos
    (zeros elsewhere)."""
    x = to_storage(normal(rng, (batch, tokens, s.hidden)), act_dtype)
    cshape = (batch, s.n_kv_heads, s_max, s.head_dim)
    kc = np.zeros(cshape, dtype=np.float32)
    vc = np.zeros(cshape, dtype=np.float32)
    if start_pos:
        kc[:, :, :start_pos] = normal(rng, (batch, s.n_kv_heads, start_pos, s.head_dim))
        vc[:, :, :start_pos] = normal(rng, (batch, s.n_kv_heads, start_pos, s.head_dim))
    return dict(x=x, k_cache=to_storage(kc, kv_dtype), v_cache=to_storage(vc, kv_dtype),
                start_pos=start_pos)


def workload_layer_and_inputs(name: str) -> tuple:
    """(weights, inputs) of a single-layer workload, in storage form."""
    w = WORKLOADS[name]
    weights = draw_layer(weights_rng(w.index), w.shape, w.act_dtype)
    rng = inputs_rng(w.index)
    if w.phase == "decode":
        inputs = draw_decode_inputs(rng, w.shape, w.batch, w.s_max, w.act_dtype, w.kv_dtype,
                                    ctx=w.ctx, ctx_range=w.ctx_range)
    elif w.phase == "prefill":
        inputs = draw_prefill_inputs(rng, w.shape, w.batch, w.tokens, w.s_max,
                                     w.act_dtype, w.kv_dtype)
    else:
        raise ValueError(f"{name} is not a single-layer workload")
    return weights, inputs
