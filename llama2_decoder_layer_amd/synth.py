"""Seeded synthetic workloads (weights, hidden states, caches, lengths).

This module holds no arithmetic of the decoder layer: it only draws seeded
random numbers, rounds them to a storage format and widens stored values back
to float64.  Both the HIP path's tests/benchmark and the fp64 oracle's tests take
their inputs from here, so the two sides see bit-identical values.

Storage forms: float32 arrays for ``f32``; uint16 bit patterns for ``bf16`` and
``f16`` (round-to-nearest-even from float32).

Recipes (the workloads the pages describe, made synthetic):
  * weights ~ N(0, 0.02) drawn in float32 then rounded; RMSNorm gains = 1 in
    the benchmark workloads, and 1 + 0.3 N(0, 1) (rounded the same way) where
    a parity case asks for learned gains;
  * prefill / decode hidden states ~ N(0, 1);
  * KV caches of decode workloads pre-filled with N(0, 1) values, read as keys
    that are already rotated;
  * batched-decode context lengths ~ U{lo .. hi} inclusive;
  * prompt ids ~ U{0 .. vocab-1}.
Seeds: weights of workload k descend from SeedSequence(1000 + k), inputs from
SeedSequence(2000 + k) (one child per tensor, one grandchild per 4 Mi elements).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
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
    index: int                 # seed index k: weights 1000+k, inputs 2000+k
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
    # Long-context decode with the NTK-aware RoPE base: a 4K-trained 7B layer
    # stretched 8x to a 32K cache.
    "decode_7b_b1_ctx32768_ntk8": Workload("decode_7b_b1_ctx32768_ntk8", 5, L7B, "bf16", "bf16",
                                           "decode", batch=1, ctx=32768, s_max=32769,
                                           extra={"ntk_scale": 8.0}),
    # The 70B batch-32 decode over a paged cache: 64-position blocks of one
    # pool, in shuffled order (same weights, input and lengths as the
    # contiguous workload: seed index 3).
    "decode_70b_b32_ragged_paged": Workload("decode_70b_b32_ragged_paged", 3, L70B, "bf16", "f16",
                                            "decode", batch=32, ctx_range=(512, 4096), s_max=4097,
                                            extra={"block_size": 64}),
    # The 70B batch-32 decode with INT8 projections (same weights, input and
    # lengths as the bf16 workload: seed index 3).
    "decode_70b_b32_ragged_w8": Workload("decode_70b_b32_ragged_w8", 3, L70B, "bf16", "f16",
                                         "decode", batch=32, ctx_range=(512, 4096), s_max=4097,
                                         extra={"w8": True}),
    # The 7B decode with weight-only INT8 projections (codes and scales made
    # on the device from the bf16 weights).
    "decode_7b_b1_ctx4096_w8": Workload("decode_7b_b1_ctx4096_w8", 7, L7B, "bf16", "bf16",
                                        "decode", batch=1, ctx=4096, s_max=4097,
                                        extra={"w8": True}),
    # The same 7B decode with weight-only INT4 projections (same weights and
    # inputs as the INT8 one: seed index 7).
    "decode_7b_b1_ctx4096_w4": Workload("decode_7b_b1_ctx4096_w4", 7, L7B, "bf16", "bf16",
                                        "decode", batch=1, ctx=4096, s_max=4097,
                                        extra={"w4": True}),
    # Sampling after the LM head: 32 rows of a 32000-token vocabulary with the
    # pages' dialogue settings and 256 previous ids per row.
    "sample_b32_v32000": Workload("sample_b32_v32000", 6, L70B, "f32", "f32", "sample",
                                  batch=32, vocab=32000,
                                  extra={"temperature": 0.7, "top_k": 50, "top_p": 0.9,
                                         "penalty": 1.1, "n_hist": 256}),
    "stack_70b_80l": Workload("stack_70b_80l", 4, L70B, "bf16", "bf16", "stack",
                              batch=1, s_max=1152, n_layers=80, vocab=32000, prompt=1024,
                              new_tokens=128),
}


# --------------------------------------------------------------------------
# Draws
# --------------------------------------------------------------------------
# Every tensor gets its own child of the workload's SeedSequence, and every
# 4 Mi-element chunk of it a grandchild, so large tensors are drawn by a thread
# pool and the values do not depend on the number of threads.

WEIGHT_STD = 0.02
GAIN_STD = 0.3             # learned gains: 1 + GAIN_STD * N(0, 1)
LAYER_TENSORS = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")
CHUNK = 1 << 22
STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def layer_tensor_shapes(s: Shape) -> dict:
    H, nh, nkv, hd, I = s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate
    return {"w_q": (nh * hd, H), "w_k": (nkv * hd, H), "w_v": (nkv * hd, H),
            "w_o": (H, nh * hd), "w_gate": (I, H), "w_up": (I, H), "w_down": (H, I)}


def normal(ss: np.random.SeedSequence, shape, std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """N(0, std^2) drawn in float32 and rounded to `dtype` storage."""
    out = np.empty(shape, dtype=STORAGE[dtype])
    flat = out.reshape(-1)
    n = flat.size
    nch = max(1, (n + CHUNK - 1) // CHUNK)
    kids = ss.spawn(nch)

    def work(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        a = np.random.Generator(np.random.PCG64(kids[i])).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        flat[lo:hi] = to_storage(a, dtype)

    if nch == 1:
        work(0)
    else:
        with cf.ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(work, range(nch)))
    return out


def draw_gain(ss: np.random.SeedSequence, hidden: int, dtype: str) -> np.ndarray:
    """A learned RMSNorm gain, 1 + GAIN_STD * N(0, 1), drawn in float32 and
    rounded to `dtype` storage."""
    g = np.random.Generator(np.random.PCG64(ss)).standard_normal(hidden, dtype=np.float32)
    return to_storage(np.float32(1.0) + np.float32(GAIN_STD) * g, dtype)


def draw_layer(ss: np.random.SeedSequence, s: Shape, dtype: str,
               learned_gains: bool = False) -> dict:
    """One layer's weights in storage form.  Gains are ones, or with
    learned_gains two independent draws of draw_gain (the projection weights
    are the same either way: the gains take the next two children)."""
    shapes = layer_tensor_shapes(s)
    kids = ss.spawn(len(LAYER_TENSORS))
    out = {name: normal(kid, shapes[name], WEIGHT_STD, dtype)
           for name, kid in zip(LAYER_TENSORS, kids)}
    if learned_gains:
        k_attn, k_ffn = ss.spawn(2)
        out["attn_norm"] = draw_gain(k_attn, s.hidden, dtype)
        out["ffn_norm"] = draw_gain(k_ffn, s.hidden, dtype)
    else:
        ones = np.ones(s.hidden, dtype=np.float32)
        out["attn_norm"] = to_storage(ones, dtype)
        out["ffn_norm"] = to_storage(ones, dtype)
    return out


def weights_seed(k: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(1000 + k)


def inputs_seed(k: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(2000 + k)


def draw_prompt(w: Workload) -> np.ndarray:
    """Prompt ids ~ U{0 .. vocab-1}, int32."""
    rng = np.random.Generator(np.random.PCG64(inputs_seed(w.index)))
    return rng.integers(0, w.vocab, size=w.prompt, dtype=np.int64).astype(np.int32)


def draw_stack(w: Workload, learned_gains: bool = False) -> dict:
    """Stack: layers, embedding table, final gain, LM head and the prompt.
    learned_gains draws every RMSNorm gain (the final one included) with
    draw_gain instead of ones; the other tensors are unchanged."""
    ss = weights_seed(w.index)
    kids = ss.spawn(w.n_layers + 2)
    layers = [draw_layer(kids[i], w.shape, w.act_dtype, learned_gains) for i in range(w.n_layers)]
    embed = normal(kids[w.n_layers], (w.vocab, w.shape.hidden), WEIGHT_STD, w.act_dtype)
    w_lm = normal(kids[w.n_layers + 1], (w.vocab, w.shape.hidden), WEIGHT_STD, w.act_dtype)
    if learned_gains:
        final_norm = draw_gain(ss.spawn(1)[0], w.shape.hidden, w.act_dtype)
    else:
        final_norm = to_storage(np.ones(w.shape.hidden, np.float32), w.act_dtype)
    return dict(layers=layers, embed=embed, w_lm=w_lm, final_norm=final_norm,
                prompt=draw_prompt(w))


# --------------------------------------------------------------------------
# Device-side draws.  The 80-layer stack holds ~140 GB of weights: they are
# drawn where they live, by torch's device generator (Philox, counter based)
# keyed by (seed, tensor id), in float32 and rounded to the storage format
# (round to nearest even).  Tests that check a layer copy its values back.
# --------------------------------------------------------------------------
DEVICE_TENSOR_IDS = 16        # ids per layer; the embedding and LM head follow the layers


def device_normal(seed: int, tensor_id: int, shape, std: float, dtype: str, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * (1 << 20) + tensor_id)
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=g)
    if dtype == "f32":
        return t
    return t.to({"bf16": torch.bfloat16, "f16": torch.float16}[dtype])


def device_gain(seed: int, tensor_id: int, hidden: int, dtype: str, device="cuda"):
    """A learned gain drawn on the device: 1 + GAIN_STD * N(0, 1) in float32
    from the (seed, tensor id) stream, rounded to the storage format."""
    import torch
    g = device_normal(seed, tensor_id, (hidden,), GAIN_STD, "f32", device) + 1.0
    if dtype == "f32":
        return g
    return g.to({"bf16": torch.bfloat16, "f16": torch.float16}[dtype])


def draw_stack_device(w: Workload, device="cuda", learned_gains: bool = False) -> dict:
    """The stack drawn on the device: layers (dicts of tensors), embedding
    table, final gain and LM head; the prompt stays a host array.  Gains are
    ones, or with learned_gains device_gain draws (tensor ids 7 and 8 of each
    layer, the final one after the LM head)."""
    import torch
    seed = 1000 + w.index
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.act_dtype]
    shapes = layer_tensor_shapes(w.shape)
    H = w.shape.hidden

    def gain(tid):
        if learned_gains:
            return device_gain(seed, tid, H, w.act_dtype, device)
        return torch.ones(H, dtype=tdt, device=device)

    layers = []
    for l in range(w.n_layers):
        d = {name: device_normal(seed, l * DEVICE_TENSOR_IDS + i, shapes[name], WEIGHT_STD,
                                 w.act_dtype, device)
             for i, name in enumerate(LAYER_TENSORS)}
        d["attn_norm"] = gain(l * DEVICE_TENSOR_IDS + len(LAYER_TENSORS))
        d["ffn_norm"] = gain(l * DEVICE_TENSOR_IDS + len(LAYER_TENSORS) + 1)
        layers.append(d)
    base = w.n_layers * DEVICE_TENSOR_IDS
    embed = device_normal(seed, base, (w.vocab, H), WEIGHT_STD, w.act_dtype, device)
    w_lm = device_normal(seed, base + 1, (w.vocab, H), WEIGHT_STD, w.act_dtype, device)
    final_norm = gain(base + 2)
    return dict(layers=layers, embed=embed, w_lm=w_lm, final_norm=final_norm,
                prompt=draw_prompt(w))


def draw_decode_inputs(ss: np.random.SeedSequence, s: Shape, batch: int, s_max: int,
                       act_dtype: str, kv_dtype: str, ctx=None, ctx_range=None) -> dict:
    """Hidden states x[B, H], per-sequence lengths and pre-filled caches."""
    k_len, k_x, k_k, k_v = ss.spawn(4)
    if ctx_range:
        lo, hi = ctx_range
        rng = np.random.Generator(np.random.PCG64(k_len))
        ctx_len = rng.integers(lo, hi + 1, size=batch, dtype=np.int64).astype(np.int32)
    else:
        ctx_len = np.full(batch, ctx, dtype=np.int32)
    x = normal(k_x, (batch, s.hidden), 1.0, act_dtype)
    cshape = (batch, s.n_kv_heads, s_max, s.head_dim)
    return dict(x=x, ctx_len=ctx_len, k_cache=normal(k_k, cshape, 1.0, kv_dtype),
                v_cache=normal(k_v, cshape, 1.0, kv_dtype))


def draw_prefill_inputs(ss: np.random.SeedSequence, s: Shape, batch: int, tokens: int,
                        s_max: int, act_dtype: str, kv_dtype: str, start_pos: int = 0) -> dict:
    """Hidden states x[B, T, H]; caches hold N(0,1) at positions < start_pos and
    zeros elsewhere."""
    k_x, k_k, k_v = ss.spawn(3)
    x = normal(k_x, (batch, tokens, s.hidden), 1.0, act_dtype)
    cshape = (batch, s.n_kv_heads, s_max, s.head_dim)
    kc = np.zeros(cshape, dtype=STORAGE[kv_dtype])
    vc = np.zeros(cshape, dtype=STORAGE[kv_dtype])
    if start_pos:
        pshape = (batch, s.n_kv_heads, start_pos, s.head_dim)
        kc[:, :, :start_pos] = normal(k_k, pshape, 1.0, kv_dtype)
        vc[:, :, :start_pos] = normal(k_v, pshape, 1.0, kv_dtype)
    return dict(x=x, k_cache=kc, v_cache=vc, start_pos=start_pos)


def draw_sample_inputs(name: str) -> dict:
    """Logits [B, V] ~ 3 N(0, 1) in float32, previous ids U{0..V-1} and the
    uniforms the draw consumes, for a sampling workload."""
    w = WORKLOADS[name]
    k_l, k_h, k_u = inputs_seed(w.index).spawn(3)
    logits = normal(k_l, (w.batch, w.vocab), 3.0, "f32")
    hist = np.random.Generator(np.random.PCG64(k_h)).integers(
        0, w.vocab, (w.batch, w.extra["n_hist"]), dtype=np.int64).astype(np.int32)
    u = np.random.Generator(np.random.PCG64(k_u)).random(w.batch).astype(np.float32)
    return dict(logits=np.asarray(logits, np.float32), history=hist, u=u)


def workload_layer_and_inputs(name: str) -> tuple:
    """(weights, inputs) of a single-layer workload, in storage form."""
    w = WORKLOADS[name]
    weights = draw_layer(weights_seed(w.index), w.shape, w.act_dtype)
    ss = inputs_seed(w.index)
    if w.phase == "decode":
        inputs = draw_decode_inputs(ss, w.shape, w.batch, w.s_max, w.act_dtype, w.kv_dtype,
                                    ctx=w.ctx, ctx_range=w.ctx_range)
    elif w.phase == "prefill":
        inputs = draw_prefill_inputs(ss, w.shape, w.batch, w.tokens, w.s_max,
                                     w.act_dtype, w.kv_dtype)
    else:
        raise ValueError(f"{name} is not a single-layer workload")
    return weights, inputs
