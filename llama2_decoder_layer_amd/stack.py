"""Greedy generation over a stack of layers, driven through the C ABI.

Prefill the prompt once, then one decode step per new token
("Llama2架构与推理全解析" §3.4, §2.6): embedding -> every layer -> final
RMSNorm + LM head -> argmax, with each layer's KV cache advanced by one
position per step.  The token ids stay on the device until the end; the host
only enqueues work.
"""
from __future__ import annotations

import torch

from . import binding as B


class Stack:
    """Device-resident layers plus the embedding table, final gain and LM head.

    layers: list of binding.LayerWeights sharing one ll_config `cfg`.
    """

    def __init__(self, cfg, layers, embed, final_norm, w_lm, vocab: int):
        self.cfg = cfg
        self.layers = layers
        self.embed = embed
        self.final_norm = final_norm
        self.w_lm = w_lm
        self.vocab = vocab

    def begin(self, prompt_ids: torch.Tensor, n_new: int, s_max: int) -> "Generation":
        """Allocate the caches and buffers of one batch-1 generation."""
        return Generation(self, prompt_ids, n_new, s_max)

    def generate_greedy(self, prompt_ids: torch.Tensor, n_new: int, s_max: int,
                        return_logits: bool = False):
        """Batch 1.  prompt_ids: int32 device tensor [T].  Returns (ids [1+n_new]
        on the host, logits [1+n_new, vocab] float32 on the device or None)."""
        g = self.begin(prompt_ids, n_new, s_max)
        g.prefill()
        for step in range(n_new):
            g.decode(step)
        return g.ids.cpu().numpy(), (g.logits if return_logits else None)


class Generation:
    """State of one generation: per-layer KV caches, workspace, the ids and
    logits produced so far.  `capture` (a set of layer indices) keeps copies of
    those layers' input and output hidden states, keyed (phase, layer), where
    phase is "prefill" or the decode step."""

    def __init__(self, stack: Stack, prompt_ids: torch.Tensor, n_new: int, s_max: int):
        cfg = stack.cfg
        self.stack, self.prompt, self.n_new, self.s_max = stack, prompt_ids, n_new, s_max
        dev = prompt_ids.device
        act = B.TORCH_DTYPE[cfg.act_dtype]
        kvt = B.TORCH_DTYPE[cfg.kv_dtype]
        H, T = cfg.hidden, int(prompt_ids.numel())
        if T + n_new > s_max:
            raise ValueError("prompt + new tokens exceed the cache capacity")
        self.T = T
        self.caches = [(torch.zeros(1, cfg.n_kv_heads, s_max, cfg.head_dim, dtype=kvt, device=dev),
                        torch.zeros(1, cfg.n_kv_heads, s_max, cfg.head_dim, dtype=kvt, device=dev))
                       for _ in stack.layers]
        self.ws = torch.empty(max(B.llama_layer_workspace_size(cfg, 1, T, s_max),
                                  B.llama_layer_workspace_size(cfg, 1, 1, s_max)),
                              dtype=torch.uint8, device=dev)
        self.h = torch.empty(T, H, dtype=act, device=dev)
        self.h2 = torch.empty_like(self.h)
        self.x = torch.empty(1, H, dtype=act, device=dev)
        self.y = torch.empty_like(self.x)
        self.ids = torch.empty(1 + n_new, dtype=torch.int32, device=dev)
        self.logits = torch.empty(1 + n_new, stack.vocab, dtype=torch.float32, device=dev)
        self.ctx = torch.arange(T, T + max(n_new, 1), dtype=torch.int32).to(dev)
        self.captured = {}

    def prefill(self, capture=()):
        """Embed the prompt, run every layer over it and pick the first id."""
        st, cfg, T = self.stack, self.stack.cfg, self.T
        h, h2 = self.h, self.h2
        B.llama_embed(st.embed, self.prompt, h, T, cfg.hidden, st.vocab, B.TORCH_DTYPE[cfg.act_dtype])
        for l, (w, (kc, vc)) in enumerate(zip(st.layers, self.caches)):
            B.llama_layer_prefill(cfg, w, h, h2, kc, vc, 1, T, 0, self.s_max, self.ws)
            if l in capture:
                self.captured[("prefill", l)] = (h.clone(), h2.clone())
            h, h2 = h2, h
        B.llama_head_argmax(st.final_norm, st.w_lm, h[T - 1:], self.ids[0:1], self.logits[0:1], 1,
                            cfg.hidden, st.vocab, cfg.eps, B.TORCH_DTYPE[cfg.act_dtype])
        self.last_hidden = h[T - 1:]

    def decode(self, step: int, capture=()):
        """Feed ids[step] at position T + step and pick ids[step + 1]."""
        st, cfg = self.stack, self.stack.cfg
        act = B.TORCH_DTYPE[cfg.act_dtype]
        x, y = self.x, self.y
        B.llama_embed(st.embed, self.ids[step:step + 1], x, 1, cfg.hidden, st.vocab, act)
        for l, (w, (kc, vc)) in enumerate(zip(st.layers, self.caches)):
            B.llama_layer_decode(cfg, w, x, y, kc, vc, self.ctx[step:step + 1], 1, self.T + step,
                                 self.s_max, self.ws)
            if l in capture:
                self.captured[(step, l)] = (x.clone(), y.clone())
            x, y = y, x
        B.llama_head_argmax(st.final_norm, st.w_lm, x, self.ids[step + 1:step + 2],
                            self.logits[step + 1:step + 2], 1, cfg.hidden, st.vocab, cfg.eps, act)
        self.last_hidden = x


def device_stack(shape, act: str, kv: str, max_pos: int, drawn: dict) -> Stack:
    """A Stack over device tensors: drawn = dict(layers=[{name: tensor}], embed,
    final_norm, w_lm) with the layer tensor names of binding.LayerWeights (the
    RoPE tables are built here, once, and shared by every layer)."""
    cfg = B.make_config(shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                        shape.intermediate, shape.eps, shape.rope_theta, act, kv, max_pos)
    dev = drawn["embed"].device
    rc = torch.empty(max_pos, shape.head_dim // 2, dtype=torch.float32, device=dev)
    rs = torch.empty_like(rc)
    B.llama_rope_table(rc, rs, max_pos, shape.head_dim, shape.rope_theta)
    layers = [B.LayerWeights({**d, "rope_cos": rc, "rope_sin": rs}) for d in drawn["layers"]]
    return Stack(cfg, layers, drawn["embed"], drawn["final_norm"], drawn["w_lm"],
                 int(drawn["embed"].shape[0]))
