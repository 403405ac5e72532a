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

    def generate_greedy(self, prompt_ids: torch.Tensor, n_new: int, s_max: int,
                        return_logits: bool = False):
        """Batch 1.  prompt_ids: int32 device tensor [T].  Returns (ids [1+n_new]
        on the host, logits [1+n_new, vocab] float32 on the device or None)."""
        cfg = self.cfg
        dev = prompt_ids.device
        act = B.TORCH_DTYPE[cfg.act_dtype]
        kvt = B.TORCH_DTYPE[cfg.kv_dtype]
        H, T = cfg.hidden, int(prompt_ids.numel())
        if T + n_new > s_max:
            raise ValueError("prompt + new tokens exceed the cache capacity")
        caches = [(torch.zeros(1, cfg.n_kv_heads, s_max, cfg.head_dim, dtype=kvt, device=dev),
                   torch.zeros(1, cfg.n_kv_heads, s_max, cfg.head_dim, dtype=kvt, device=dev))
                  for _ in self.layers]
        ws = torch.empty(max(B.llama_layer_workspace_size(cfg, 1, T, s_max),
                             B.llama_layer_workspace_size(cfg, 1, 1, s_max)),
                         dtype=torch.uint8, device=dev)
        h = torch.empty(T, H, dtype=act, device=dev)
        h2 = torch.empty_like(h)
        B.llama_embed(self.embed, prompt_ids, h, T, H, self.vocab, act)
        for w, (kc, vc) in zip(self.layers, caches):
            B.llama_layer_prefill(cfg, w, h, h2, kc, vc, 1, T, 0, s_max, ws)
            h, h2 = h2, h
        ids = torch.empty(1 + n_new, dtype=torch.int32, device=dev)
        logits = torch.empty(1 + n_new, self.vocab, dtype=torch.float32, device=dev)
        B.llama_head_argmax(self.final_norm, self.w_lm, h[T - 1:], ids[0:1], logits[0:1], 1, H,
                            self.vocab, cfg.eps, act)
        x = torch.empty(1, H, dtype=act, device=dev)
        y = torch.empty_like(x)
        ctx = torch.empty(n_new, dtype=torch.int32, device=dev)
        ctx.copy_(torch.arange(T, T + n_new, dtype=torch.int32))
        for step in range(n_new):
            B.llama_embed(self.embed, ids[step:step + 1], x, 1, H, self.vocab, act)
            for w, (kc, vc) in zip(self.layers, caches):
                B.llama_layer_decode(cfg, w, x, y, kc, vc, ctx[step:step + 1], 1, T + step,
                                     s_max, ws)
                x, y = y, x
            B.llama_head_argmax(self.final_norm, self.w_lm, x, ids[step + 1:step + 2],
                                logits[step + 1:step + 2], 1, H, self.vocab, cfg.eps, act)
        return ids.cpu().numpy(), (logits if return_logits else None)
