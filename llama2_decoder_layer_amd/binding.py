"""ctypes binding of libllama_layer.so (include/llama_layer.h).

Argument marshalling only: torch tensors become device pointers, Python ints
become C ints, the current torch stream becomes the hipStream_t.  Every step of
the layer runs in the library's HIP kernels; there is no fallback.  The library
is opened after torch so that it binds to the HIP runtime torch already loaded
(one runtime per process: the stream and pointers are shared).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libllama_layer.so")

LL_F32, LL_BF16, LL_F16 = 0, 1, 2
DTYPE_CODE = {"f32": LL_F32, "bf16": LL_BF16, "f16": LL_F16,
              torch.float32: LL_F32, torch.bfloat16: LL_BF16, torch.float16: LL_F16}
TORCH_DTYPE = {LL_F32: torch.float32, LL_BF16: torch.bfloat16, LL_F16: torch.float16}

ERRORS = {0: "LL_OK", -1: "LL_EINVAL", -2: "LL_ENULL", -3: "LL_EALIGN", -4: "LL_ECACHE_FULL",
          -5: "LL_EWORKSPACE", -6: "LL_EHIP", -7: "LL_EUNSUPPORTED", -8: "LL_ESCRATCH"}


class LlamaLayerError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({llama_layer_strerror(code)})")


class ll_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("max_pos", ctypes.c_int32)]


class ll_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "w_q", "w_k", "w_v", "w_o", "ffn_norm", "w_gate", "w_up",
                 "w_down", "rope_cos", "rope_sin")]


class ll_weights_w8(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "w_q", "w_k", "w_v", "w_o", "ffn_norm", "w_gate", "w_up",
                 "w_down", "s_q", "s_k", "s_v", "s_o", "s_gate", "s_up", "s_down",
                 "rope_cos", "rope_sin")]


class ll_weights_w4(ll_weights_w8):
    """Same fields as ll_weights_w8; the w_* point to packed int4 rows."""


_lib = None


def lib() -> ctypes.CDLL:
    """Open the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m llama2_decoder_layer_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        CP = ctypes.POINTER(ll_config)
        WP = ctypes.POINTER(ll_weights)
        L.llama_layer_workspace_size.argtypes = [CP, I32, I32, I32]
        L.llama_layer_workspace_size.restype = SZ
        L.llama_layer_prefill.argtypes = [CP, WP, P, P, P, P, I32, I32, I32, I32, P, SZ, P]
        L.llama_layer_prefill.restype = ctypes.c_int
        L.llama_layer_decode.argtypes = [CP, WP, P, P, P, P, P, I32, I32, I32, P, SZ, P]
        L.llama_layer_decode.restype = ctypes.c_int
        L.llama_layer_decode_noalloc.argtypes = [CP, WP, P, P, P, P, P, I32, I32, I32, P]
        L.llama_layer_decode_noalloc.restype = ctypes.c_int
        L.llama_rope_table.argtypes = [P, P, I32, I32, F, P]
        L.llama_rope_table.restype = ctypes.c_int
        L.llama_rope_table_ntk.argtypes = [P, P, I32, I32, F, F, P]
        L.llama_rope_table_ntk.restype = ctypes.c_int
        L.llama_sample.argtypes = [P, P, I32, P, P, I32, I32, F, I32, F, F, P]
        L.llama_sample.restype = ctypes.c_int
        L.llama_layer_decode_paged.argtypes = [CP, WP, P, P, P, P, I32, I32, P, I32, P, I32, I32,
                                               P, SZ, P]
        L.llama_layer_decode_paged.restype = ctypes.c_int
        L.llama_layer_prefill_paged.argtypes = [CP, WP, P, P, P, P, I32, I32, P, I32, I32, I32,
                                                I32, P, SZ, P]
        L.llama_layer_prefill_paged.restype = ctypes.c_int
        L.llama_kv_pages_write.argtypes = [P, P, I32, I32, I32, P, P, I32, I32, P, I32, I32, I32,
                                           I32, I32, P]
        L.llama_kv_pages_write.restype = ctypes.c_int
        L.llama_quantize_w8.argtypes = [P, P, P, I32, I32, I32, P]
        L.llama_quantize_w8.restype = ctypes.c_int
        L.llama_layer_decode_w8.argtypes = [CP, ctypes.POINTER(ll_weights_w8), P, P, P, P, P,
                                            I32, I32, I32, P, SZ, P]
        L.llama_layer_decode_w8.restype = ctypes.c_int
        L.llama_quantize_w4.argtypes = [P, P, P, I32, I32, I32, P]
        L.llama_quantize_w4.restype = ctypes.c_int
        L.llama_layer_decode_w4.argtypes = [CP, ctypes.POINTER(ll_weights_w4), P, P, P, P, P,
                                            I32, I32, I32, P, SZ, P]
        L.llama_layer_decode_w4.restype = ctypes.c_int
        L.llama_embed.argtypes = [P, P, P, I32, I32, I32, I32, P]
        L.llama_embed.restype = ctypes.c_int
        L.llama_head_argmax.argtypes = [P, P, P, P, P, I32, I32, I32, F, I32, P]
        L.llama_head_argmax.restype = ctypes.c_int
        L.llama_peak_read.argtypes = [P, SZ, P, P]
        L.llama_peak_read.restype = ctypes.c_int
        L.llama_peak_copy.argtypes = [P, P, SZ, P]
        L.llama_peak_copy.restype = ctypes.c_int
        L.llama_peak_mfma_bf16.argtypes = [P, I32, ctypes.POINTER(ctypes.c_double), P]
        L.llama_peak_mfma_bf16.restype = ctypes.c_int
        L.llama_layer_strerror.argtypes = [ctypes.c_int]
        L.llama_layer_strerror.restype = ctypes.c_char_p
        L.llama_layer_timer_start.argtypes = [I32, I32]
        L.llama_layer_timer_start.restype = ctypes.c_int
        L.llama_layer_timer_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32)]
        L.llama_layer_timer_stop.restype = ctypes.c_int
        L.llama_layer_kernel_name.argtypes = [I32]
        L.llama_layer_kernel_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise LlamaLayerError(rc, what)


# --------------------------------------------------------------------------
# Structures
# --------------------------------------------------------------------------

def make_config(hidden, n_heads, n_kv_heads, head_dim, intermediate, eps, rope_theta,
                act_dtype, kv_dtype, max_pos) -> ll_config:
    return ll_config(hidden, n_heads, n_kv_heads, head_dim, intermediate, eps, rope_theta,
                     DTYPE_CODE[act_dtype], DTYPE_CODE[kv_dtype], max_pos)


class LayerWeights:
    """Holds one layer's device tensors (keeping them alive) and their ll_weights."""

    NAMES = ("attn_norm", "w_q", "w_k", "w_v", "w_o", "ffn_norm", "w_gate", "w_up", "w_down",
             "rope_cos", "rope_sin")

    def __init__(self, tensors: dict):
        self.tensors = dict(tensors)
        self.struct = ll_weights(*[_ptr(self.tensors[n]) for n in self.NAMES])


# --------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# --------------------------------------------------------------------------

def llama_layer_workspace_size(cfg: ll_config, batch: int, tokens: int, s_max: int) -> int:
    return int(lib().llama_layer_workspace_size(ctypes.byref(cfg), batch, tokens, s_max))


def llama_layer_prefill(cfg, weights: LayerWeights, x, y, k_cache, v_cache, batch, tokens,
                        start_pos, s_max, ws, ws_bytes=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    rc = lib().llama_layer_prefill(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x),
                                   _ptr(y), _ptr(k_cache), _ptr(v_cache), batch, tokens,
                                   start_pos, s_max, _ptr(ws), nbytes, _stream(stream))
    _check(rc, "llama_layer_prefill")


def llama_layer_decode(cfg, weights: LayerWeights, x, y, k_cache, v_cache, ctx_len, batch,
                       max_ctx, s_max, ws, ws_bytes=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    rc = lib().llama_layer_decode(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x),
                                  _ptr(y), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), batch,
                                  max_ctx, s_max, _ptr(ws), nbytes, _stream(stream))
    _check(rc, "llama_layer_decode")


def llama_layer_decode_noalloc(cfg, weights: LayerWeights, x, y, k_cache, v_cache, ctx_len, batch,
                               max_ctx, s_max, stream=None) -> None:
    """llama_layer_decode with the library's built-in device scratch (no
    workspace argument, nothing allocated)."""
    rc = lib().llama_layer_decode_noalloc(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x),
                                          _ptr(y), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len),
                                          batch, max_ctx, s_max, _stream(stream))
    _check(rc, "llama_layer_decode_noalloc")


class LayerWeightsW8:
    """Holds an INT8 layer's device tensors (codes, scales, norms, RoPE tables)
    and their ll_weights_w8."""

    NAMES = tuple(n for n, _ in ll_weights_w8._fields_)

    def __init__(self, tensors: dict):
        self.tensors = dict(tensors)
        self.struct = ll_weights_w8(*[_ptr(self.tensors[n]) for n in self.NAMES])


class LayerWeightsW4:
    """Holds an INT4 layer's device tensors (packed codes, scales, norms, RoPE
    tables) and their ll_weights_w4."""

    NAMES = tuple(n for n, _ in ll_weights_w8._fields_)

    def __init__(self, tensors: dict):
        self.tensors = dict(tensors)
        self.struct = ll_weights_w4(*[_ptr(self.tensors[n]) for n in self.NAMES])


def llama_layer_decode_paged(cfg, weights: LayerWeights, x, y, k_pool, v_pool, block_size,
                             block_table, ctx_len, batch, max_ctx, ws, ws_bytes=None,
                             stream=None) -> None:
    """k_pool, v_pool [n_blocks, n_kv_heads, block_size, head_dim]; block_table
    [batch, max_blocks] int32; all device tensors."""
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    rc = lib().llama_layer_decode_paged(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x),
                                        _ptr(y), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
                                        block_size, _ptr(block_table), block_table.shape[1],
                                        _ptr(ctx_len), batch, max_ctx, _ptr(ws), nbytes,
                                        _stream(stream))
    _check(rc, "llama_layer_decode_paged")


def llama_layer_prefill_paged(cfg, weights: LayerWeights, x, y, k_pool, v_pool, block_size,
                              block_table, batch, tokens, start_pos, ws, ws_bytes=None,
                              stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    rc = lib().llama_layer_prefill_paged(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x),
                                         _ptr(y), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
                                         block_size, _ptr(block_table), block_table.shape[1],
                                         batch, tokens, start_pos, _ptr(ws), nbytes,
                                         _stream(stream))
    _check(rc, "llama_layer_prefill_paged")


def llama_kv_pages_write(k_src, v_src, start, count, k_pool, v_pool, block_size, block_table,
                         kv_dtype, stream=None) -> None:
    """k_src, v_src [batch, n_kv_heads, s_max, head_dim] into the pools."""
    batch, nkv, s_max, hd = k_src.shape
    _check(lib().llama_kv_pages_write(_ptr(k_src), _ptr(v_src), s_max, start, count, _ptr(k_pool),
                                      _ptr(v_pool), k_pool.shape[0], block_size,
                                      _ptr(block_table), block_table.shape[1], batch, nkv, hd,
                                      DTYPE_CODE[kv_dtype], _stream(stream)),
           "llama_kv_pages_write")


def llama_quantize_w8(w, q, scale, dtype, stream=None) -> None:
    """w [rows, cols] device tensor stored in `dtype`; q int8 and scale float32 outputs."""
    rows, cols = w.shape
    _check(lib().llama_quantize_w8(_ptr(w), _ptr(q), _ptr(scale), rows, cols, DTYPE_CODE[dtype],
                                   _stream(stream)), "llama_quantize_w8")


def llama_quantize_w4(w, q, scale, dtype, stream=None) -> None:
    """w [rows, cols] device tensor stored in `dtype`; q uint8 [rows, cols/2]
    (packed codes) and scale float32 outputs."""
    rows, cols = w.shape
    _check(lib().llama_quantize_w4(_ptr(w), _ptr(q), _ptr(scale), rows, cols, DTYPE_CODE[dtype],
                                   _stream(stream)), "llama_quantize_w4")


def llama_layer_decode_w4(cfg, weights: LayerWeightsW4, x, y, k_cache, v_cache, ctx_len, batch,
                          max_ctx, s_max, ws, ws_bytes=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    rc = lib().llama_layer_decode_w4(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x),
                                     _ptr(y), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), batch,
                                     max_ctx, s_max, _ptr(ws), nbytes, _stream(stream))
    _check(rc, "llama_layer_decode_w4")


def llama_layer_decode_w8(cfg, weights: LayerWeightsW8, x, y, k_cache, v_cache, ctx_len, batch,
                          max_ctx, s_max, ws, ws_bytes=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    rc = lib().llama_layer_decode_w8(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x),
                                     _ptr(y), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), batch,
                                     max_ctx, s_max, _ptr(ws), nbytes, _stream(stream))
    _check(rc, "llama_layer_decode_w8")


def llama_rope_table(cos, sin, max_pos, head_dim, rope_theta, stream=None) -> None:
    _check(lib().llama_rope_table(_ptr(cos), _ptr(sin), max_pos, head_dim, rope_theta,
                                  _stream(stream)), "llama_rope_table")


def llama_sample(logits, history, u, ids_out, temperature, top_k, top_p, penalty,
                 stream=None) -> None:
    """logits [n, vocab] float32, history [n, n_hist] int32 or None, u [n]
    float32, ids_out [n] int32; all device tensors."""
    n, vocab = logits.shape
    n_hist = 0 if history is None else history.shape[1]
    _check(lib().llama_sample(_ptr(logits), _ptr(history) if n_hist else None, n_hist, _ptr(u),
                              _ptr(ids_out), n, vocab, temperature, top_k, top_p, penalty,
                              _stream(stream)), "llama_sample")


def llama_rope_table_ntk(cos, sin, max_pos, head_dim, rope_theta, ntk_scale, stream=None) -> None:
    _check(lib().llama_rope_table_ntk(_ptr(cos), _ptr(sin), max_pos, head_dim, rope_theta,
                                      ntk_scale, _stream(stream)), "llama_rope_table_ntk")


def llama_embed(table, ids, h, n, hidden, vocab, dtype, stream=None) -> None:
    _check(lib().llama_embed(_ptr(table), _ptr(ids), _ptr(h), n, hidden, vocab,
                             DTYPE_CODE[dtype], _stream(stream)), "llama_embed")


def llama_head_argmax(final_norm, w_lm, h, ids_out, logits, n, hidden, vocab, eps, dtype,
                      stream=None) -> None:
    _check(lib().llama_head_argmax(_ptr(final_norm), _ptr(w_lm), _ptr(h), _ptr(ids_out),
                                   _ptr(logits), n, hidden, vocab, eps, DTYPE_CODE[dtype],
                                   _stream(stream)), "llama_head_argmax")


def llama_layer_strerror(code: int) -> str:
    return lib().llama_layer_strerror(code).decode()


def llama_layer_timer_start(kernel_id: int, max_launches: int) -> None:
    _check(lib().llama_layer_timer_start(kernel_id, max_launches), "llama_layer_timer_start")


def llama_layer_timer_stop() -> tuple:
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    _check(lib().llama_layer_timer_stop(ctypes.byref(ms), ctypes.byref(n)), "llama_layer_timer_stop")
    return ms.value, n.value


def llama_layer_kernel_name(kernel_id: int):
    r = lib().llama_layer_kernel_name(kernel_id)
    return None if r is None else r.decode()


def kernel_id(name: str) -> int:
    i = 0
    while True:
        n = llama_layer_kernel_name(i)
        if n is None:
            raise KeyError(name)
        if n == name:
            return i
        i += 1


def llama_peak_read(src, sink, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    _check(lib().llama_peak_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "llama_peak_read")


def llama_peak_copy(dst, src, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    _check(lib().llama_peak_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)), "llama_peak_copy")


def llama_peak_mfma_bf16(out, iters: int, stream=None) -> float:
    """Enqueues the MFMA loop; returns the FLOPs it performs."""
    fl = ctypes.c_double()
    _check(lib().llama_peak_mfma_bf16(_ptr(out), iters, ctypes.byref(fl), _stream(stream)),
           "llama_peak_mfma_bf16")
    return fl.value
