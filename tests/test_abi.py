"""The C ABI on the host: the library loads, exports every declared entry point,
and rejects bad arguments with the documented codes before touching the GPU
(every call below fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest

from llama2_decoder_layer_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llama_layer.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(llama_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert "llama_layer_prefill" in names and "llama_layer_decode" in names
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_one_hip_runtime_in_process():
    B.lib()
    maps = open("/proc/self/maps").read().splitlines()
    hip = {m.split()[-1] for m in maps if "libamdhip64" in m}
    assert len(hip) == 1, hip


def test_strerror():
    assert B.llama_layer_strerror(0) == "ok"
    for code in range(-8, 0):
        assert B.llama_layer_strerror(code) != "unknown error"
    assert B.llama_layer_strerror(-99) == "unknown error"


def test_kernel_names():
    names = []
    i = 0
    while B.llama_layer_kernel_name(i) is not None:
        names.append(B.llama_layer_kernel_name(i))
        i += 1
    assert {"gemv_qkv", "gemv_gate_up", "gemm_qkv", "attn_decode", "attn_prefill",
            "sample"} <= set(names)


FAKE = 0x7F0000000000  # never dereferenced: every call here fails validation first


def cfg(**kw):
    base = dict(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=688, eps=1e-5,
                rope_theta=1e4, act_dtype="bf16", kv_dtype="bf16", max_pos=64)
    base.update(kw)
    return B.make_config(**base)


def weights(**kw):
    ptrs = {n: FAKE + 256 * i for i, n in enumerate(B.LayerWeights.NAMES)}
    ptrs.update(kw)
    w = B.LayerWeights.__new__(B.LayerWeights)
    w.tensors = {}
    w.struct = B.ll_weights(*[ptrs[n] for n in B.LayerWeights.NAMES])
    return w


def prefill_rc(c, w=None, x=FAKE + 0x100000, y=FAKE + 0x200000, kc=FAKE + 0x300000,
               vc=FAKE + 0x400000, batch=1, tokens=8, start_pos=0, s_max=32, ws=FAKE + 0x500000,
               ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = 1  # too small: the last check, reached only if everything else passes
    w = w or weights()
    return B.lib().llama_layer_prefill(ctypes.byref(c), ctypes.byref(w.struct), x, y, kc, vc,
                                       batch, tokens, start_pos, s_max, ws, ws_bytes, None)


def decode_rc(c, w=None, x=FAKE + 0x100000, y=FAKE + 0x200000, kc=FAKE + 0x300000,
              vc=FAKE + 0x400000, ctx=FAKE + 0x600000, batch=2, max_ctx=10, s_max=32,
              ws=FAKE + 0x500000, ws_bytes=1):
    w = w or weights()
    return B.lib().llama_layer_decode(ctypes.byref(c), ctypes.byref(w.struct), x, y, kc, vc, ctx,
                                      batch, max_ctx, s_max, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,code", [
    (dict(n_kv_heads=3), -1),          # n_heads % n_kv_heads != 0
    (dict(hidden=250), -1),            # hidden not a multiple of 8
    (dict(intermediate=690), -1),
    (dict(head_dim=96), -7),           # unsupported head_dim
    (dict(head_dim=63), -1),           # odd head_dim
    (dict(eps=0.0), -1),
    (dict(rope_theta=1.0), -1),
    (dict(act_dtype="f32", kv_dtype="bf16"), -1),
    (dict(act_dtype="bf16", kv_dtype="f32"), -1),
    (dict(max_pos=0), -1),
])
def test_bad_config(bad, code):
    c = cfg(**bad)
    assert prefill_rc(c) == code
    assert decode_rc(c) == code
    assert B.llama_layer_workspace_size(c, 1, 8, 32) == 0


def test_null_and_alignment():
    c = cfg()
    assert prefill_rc(c, x=None) == -2
    assert prefill_rc(c, w=weights(w_o=None)) == -2
    assert prefill_rc(c, w=weights(rope_cos=None)) == -2
    assert prefill_rc(c, y=FAKE + 0x200008) == -3
    assert prefill_rc(c, w=weights(w_down=FAKE + 4)) == -3
    assert decode_rc(c, ctx=None) == -2
    assert decode_rc(c, ctx=FAKE + 0x600002) == -3
    assert decode_rc(c, ctx=FAKE + 0x600004) == -5   # 4-byte aligned lengths are fine
    assert B.lib().llama_layer_prefill(None, ctypes.byref(weights().struct), FAKE, FAKE, FAKE,
                                       FAKE, 1, 1, 0, 8, FAKE, 1, None) == -2


def test_sizes_and_cache_capacity():
    c = cfg()
    assert prefill_rc(c, batch=0) == -1
    assert prefill_rc(c, tokens=0) == -1
    assert prefill_rc(c, start_pos=-1) == -1
    assert prefill_rc(c, start_pos=30, tokens=3, s_max=32) == -4
    assert prefill_rc(c, start_pos=29, tokens=3, s_max=32) == -5   # fits: workspace is next
    assert prefill_rc(cfg(max_pos=16), tokens=17, s_max=32) == -4  # past the RoPE table
    assert decode_rc(c, max_ctx=32, s_max=32) == -4   # the new token would sit at 32
    assert decode_rc(c, max_ctx=31, s_max=32) == -5
    assert decode_rc(cfg(max_pos=20), max_ctx=20, s_max=32) == -4
    assert decode_rc(c, batch=0) == -1
    assert decode_rc(c, max_ctx=-1) == -1


def test_overlap_and_workspace():
    c = cfg()
    x = FAKE + 0x100000
    assert prefill_rc(c, x=x, y=x + 16) == -1          # y overlaps x
    need = B.llama_layer_workspace_size(c, 1, 8, 32)
    assert need > 0
    assert prefill_rc(c, ws=None) == -5
    assert prefill_rc(c, ws=FAKE + 0x500008) == -3
    assert prefill_rc(c, ws_bytes=need - 1) == -5
    dneed = B.llama_layer_workspace_size(c, 2, 1, 32)
    assert decode_rc(c, ws_bytes=dneed - 1) == -5


def test_workspace_grows_with_work():
    # Within one plan (token-skinny: <= 32 tokens per pass; wide: whole-prompt
    # GEMMs) more tokens or a longer cache need more workspace.  The two plans
    # hold different buffers, so the size is not monotonic across the boundary.
    c = cfg()
    ws = B.llama_layer_workspace_size
    assert ws(c, 1, 128, 128) > ws(c, 1, 64, 128)      # wide
    assert ws(c, 1, 8, 128) > ws(c, 1, 2, 128)         # skinny
    assert ws(c, 1, 1, 4096) > ws(c, 1, 1, 64)


def test_glue_validation():
    L = B.lib()
    assert L.llama_rope_table(None, FAKE, 8, 64, 1e4, None) == -2
    assert L.llama_rope_table(FAKE, FAKE, 8, 63, 1e4, None) == -1
    assert L.llama_rope_table(FAKE, FAKE, 0, 64, 1e4, None) == -1
    assert L.llama_rope_table_ntk(None, FAKE, 8, 64, 1e4, 8.0, None) == -2
    assert L.llama_rope_table_ntk(FAKE, FAKE, 8, 2, 1e4, 8.0, None) == -1      # d - 2 = 0
    assert L.llama_rope_table_ntk(FAKE, FAKE, 8, 64, 1e4, 0.5, None) == -1     # shrinks
    assert L.llama_rope_table_ntk(FAKE, FAKE, 8, 64, 1e4, float("inf"), None) == -1
    assert L.llama_rope_table_ntk(FAKE, FAKE, 8, 64, 1e4, float("nan"), None) == -1
    # llama_sample: logits, history, n_hist, u, ids, n, vocab, T, top_k, top_p, penalty
    S = L.llama_sample
    assert S(None, None, 0, FAKE, FAKE, 4, 32000, 0.7, 50, 0.9, 1.1, None) == -2
    assert S(FAKE, None, 3, FAKE, FAKE, 4, 32000, 0.7, 50, 0.9, 1.1, None) == -2  # history needed
    assert S(FAKE + 2, None, 0, FAKE, FAKE, 4, 32000, 0.7, 50, 0.9, 1.1, None) == -3
    assert S(FAKE, None, 0, FAKE, FAKE, 4, 32769, 0.7, 50, 0.9, 1.1, None) == -1
    assert S(FAKE, None, 0, FAKE, FAKE, 4, 32000, 0.7, 1025, 0.9, 1.1, None) == -1
    assert S(FAKE, None, 0, FAKE, FAKE, 4, 32000, 0.7, 0, 0.9, 1.1, None) == -1
    assert S(FAKE, None, 0, FAKE, FAKE, 4, 32000, 0.7, 50, 0.0, 1.1, None) == -1
    assert S(FAKE, None, 0, FAKE, FAKE, 4, 32000, 0.7, 50, 1.5, 1.1, None) == -1
    assert S(FAKE, None, 0, FAKE, FAKE, 4, 32000, -0.1, 50, 0.9, 1.1, None) == -1
    assert S(FAKE, None, 0, FAKE, FAKE, 4, 32000, float("inf"), 50, 0.9, 1.1, None) == -1
    assert S(FAKE, None, 0, FAKE, FAKE, 4, 32000, 0.7, 50, 0.9, 0.0, None) == -1
    assert S(FAKE, None, 0, FAKE, FAKE, -1, 32000, 0.7, 50, 0.9, 1.1, None) == -1
    assert S(FAKE, None, 0, FAKE, FAKE, 0, 32000, 0.7, 50, 0.9, 1.1, None) == 0  # empty: no launch
    W = L.llama_kv_pages_write  # k, v, s_max, start, count, kp, vp, n_blocks, bs, table, max_blocks, B, nkv, hd, dt
    assert W(FAKE, FAKE, 64, 0, 8, FAKE, FAKE, 4, 16, None, 4, 1, 2, 64, 1, None) == -2
    assert W(FAKE, FAKE, 64, 0, 8, FAKE, FAKE, 4, 24, FAKE, 4, 1, 2, 64, 1, None) == -1  # not 2^k
    assert W(FAKE, FAKE, 64, 0, 8, FAKE, FAKE, 4, 8, FAKE, 4, 1, 2, 64, 1, None) == -1   # < 16
    assert W(FAKE, FAKE, 64, 60, 8, FAKE, FAKE, 4, 16, FAKE, 4, 1, 2, 64, 1, None) == -4  # past s_max
    assert W(FAKE, FAKE, 256, 60, 8, FAKE, FAKE, 4, 16, FAKE, 4, 1, 2, 64, 1, None) == -4  # past pages
    assert W(FAKE, FAKE, 64, 0, 8, FAKE, FAKE, 0, 16, FAKE, 4, 1, 2, 64, 1, None) == -1   # no blocks
    assert W(FAKE, FAKE, 64, 0, 0, FAKE, FAKE, 4, 16, FAKE, 4, 1, 2, 64, 1, None) == 0    # nothing
    Q = L.llama_quantize_w8
    assert Q(None, FAKE, FAKE, 4, 32, 1, None) == -2
    assert Q(FAKE, FAKE + 4, FAKE, 4, 32, 1, None) == -3
    assert Q(FAKE, FAKE, FAKE, 4, 40, 1, None) == -1      # cols % 16
    assert Q(FAKE, FAKE, FAKE, 0, 32, 1, None) == -1
    assert Q(FAKE, FAKE, FAKE, 4, 32, 9, None) == -1      # dtype
    Q4 = L.llama_quantize_w4
    assert Q4(None, FAKE, FAKE, 4, 64, 1, None) == -2
    assert Q4(FAKE, FAKE, FAKE + 2, 4, 64, 1, None) == -3
    assert Q4(FAKE, FAKE, FAKE, 4, 48, 1, None) == -1     # cols % 32
    assert Q4(FAKE, FAKE, FAKE, -1, 64, 1, None) == -1
    assert Q4(FAKE, FAKE, FAKE, 4, 64, 3, None) == -1     # dtype
    assert L.llama_embed(FAKE, FAKE, FAKE, 0, 256, 512, 1, None) == -1
    assert L.llama_embed(FAKE, FAKE + 2, FAKE, 1, 256, 512, 1, None) == -3
    assert L.llama_embed(FAKE, FAKE, FAKE, 1, 256, 512, 7, None) == -1
    assert L.llama_head_argmax(FAKE, FAKE, FAKE, FAKE, None, 1, 256, 512, 1e-5, 1, None) == -2
    assert L.llama_head_argmax(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 256, 512, 0.0, 1, None) == -1


def test_timer_validation():
    L = B.lib()
    assert L.llama_layer_timer_start(-1, 4) == -1
    assert L.llama_layer_timer_start(0, 0) == -1


def paged_decode_rc(c, table=FAKE + 0x700000, n_blocks=8, block_size=16, max_blocks=2, ctx=FAKE + 0x600000,
                    batch=2, max_ctx=10, ws_bytes=1, kp=FAKE + 0x300000):
    w = weights()
    return B.lib().llama_layer_decode_paged(ctypes.byref(c), ctypes.byref(w.struct), FAKE + 0x100000,
                                            FAKE + 0x200000, kp, FAKE + 0x400000, n_blocks,
                                            block_size, table, max_blocks, ctx, batch, max_ctx,
                                            FAKE + 0x500000, ws_bytes, None)


def paged_prefill_rc(c, table=FAKE + 0x700000, n_blocks=8, block_size=16, max_blocks=2, tokens=8,
                     start_pos=0, ws_bytes=1):
    w = weights()
    return B.lib().llama_layer_prefill_paged(ctypes.byref(c), ctypes.byref(w.struct),
                                             FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000,
                                             FAKE + 0x400000, n_blocks, block_size, table,
                                             max_blocks, 1, tokens, start_pos, FAKE + 0x500000,
                                             ws_bytes, None)


def test_paged_validation():
    c = cfg()
    assert paged_decode_rc(c) == -5                      # everything valid up to the workspace
    assert paged_decode_rc(c, table=None) == -2
    assert paged_decode_rc(c, table=FAKE + 0x700002) == -3
    assert paged_decode_rc(c, kp=FAKE + 0x300008) == -3
    assert paged_decode_rc(c, block_size=24) == -1       # not a power of two
    assert paged_decode_rc(c, block_size=8) == -1        # below 16
    assert paged_decode_rc(c, block_size=2048) == -1     # above 1024
    assert paged_decode_rc(c, n_blocks=0) == -1
    assert paged_decode_rc(c, max_blocks=0) == -1
    assert paged_decode_rc(c, max_ctx=32) == -4          # 2 blocks of 16: position 32 is past
    assert paged_decode_rc(c, max_ctx=31) == -5
    assert paged_decode_rc(c, batch=0) == -1
    assert paged_prefill_rc(c) == -5
    assert paged_prefill_rc(c, table=None) == -2
    assert paged_prefill_rc(c, block_size=12) == -1
    assert paged_prefill_rc(c, start_pos=30, tokens=3) == -4
    assert paged_prefill_rc(c, start_pos=24, tokens=8) == -5


def test_w8_decode_validation():
    c = cfg()
    names = [n for n, _ in B.ll_weights_w8._fields_]
    ptrs = {n: FAKE + 256 * i for i, n in enumerate(names)}

    def rc(c=c, **kw):
        p = dict(ptrs)
        p.update(kw)
        w = B.ll_weights_w8(*[p[n] for n in names])
        return B.lib().llama_layer_decode_w8(ctypes.byref(c), ctypes.byref(w), FAKE + 0x100000,
                                             FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                                             FAKE + 0x600000, 2, 10, 32, FAKE + 0x500000, 1, None)
    assert rc() == -5
    assert rc(w_down=None) == -2
    assert rc(s_gate=None) == -2
    assert rc(s_up=FAKE + 2) == -3
    assert rc(c=cfg(intermediate=680)) == -1             # not a multiple of 16
    assert B.lib().llama_layer_decode_w8(ctypes.byref(c), None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1,
                                         32, FAKE, 1, None) == -2


def test_w4_decode_validation():
    c = cfg(intermediate=704)
    names = [n for n, _ in B.ll_weights_w4._fields_]
    ptrs = {n: FAKE + 256 * i for i, n in enumerate(names)}

    def rc(c=c, **kw):
        p = dict(ptrs)
        p.update(kw)
        w = B.ll_weights_w4(*[p[n] for n in names])
        return B.lib().llama_layer_decode_w4(ctypes.byref(c), ctypes.byref(w), FAKE + 0x100000,
                                             FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                                             FAKE + 0x600000, 2, 10, 32, FAKE + 0x500000, 1, None)
    assert rc() == -5                                    # workspace too small
    assert rc(w_q=None) == -2
    assert rc(s_o=None) == -2
    assert rc(s_down=FAKE + 1) == -3
    assert rc(c=cfg(intermediate=688)) == -1             # not a multiple of 32
    assert B.lib().llama_layer_decode_w4(ctypes.byref(c), None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1,
                                         32, FAKE, 1, None) == -2


def test_noalloc_validation():
    """llama_layer_decode_noalloc validates like llama_layer_decode, and refuses
    a call whose workspace would exceed its built-in scratch with LL_ESCRATCH
    before touching the device."""
    L = B.lib()

    def rc(c, batch=1, max_ctx=8, s_max=32, x=FAKE, y=FAKE + 0x100000, ctx=FAKE + 0x600000):
        return L.llama_layer_decode_noalloc(ctypes.byref(c), ctypes.byref(weights().struct), x, y,
                                            FAKE + 0x200000, FAKE + 0x300000, ctx, batch, max_ctx,
                                            s_max, None)

    c = cfg()
    assert rc(c, batch=0) == -1
    assert rc(c, max_ctx=-1) == -1
    assert rc(c, max_ctx=32, s_max=32) == -4
    assert rc(c, y=FAKE + 16) == -1                    # y overlaps x
    assert rc(c, ctx=FAKE + 0x600002) == -3
    assert rc(c, x=None) == -2
    assert L.llama_layer_decode_noalloc(None, ctypes.byref(weights().struct), FAKE, FAKE, FAKE,
                                        FAKE, FAKE, 1, 8, 32, None) == -2
    big = cfg(hidden=8192, n_heads=64, n_kv_heads=8, head_dim=128, intermediate=28672,
              max_pos=8192)
    assert rc(big, batch=1024, max_ctx=4096, s_max=4097, y=FAKE + 0x10000000) == -8
    assert "64 MiB" in B.llama_layer_strerror(-8)
