"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (max|got - want| / max|want| per tensor, see gpu_util): 1e-4 for the
float32 path and 2e-2 for bf16/f16, applied to the output, the branch delta
out - x and the appended K/V entries; the tiny stack must pick identical greedy
ids.  Small cases span several tiles with ragged tails in every dimension;
full-size cases run the shapes and launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

from gpu_util import (TOL, DeviceLayer, check_errors, delta_error, from_dev, oracle_cfg,
                      oracle_weights, random_layer, rel_err, scale_stored, to_dev)
from llama2_decoder_layer_amd import binding as B
from llama2_decoder_layer_amd import synth as S
from oracle import llama_ref as R

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def run_prefill_case(label, shape, act, kv, batch, tokens, start_pos, s_max, seed,
                     out_rows=None, x_scale=1.0, gpu_edit=None):
    say(f"[{label}] prefill B={batch} T={tokens} start={start_pos} s_max={s_max} {act}/{kv} "
        f"x*{x_scale} {shape}")
    stored = random_layer(shape, act, seed)
    inp = S.draw_prefill_inputs(np.random.SeedSequence(seed + 1), shape, batch, tokens, s_max,
                                act, kv, start_pos)
    if x_scale != 1.0:
        inp["x"] = scale_stored(inp["x"], act, x_scale)
    # gpu_edit(stored) -> the weights the GPU gets instead (negative controls)
    dl = DeviceLayer(shape, gpu_edit(stored) if gpu_edit else stored, act, kv, max_pos=s_max)
    x = to_dev(inp["x"], act)
    kc = to_dev(inp["k_cache"], kv)
    vc = to_dev(inp["v_cache"], kv)
    y = dl.prefill(x, kc, vc, batch, tokens, start_pos, s_max)
    torch.cuda.synchronize()
    cfg, w = oracle_cfg(shape), oracle_weights(stored, act)
    x64 = S.to_f64(inp["x"], act)
    kc64 = S.to_f64(inp["k_cache"], kv)
    vc64 = S.to_f64(inp["v_cache"], kv)
    want = R.layer_prefill(cfg, w, x64, kc64, vc64, start_pos, out_rows=out_rows)
    got = from_dev(y)
    xs = x64
    if out_rows is not None:
        got = got[:, out_rows]
        xs = x64[:, out_rows]
    new = slice(start_pos, start_pos + tokens)
    d_err, d_allow = delta_error(got, want, xs, act)
    errs = {"out": rel_err(got, want), "delta": d_err,
            "k_new": rel_err(from_dev(kc)[:, :, new], kc64[:, :, new]),
            "v_new": rel_err(from_dev(vc)[:, :, new], vc64[:, :, new])}
    # entries outside the written positions are untouched
    old_k = S.to_f64(inp["k_cache"], kv)
    gk = from_dev(kc)
    assert np.array_equal(gk[:, :, :start_pos], old_k[:, :, :start_pos])
    assert np.array_equal(gk[:, :, start_pos + tokens:], old_k[:, :, start_pos + tokens:])
    check_errors(label, errs, TOL[act], {"delta": d_allow})
    return errs


def run_decode_case(label, shape, act, kv, ctx_len, s_max, seed, x_scale=1.0, ntk_scale=None,
                    gpu_edit=None):
    batch = len(ctx_len)
    say(f"[{label}] decode B={batch} ctx={[int(c) for c in ctx_len][:8]} s_max={s_max} "
        f"{act}/{kv} x*{x_scale} ntk={ntk_scale} {shape}")
    stored = random_layer(shape, act, seed)
    inp = S.draw_decode_inputs(np.random.SeedSequence(seed + 1), shape, batch, s_max, act, kv,
                               ctx=0)
    if x_scale != 1.0:
        inp["x"] = scale_stored(inp["x"], act, x_scale)
    ctx = np.asarray(ctx_len, dtype=np.int32)
    dl = DeviceLayer(shape, gpu_edit(stored) if gpu_edit else stored, act, kv, max_pos=s_max,
                     ntk_scale=ntk_scale)
    x = to_dev(inp["x"], act)
    kc = to_dev(inp["k_cache"], kv)
    vc = to_dev(inp["v_cache"], kv)
    dctx = torch.from_numpy(ctx).cuda()
    y = dl.decode(x, kc, vc, dctx, batch, int(ctx.max()), s_max)
    torch.cuda.synchronize()
    cfg, w = oracle_cfg(shape, ntk_scale), oracle_weights(stored, act)
    x64 = S.to_f64(inp["x"], act)
    kc64 = S.to_f64(inp["k_cache"], kv)
    vc64 = S.to_f64(inp["v_cache"], kv)
    want = R.layer_decode(cfg, w, x64, kc64, vc64, ctx)
    got = from_dev(y)
    gk, gv = from_dev(kc), from_dev(vc)
    bi = np.arange(batch)
    d_err, d_allow = delta_error(got, want, x64, act)
    errs = {"out": rel_err(got, want), "delta": d_err,
            "k_new": rel_err(gk[bi, :, ctx], kc64[bi, :, ctx]),
            "v_new": rel_err(gv[bi, :, ctx], vc64[bi, :, ctx])}
    # only position ctx_len[b] of each sequence changed
    mask = np.ones(gk.shape[:3], dtype=bool)
    mask[bi, :, ctx] = False
    assert np.array_equal(gk[mask], S.to_f64(inp["k_cache"], kv)[mask])
    check_errors(label, errs, TOL[act], {"delta": d_allow})
    return errs


# ---------------------------------------------------------------------------
# float32 path
# ---------------------------------------------------------------------------

def test_f32_tiny_prefill():
    run_prefill_case("f32-tiny-prefill", S.TINY, "f32", "f32", 1, 16, 0, 24, 100)


def test_f32_prefill_multi_chunk_ragged():
    # 45 tokens: two launch groups (32 + 13), after 5 cached positions, 2 sequences
    run_prefill_case("f32-prefill-45", S.Shape(128, 2, 1, 64, 344), "f32", "f32", 2, 45, 5, 64, 101)


def test_f32_decode_ragged():
    run_decode_case("f32-decode", S.Shape(256, 4, 2, 64, 688), "f32", "f32", [0, 7, 23, 64, 100],
                    128, 102)


def test_f32_hd128_mha():
    run_decode_case("f32-decode-hd128", S.Shape(256, 2, 2, 128, 520), "f32", "f32", [3, 40], 64, 103)


# ---------------------------------------------------------------------------
# bf16 / f16: token-skinny plan (decode, short prefill)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("label,shape,act,kv,ctx", [
    ("piece-bf16", S.Shape(2048, 16, 4, 128, 4096), "bf16", "bf16", [37]),
    ("piece-f16", S.Shape(2048, 16, 4, 128, 4096), "f16", "f16", [200]),
    ("piece-k16384", S.Shape(1024, 8, 8, 128, 16384), "bf16", "bf16", [5]),
])
def test_decode_one_token_piece_gemv(label, shape, act, kv, ctx):
    """One token per launch with K a multiple of 2048: O (K = 2048: 8 rows per
    piece) and down (K = 4096: 4 rows; K = 16384: one row) take the
    piece-ordered GEMV."""
    run_decode_case(label, shape, act, kv, ctx, 256, 151)


def test_bf16_decode_gqa_f16_cache():
    run_decode_case("bf16-decode-gqa", S.Shape(512, 8, 2, 128, 1376), "bf16", "f16",
                    [0, 1, 63, 64, 65, 300, 511], 512, 110)


def test_bf16_decode_gqa8_hd64_long():
    # 8 query heads per KV head at head_dim 64 (the MFMA decode attention with
    # GC = 8, HD = 64), contexts from one key to several chunks, odd and even
    # numbers of 64-key steps per workgroup
    run_decode_case("bf16-decode-gqa8-hd64", S.Shape(512, 8, 1, 64, 1376), "bf16", "f16",
                    [0, 15, 16, 17, 129, 255, 256, 1000, 2998], 3000, 113)


def test_bf16_decode_batch_over_32():
    ctx = list(np.random.Generator(np.random.PCG64(5)).integers(0, 200, 40))
    run_decode_case("bf16-decode-b40", S.Shape(256, 4, 1, 64, 688), "bf16", "bf16", ctx, 256, 111)


@pytest.mark.parametrize("label,act,x_scale,norm_passes", [
    ("deferred-ffn-norm", "bf16", 1.0, 1),
    ("deferred-ffn-norm-small-x", "bf16", 2.0 ** -8, 1),
    ("f16-ffn-norm-pass", "f16", 1.0, 2),
])
def test_decode_deferred_ffn_norm(label, act, x_scale, norm_passes):
    """24 tokens at hidden 2048 with learned gains: the O projection takes the
    K-split streaming path, so with bf16 activations its reduction also writes
    h1 * ffn_norm and per-token partial sums of h1^2, and the gate/up epilogue
    applies 1/rms; one norm pass per call instead of two.  f16 activations keep
    the pass.  The small-x case makes the branches dominate the output."""
    ctx = list(np.random.Generator(np.random.PCG64(9)).integers(0, 500, 24))
    B.llama_layer_timer_start(B.kernel_id("rmsnorm"), 16)
    try:
        run_decode_case(label, S.Shape(2048, 16, 4, 128, 5632), act, "f16", ctx, 512, 160,
                        x_scale=x_scale)
    finally:
        _, launches = B.llama_layer_timer_stop()
    assert launches == norm_passes, (label, launches)


@pytest.mark.parametrize("label,shape", [
    # K = 1088: the last 128-k stage is half empty (no stage rotation)
    ("wide-gate-up-partial-stage", S.Shape(1088, 17, 1, 64, 16424)),
    # K = 1024: eight whole stages, rotated by workgroup
    ("wide-gate-up-rotated", S.Shape(1024, 8, 2, 128, 16424)),
])
def test_decode_32_tokens_wide_gate_up(label, shape):
    """32 tokens with an intermediate size of 16424: gate/up has 257 blocks of
    64 features, so it runs unsplit in the 128-row streaming shape, its last
    workgroup holding 40 features."""
    ctx = list(np.random.Generator(np.random.PCG64(11)).integers(0, 200, 32))
    run_decode_case(label, shape, "bf16", "f16", ctx, 256, 170)


def test_f16_decode_mha():
    run_decode_case("f16-decode", S.Shape(256, 4, 4, 64, 768), "f16", "f16", [10, 129], 160, 112)


def test_rope_table_ntk():
    """The NTK-aware tables against the oracle's angles with the scaled base,
    over a 32K table: within one float32 rounding of cos/sin."""
    hd, max_pos, scale = 128, 32769, 8.0
    c = torch.empty(max_pos, hd // 2, dtype=torch.float32, device="cuda")
    s = torch.empty_like(c)
    from llama2_decoder_layer_amd import binding as B
    B.llama_rope_table_ntk(c, s, max_pos, hd, 10000.0, scale)
    torch.cuda.synchronize()
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * \
        R.rope_inv_freq(hd, R.ntk_rope_base(10000.0, scale, hd))[None, :]
    ec = np.max(np.abs(c.cpu().numpy() - np.cos(ang)))
    es = np.max(np.abs(s.cpu().numpy() - np.sin(ang)))
    say(f"[rope-ntk] max |cos err| {ec:.2e}, |sin err| {es:.2e}")
    assert ec < 2 ** -23 and es < 2 ** -23
    # scale 1 gives the plain tables bit for bit
    c1, s1 = torch.empty_like(c[:4097]), torch.empty_like(s[:4097])
    c0, s0 = torch.empty_like(c1), torch.empty_like(s1)
    B.llama_rope_table_ntk(c1, s1, 4097, hd, 10000.0, 1.0)
    B.llama_rope_table(c0, s0, 4097, hd, 10000.0)
    assert torch.equal(c1, c0) and torch.equal(s1, s0)


def test_bf16_decode_ntk_long_context():
    # positions past 4K with the base scaled for a 4x longer context; GQA 4:1,
    # f16 cache, contexts spanning several attention chunks and a ragged tail
    run_decode_case("bf16-decode-ntk4", S.Shape(512, 8, 2, 128, 1376), "bf16", "f16",
                    [4096, 6001, 8191, 300], 8192, 114, ntk_scale=4.0)


def test_bf16_short_prefill_skinny():
    run_prefill_case("bf16-prefill-20", S.Shape(256, 4, 2, 64, 688), "bf16", "bf16", 1, 20, 7, 40,
                     113)


# ---------------------------------------------------------------------------
# bf16 / f16: token-wide plan (GEMM + MFMA attention)
# ---------------------------------------------------------------------------

def test_bf16_prefill_wide_ragged():
    # 200 tokens x 2 sequences: 128-token tiles with a 72-token tail; I = 688
    run_prefill_case("bf16-prefill-wide", S.TINY, "bf16", "bf16", 2, 200, 0, 200, 120)


def test_bf16_prefill_wide_hd128_gqa_offset():
    run_prefill_case("bf16-prefill-hd128", S.Shape(512, 8, 2, 128, 1032), "bf16", "bf16", 1, 300,
                     50, 400, 121)


def test_bf16_prefill_split_k_tiles():
    # 2 sequences x 1280 tokens at hidden 1024: QKV (3072 features, 10 x 12
    # tiles of 256) and gate/up (2816 features) fall below one round of
    # 256 x 256 tiles and are split along K; O and down take 128 x 128 tiles.
    # Rows sampled across token tiles, every appended K/V entry checked.
    rows = np.array([0, 1, 255, 256, 700, 1023, 1024, 1279])
    run_prefill_case("bf16-prefill-split-k", S.Shape(1024, 8, 8, 128, 2816), "bf16", "bf16", 2,
                     1280, 0, 1280, 131, out_rows=rows)


def test_bf16_prefill_192_row_tiles():
    # 3072 tokens (12 token panels) at hidden 3072, 24 query heads over 2 KV
    # heads: the QKV (3584 features: 168 tiles of 256 rows, 228 of 192), O and
    # down (3072: 144 and 192) fill more than half a round of 256 x 256 tiles
    # and take 192 x 256 tiles; the QKV tile at features 3264-3455 straddles
    # the k/v boundary (3328).  Rows sampled across token tiles, every K/V
    # entry checked.
    rows = np.array([0, 255, 256, 1500, 2047, 2048, 3071])
    run_prefill_case("bf16-prefill-192", S.Shape(3072, 24, 2, 128, 2048), "bf16", "bf16", 1,
                     3072, 0, 3072, 141, out_rows=rows)


def test_bf16_prefill_wide_f16_cache_mqa():
    run_prefill_case("bf16-prefill-f16kv", S.Shape(256, 4, 1, 64, 512), "bf16", "f16", 1, 130, 3,
                     140, 122)


def test_bf16_prefill_wide_branch_dominant():
    """x scaled by 2^-8: the branches dominate out, so out itself checks them."""
    run_prefill_case("bf16-prefill-small-x", S.Shape(256, 4, 2, 64, 688), "bf16", "bf16", 1, 150,
                     0, 160, 124, x_scale=2.0 ** -8)


def test_bf16_decode_branch_dominant():
    shape, act, kv = S.Shape(512, 8, 2, 128, 1376), "bf16", "bf16"
    run_decode_case("bf16-decode-small-x", shape, act, kv, [5, 200, 33], 256, 125, x_scale=2.0 ** -8)


def test_f16_prefill_wide():
    run_prefill_case("f16-prefill-wide", S.Shape(384, 6, 3, 64, 1024), "f16", "f16", 1, 33, 0, 33,
                     123)


def test_bf16_prefill_then_decode_matches_longer_prefill():
    """GPU prefill(T) followed by decodes equals GPU prefill(T + k) on the new rows."""
    shape, act, kv = S.Shape(256, 4, 2, 64, 688), "bf16", "bf16"
    T, k, s_max = 100, 3, 128
    say(f"[prefill-then-decode] T={T} k={k}")
    stored = random_layer(shape, act, 130)
    inp = S.draw_prefill_inputs(np.random.SeedSequence(131), shape, 1, T + k, s_max, act, kv)
    dl = DeviceLayer(shape, stored, act, kv, max_pos=s_max)
    x = to_dev(inp["x"], act)
    kc1, vc1 = to_dev(inp["k_cache"], kv), to_dev(inp["v_cache"], kv)
    y_full = dl.prefill(x, kc1, vc1, 1, T + k, 0, s_max)
    kc2, vc2 = to_dev(inp["k_cache"], kv), to_dev(inp["v_cache"], kv)
    dl.prefill(x[:, :T].contiguous(), kc2, vc2, 1, T, 0, s_max)
    outs = []
    for i in range(k):
        ctx = torch.tensor([T + i], dtype=torch.int32, device="cuda")
        outs.append(dl.decode(x[:, T + i].contiguous(), kc2, vc2, ctx, 1, T + i, s_max))
    torch.cuda.synchronize()
    got = np.stack([from_dev(o)[0] for o in outs])
    want = from_dev(y_full)[0, T:]
    err = rel_err(got, want)
    say(f"[prefill-then-decode] err={err:.2e}")
    assert err < TOL[act]


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

def test_decode_7b_full():
    name = "decode_7b_b1_ctx4096"
    wl = S.WORKLOADS[name]
    say(f"[{name}] drawing inputs")
    stored, inp = S.workload_layer_and_inputs(name)
    dl = DeviceLayer(wl.shape, stored, wl.act_dtype, wl.kv_dtype, max_pos=wl.s_max)
    x = to_dev(inp["x"], wl.act_dtype)
    kc, vc = to_dev(inp["k_cache"], wl.kv_dtype), to_dev(inp["v_cache"], wl.kv_dtype)
    ctx = torch.from_numpy(inp["ctx_len"]).cuda()
    say(f"[{name}] decode on GPU")
    y = dl.decode(x, kc, vc, ctx, wl.batch, int(inp["ctx_len"].max()), wl.s_max)
    torch.cuda.synchronize()
    kc64, vc64 = S.to_f64(inp["k_cache"], wl.kv_dtype), S.to_f64(inp["v_cache"], wl.kv_dtype)
    x64 = S.to_f64(inp["x"], wl.act_dtype)
    want = R.layer_decode(oracle_cfg(wl.shape), oracle_weights(stored, wl.act_dtype), x64, kc64,
                          vc64, inp["ctx_len"])
    got = from_dev(y)
    p = int(inp["ctx_len"][0])
    d_err, d_allow = delta_error(got, want, x64, wl.act_dtype)
    errs = {"out": rel_err(got, want), "delta": d_err,
            "k_new": rel_err(from_dev(kc)[:, :, p], kc64[:, :, p]),
            "v_new": rel_err(from_dev(vc)[:, :, p], vc64[:, :, p])}
    check_errors(name, errs, TOL[wl.act_dtype], {"delta": d_allow})


def test_decode_7b_ntk8_ctx32768_full():
    """The long-context benchmark case: a 7B layer decoding at position 32768
    with the NTK-aware tables for an 8x context."""
    name = "decode_7b_b1_ctx32768_ntk8"
    wl = S.WORKLOADS[name]
    ntk = wl.extra["ntk_scale"]
    say(f"[{name}] drawing inputs")
    stored, inp = S.workload_layer_and_inputs(name)
    dl = DeviceLayer(wl.shape, stored, wl.act_dtype, wl.kv_dtype, max_pos=wl.s_max, ntk_scale=ntk)
    x = to_dev(inp["x"], wl.act_dtype)
    kc, vc = to_dev(inp["k_cache"], wl.kv_dtype), to_dev(inp["v_cache"], wl.kv_dtype)
    ctx = torch.from_numpy(inp["ctx_len"]).cuda()
    say(f"[{name}] decode on GPU")
    y = dl.decode(x, kc, vc, ctx, wl.batch, int(inp["ctx_len"].max()), wl.s_max)
    torch.cuda.synchronize()
    say(f"[{name}] oracle")
    kc64, vc64 = S.to_f64(inp["k_cache"], wl.kv_dtype), S.to_f64(inp["v_cache"], wl.kv_dtype)
    x64 = S.to_f64(inp["x"], wl.act_dtype)
    want = R.layer_decode(oracle_cfg(wl.shape, ntk), oracle_weights(stored, wl.act_dtype), x64,
                          kc64, vc64, inp["ctx_len"])
    got = from_dev(y)
    p = int(inp["ctx_len"][0])
    d_err, d_allow = delta_error(got, want, x64, wl.act_dtype)
    errs = {"out": rel_err(got, want), "delta": d_err,
            "k_new": rel_err(from_dev(kc)[:, :, p], kc64[:, :, p]),
            "v_new": rel_err(from_dev(vc)[:, :, p], vc64[:, :, p])}
    check_errors(name, errs, TOL[wl.act_dtype], {"delta": d_allow})


def test_decode_70b_b32_full():
    name = "decode_70b_b32_ragged"
    wl = S.WORKLOADS[name]
    say(f"[{name}] drawing inputs")
    stored, inp = S.workload_layer_and_inputs(name)
    dl = DeviceLayer(wl.shape, stored, wl.act_dtype, wl.kv_dtype, max_pos=wl.s_max)
    x = to_dev(inp["x"], wl.act_dtype)
    kc, vc = to_dev(inp["k_cache"], wl.kv_dtype), to_dev(inp["v_cache"], wl.kv_dtype)
    ctx = torch.from_numpy(inp["ctx_len"]).cuda()
    say(f"[{name}] decode on GPU")
    y = dl.decode(x, kc, vc, ctx, wl.batch, int(inp["ctx_len"].max()), wl.s_max)
    torch.cuda.synchronize()
    say(f"[{name}] oracle")
    kc64, vc64 = S.to_f64(inp["k_cache"], wl.kv_dtype), S.to_f64(inp["v_cache"], wl.kv_dtype)
    x64 = S.to_f64(inp["x"], wl.act_dtype)
    want = R.layer_decode(oracle_cfg(wl.shape), oracle_weights(stored, wl.act_dtype), x64, kc64,
                          vc64, inp["ctx_len"])
    got = from_dev(y)
    bi = np.arange(wl.batch)
    c = inp["ctx_len"]
    d_err, d_allow = delta_error(got, want, x64, wl.act_dtype)
    errs = {"out": rel_err(got, want), "delta": d_err,
            "k_new": rel_err(from_dev(kc)[bi, :, c], kc64[bi, :, c]),
            "v_new": rel_err(from_dev(vc)[bi, :, c], vc64[bi, :, c])}
    check_errors(name, errs, TOL[wl.act_dtype], {"delta": d_allow})


def test_prefill_13b_full_sampled_rows():
    name = "prefill_13b_t4096"
    wl = S.WORKLOADS[name]
    say(f"[{name}] drawing inputs")
    stored, inp = S.workload_layer_and_inputs(name)
    dl = DeviceLayer(wl.shape, stored, wl.act_dtype, wl.kv_dtype, max_pos=wl.s_max)
    x = to_dev(inp["x"], wl.act_dtype)
    kc, vc = to_dev(inp["k_cache"], wl.kv_dtype), to_dev(inp["v_cache"], wl.kv_dtype)
    say(f"[{name}] prefill on GPU")
    y = dl.prefill(x, kc, vc, 1, wl.tokens, 0, wl.s_max)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 1000, 2047, 2048, 3000, 4094, 4095])
    say(f"[{name}] oracle on rows {list(rows)}")
    kc64 = np.zeros((1, wl.shape.n_kv_heads, wl.s_max, wl.shape.head_dim))
    vc64 = np.zeros_like(kc64)
    x64 = S.to_f64(inp["x"], wl.act_dtype)
    want = R.layer_prefill(oracle_cfg(wl.shape), oracle_weights(stored, wl.act_dtype), x64, kc64,
                           vc64, 0, out_rows=rows)
    got = from_dev(y)[:, rows]
    xs = x64[:, rows]
    d_err, d_allow = delta_error(got, want, xs, wl.act_dtype)
    errs = {"out": rel_err(got, want), "delta": d_err,
            "k_all": rel_err(from_dev(kc), kc64), "v_all": rel_err(from_dev(vc), vc64)}
    check_errors(name, errs, TOL[wl.act_dtype], {"delta": d_allow})


# ---------------------------------------------------------------------------
# Tiny stack: greedy ids
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("learned_gains", [False, True], ids=["unit-gains", "learned-gains"])
def test_tiny_stack_greedy_ids(learned_gains):
    """The tiny fp32 stack as specified (every gain 1), and the same stack with
    learned gains in both norms of each layer and in the final norm."""
    from llama2_decoder_layer_amd import binding as B
    from llama2_decoder_layer_amd.stack import Stack
    wl = S.WORKLOADS["tiny_stack_f32"]
    st = S.draw_stack(wl, learned_gains=learned_gains)
    act = wl.act_dtype
    say(f"[tiny-stack] generate on GPU (learned gains: {learned_gains})")
    layers = [DeviceLayer(wl.shape, lw, act, wl.kv_dtype, max_pos=wl.s_max) for lw in st["layers"]]
    stack = Stack(layers[0].cfg, [l.weights for l in layers], to_dev(st["embed"], act),
                  to_dev(st["final_norm"], act), to_dev(st["w_lm"], act), wl.vocab)
    prompt = torch.from_numpy(st["prompt"]).cuda()
    ids, logits = stack.generate_greedy(prompt, wl.new_tokens, wl.s_max, return_logits=True)
    torch.cuda.synchronize()
    cfg = oracle_cfg(wl.shape)
    want_ids, want_logits = R.generate_greedy(
        cfg, [oracle_weights(lw, act) for lw in st["layers"]], S.to_f64(st["embed"], act),
        S.to_f64(st["final_norm"], act), S.to_f64(st["w_lm"], act), st["prompt"], wl.new_tokens,
        wl.s_max)
    got_logits = from_dev(logits)
    err = rel_err(got_logits, want_logits)
    srt = np.sort(want_logits, axis=1)
    gap = (srt[:, -1] - srt[:, -2]) / np.max(np.abs(want_logits))
    say(f"[tiny-stack] ids gpu={list(ids)} oracle={list(want_ids)} logits err={err:.2e} "
        f"min top1-top2 gap={gap.min():.2e}")
    assert err < TOL[act]
    assert gap.min() > 10 * TOL[act], "near-tie: ids cannot be compared"
    assert list(ids) == list(want_ids)


# ---------------------------------------------------------------------------
# RMSNorm gains: negative controls and the f16 range
# ---------------------------------------------------------------------------

def _ones_like_gain(g, act):
    return S.to_storage(np.ones(g.shape, np.float32), act)


GAIN_PATHS = {
    # label: (runner, args) -- which kernels apply the gains
    "decode1-bf16-fused": ("decode", S.Shape(512, 8, 2, 128, 1376), "bf16", "bf16", [100], 256),
    "decode3-f32-fused": ("decode", S.Shape(256, 4, 2, 64, 688), "f32", "f32", [5, 60, 9], 64),
    "decode2-f16-fused": ("decode", S.Shape(256, 4, 4, 64, 768), "f16", "f16", [10, 129], 160),
    "decode7-bf16-normpass": ("decode", S.Shape(512, 8, 2, 128, 1376), "bf16", "f16",
                              [0, 1, 63, 64, 65, 300, 200], 512),
    "prefill64-bf16-wide": ("prefill", S.Shape(256, 4, 2, 64, 688), "bf16", "bf16", 64, 64),
}


def _run_gain_path(label, edit=None):
    kind, shape, act, kv, arg, s_max = GAIN_PATHS[label]
    gpu_edit = None
    if edit == "ones":
        def gpu_edit(st):
            d = dict(st)
            d["attn_norm"] = _ones_like_gain(st["attn_norm"], act)
            d["ffn_norm"] = _ones_like_gain(st["ffn_norm"], act)
            return d
    elif edit == "swap":
        def gpu_edit(st):
            d = dict(st)
            d["attn_norm"], d["ffn_norm"] = st["ffn_norm"], st["attn_norm"]
            return d
    tag = f"{label}-{edit or 'as-drawn'}"
    if kind == "decode":
        run_decode_case(tag, shape, act, kv, arg, s_max, 170, gpu_edit=gpu_edit)
    else:
        run_prefill_case(tag, shape, act, kv, 1, arg, 0, s_max, 170, gpu_edit=gpu_edit)


@pytest.mark.parametrize("label", sorted(GAIN_PATHS))
def test_learned_gains(label):
    """Learned attn_norm and ffn_norm gains (different draws) on each path
    that applies them: the fused staging of the row kernels (bf16, f16, f32),
    the separate norm pass of the streaming projections, the prefill norms."""
    _run_gain_path(label)


@pytest.mark.parametrize("edit", ["ones", "swap"])
@pytest.mark.parametrize("label", sorted(GAIN_PATHS))
def test_learned_gains_negative_control(label, edit):
    """The same cases with the GPU given unit gains, or attn_norm and ffn_norm
    swapped, while the oracle keeps the drawn ones: the comparison must fail,
    so the passing cases above do test the gains."""
    with pytest.raises(AssertionError, match="errors above"):
        _run_gain_path(label, edit)


@pytest.mark.parametrize("batch", [1, 7])
def test_f16_large_activation_with_gain(batch):
    """f16 activations with an outlier of 30000 in x and gains up to 4: x times
    the gain (120000) is beyond f16's range, the normalised row is not.  Both
    the fused staging (1 token) and the norm pass (7 tokens) stay finite and
    match the oracle."""
    shape, act, kv = S.Shape(256, 4, 4, 64, 768), "f16", "f16"
    s_max = 64
    stored = random_layer(shape, act, 171)
    g = S.to_f64(stored["attn_norm"], act)
    g[3] = 4.0
    stored["attn_norm"] = S.to_storage(g.astype(np.float32), act)
    g2 = S.to_f64(stored["ffn_norm"], act)
    g2[3] = 4.0
    stored["ffn_norm"] = S.to_storage(g2.astype(np.float32), act)
    inp = S.draw_decode_inputs(np.random.SeedSequence(172), shape, batch, s_max, act, kv, ctx=0)
    x = S.to_f64(inp["x"], act)
    x[:, 3] = 30000.0
    inp["x"] = S.to_storage(x.astype(np.float32), act)
    ctx = np.arange(batch, dtype=np.int32) * 7 + 3
    say(f"[f16-outlier B={batch}] decode")
    dl = DeviceLayer(shape, stored, act, kv, max_pos=s_max)
    xd = to_dev(inp["x"], act)
    kc, vc = to_dev(inp["k_cache"], kv), to_dev(inp["v_cache"], kv)
    y = dl.decode(xd, kc, vc, torch.from_numpy(ctx).cuda(), batch, int(ctx.max()), s_max)
    torch.cuda.synchronize()
    got = from_dev(y)
    assert np.all(np.isfinite(got)), "non-finite output"
    want = R.layer_decode(oracle_cfg(shape), oracle_weights(stored, act), x,
                          S.to_f64(inp["k_cache"], kv), S.to_f64(inp["v_cache"], kv), ctx)
    d_err, d_allow = delta_error(got, want, x, act)
    check_errors(f"f16-outlier-B{batch}", {"out": rel_err(got, want), "delta": d_err}, TOL[act],
                 {"delta": d_allow})
