"""GPU parity of the paged KV cache: llama_layer_decode_paged against
llama_layer_decode on the same layer, input and cache contents laid out as
shuffled pool blocks.  Only the addresses differ, so the outputs and the
appended K/V entries must agree bit for bit; one case is also checked against
the fp64 oracle, and llama_kv_pages_write against a host-side scatter."""
import numpy as np
import pytest
import torch

from gpu_util import (TOL, DeviceLayer, check_errors, delta_error, from_dev, oracle_cfg,
                      oracle_weights, random_layer, rel_err, scale_stored, to_dev)
from llama2_decoder_layer_amd import binding as B
from llama2_decoder_layer_amd import synth as S
from oracle import llama_ref as R

pytestmark = pytest.mark.gpu

STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}


def say(msg):
    print(msg, flush=True)


def make_pages(batch, nkv, s_max, hd, bs, kv, seed, spare=3):
    """A shuffled block table covering s_max positions per sequence, plus a few
    pool blocks no sequence uses."""
    max_blocks = -(-s_max // bs)
    n_blocks = batch * max_blocks + spare
    perm = np.random.default_rng(seed).permutation(n_blocks)[:batch * max_blocks]
    table = perm.reshape(batch, max_blocks).astype(np.int32)
    return table, n_blocks, max_blocks


def scatter(cache, table, n_blocks, bs, fill):
    """Host-side copy of contiguous caches [B, nkv, S, hd] into a pool."""
    batch, nkv, s_max, hd = cache.shape
    pool = np.full((n_blocks, nkv, bs, hd), fill, dtype=cache.dtype)
    for b in range(batch):
        for i in range(table.shape[1]):
            lo, hi = i * bs, min((i + 1) * bs, s_max)
            if lo < hi:
                pool[table[b, i], :, :hi - lo] = cache[b, :, lo:hi]
    return pool


def gather(pool, table, s_max):
    batch = table.shape[0]
    nkv, bs, hd = pool.shape[1:]
    out = np.empty((batch, nkv, s_max, hd), dtype=pool.dtype)
    for b in range(batch):
        for i in range(table.shape[1]):
            lo, hi = i * bs, min((i + 1) * bs, s_max)
            if lo < hi:
                out[b, :, lo:hi] = pool[table[b, i], :, :hi - lo]
    return out


def run_paged_case(label, shape, act, kv, ctx_len, s_max, bs, seed, oracle=False, stored=None,
                   inp=None, x_scale=1.0):
    batch = len(ctx_len)
    say(f"[{label}] paged decode B={batch} ctx={[int(c) for c in ctx_len][:8]} s_max={s_max} "
        f"block={bs} {act}/{kv} {shape}")
    if stored is None:
        stored = random_layer(shape, act, seed)
    if inp is None:
        inp = S.draw_decode_inputs(np.random.SeedSequence(seed + 1), shape, batch, s_max, act, kv,
                                   ctx=0)
    if x_scale != 1.0:
        inp = dict(inp, x=scale_stored(inp["x"], act, x_scale))
    ctx = np.asarray(ctx_len, dtype=np.int32)
    dl = DeviceLayer(shape, stored, act, kv, max_pos=s_max)
    x = to_dev(inp["x"], act)
    dctx = torch.from_numpy(ctx).cuda()
    # contiguous reference run
    kc, vc = to_dev(inp["k_cache"], kv), to_dev(inp["v_cache"], kv)
    y_ref = dl.decode(x, kc, vc, dctx, batch, int(ctx.max()), s_max)
    # paged run over the same contents
    table, n_blocks, max_blocks = make_pages(batch, shape.n_kv_heads, s_max, shape.head_dim, bs,
                                             kv, seed + 7)
    fill = np.array(0x7FC0 if kv != "f32" else np.nan, dtype=STORAGE[kv])  # NaN in unused slots
    kp_h = scatter(inp["k_cache"], table, n_blocks, bs, fill)
    vp_h = scatter(inp["v_cache"], table, n_blocks, bs, fill)
    kp, vp = to_dev(kp_h, kv), to_dev(vp_h, kv)
    dtab = torch.from_numpy(table).cuda()
    y = torch.full_like(x, float("nan"))
    ws = dl.workspace(batch, 1, max_blocks * bs)
    B.llama_layer_decode_paged(dl.cfg, dl.weights, x, y, kp, vp, bs, dtab, dctx, batch,
                               int(ctx.max()), ws)
    torch.cuda.synchronize()
    got, ref = from_dev(y), from_dev(y_ref)
    assert np.array_equal(got, ref), f"{label}: paged output differs from contiguous"
    # the pool, gathered back, equals the contiguous cache after its append
    gk = gather(kp.view(torch.int16 if kv != "f32" else torch.float32).cpu().numpy()
                .view(STORAGE[kv]), table, s_max)
    gv = gather(vp.view(torch.int16 if kv != "f32" else torch.float32).cpu().numpy()
                .view(STORAGE[kv]), table, s_max)
    rk = kc.view(torch.int16 if kv != "f32" else torch.float32).cpu().numpy().view(STORAGE[kv])
    rv = vc.view(torch.int16 if kv != "f32" else torch.float32).cpu().numpy().view(STORAGE[kv])
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv), f"{label}: caches differ"
    say(f"[{label}] paged == contiguous, bit for bit (output and caches)")
    if oracle:
        x64 = S.to_f64(inp["x"], act)
        kc64, vc64 = S.to_f64(inp["k_cache"], kv), S.to_f64(inp["v_cache"], kv)
        want = R.layer_decode(oracle_cfg(shape), oracle_weights(stored, act), x64, kc64, vc64, ctx)
        bi = np.arange(batch)
        d_err, d_allow = delta_error(got, want, x64, act)
        errs = {"out": rel_err(got, want), "delta": d_err,
                "k_new": rel_err(S.to_f64(gk, kv)[bi, :, ctx], kc64[bi, :, ctx]),
                "v_new": rel_err(S.to_f64(gv, kv)[bi, :, ctx], vc64[bi, :, ctx])}
        check_errors(label, errs, TOL[act], {"delta": d_allow})


def test_paged_mha_split_kernel_block16():
    # one query head per KV head: the split kernel; contexts at and around block edges
    run_paged_case("paged-mha", S.Shape(512, 4, 4, 128, 1376), "bf16", "bf16",
                   [0, 15, 16, 17, 300, 511], 512, 16, 150, oracle=True)


def test_paged_gqa4_f16_block64():
    run_paged_case("paged-gqa4", S.Shape(512, 8, 2, 128, 1376), "bf16", "f16",
                   [1, 63, 64, 65, 700, 1023], 1024, 64, 151)


def test_paged_gqa8_whole_contexts():
    # 64 sequences x 4 KV heads >= 256 groups: the 8-wave whole-context kernel
    ctx = list(np.random.default_rng(3).integers(0, 300, 64))
    run_paged_case("paged-gqa8-whole", S.Shape(512, 32, 4, 64, 512), "bf16", "bf16", ctx, 320, 32,
                   152)


@pytest.mark.parametrize("label,shape,kv", [
    ("paged-piece-4", S.Shape(2048, 16, 4, 128, 4096), "bf16"),
    ("paged-piece-4-f16", S.Shape(2048, 16, 4, 128, 4096), "f16"),
    ("paged-piece-2", S.Shape(8192, 64, 8, 128, 1024), "bf16"),
])
def test_paged_one_token_piece_gemv(label, shape, kv):
    """One sequence (one token per launch) with hidden 2048 or 8192: the QKV
    projection runs the piece-ordered kernel, whose epilogue (groups of 4
    features, or RoPE pairs at K = 8192) writes K and V through the block
    table; the new position opens a block."""
    run_paged_case(label, shape, "bf16", kv, [64], 128, 16, 157, oracle=True)


def test_paged_f32_cache_single_block():
    run_paged_case("paged-f32", S.TINY, "f32", "f32", [3, 20, 23], 24, 256, 153, oracle=True)


def test_paged_batch_over_32_and_full_table():
    # 40 sequences: two launch groups (32 + 8), the second reading its block
    # table rows from an offset; one context on the table's last position
    ctx = list(np.random.default_rng(4).integers(0, 255, 40))
    ctx[37] = 255
    run_paged_case("paged-b40", S.Shape(256, 4, 1, 64, 688), "bf16", "bf16", ctx, 256, 16, 155)


def test_paged_largest_block():
    run_paged_case("paged-bs1024", S.Shape(512, 8, 2, 128, 1376), "bf16", "f16", [100, 1500, 2047],
                   2048, 1024, 156)


def test_paged_70b_b32_full():
    """The benchmark's batched decode, 64-position blocks in a shuffled pool."""
    name = "decode_70b_b32_ragged"
    wl = S.WORKLOADS[name]
    say(f"[{name}] drawing inputs")
    stored, inp = S.workload_layer_and_inputs(name)
    run_paged_case(name + "-paged", wl.shape, wl.act_dtype, wl.kv_dtype, list(inp["ctx_len"]),
                   wl.s_max, 64, 154, stored=stored, inp=inp)


def run_paged_prefill_case(label, shape, act, kv, batch, tokens, start_pos, s_max, bs, seed):
    """Prefill over a paged cache whose first start_pos positions hold earlier
    tokens, against the same prefill on the contiguous cache: bit for bit."""
    say(f"[{label}] paged prefill B={batch} T={tokens} start={start_pos} s_max={s_max} block={bs} "
        f"{act}/{kv} {shape}")
    stored = random_layer(shape, act, seed)
    inp = S.draw_prefill_inputs(np.random.SeedSequence(seed + 1), shape, batch, tokens, s_max,
                                act, kv, start_pos)
    dl = DeviceLayer(shape, stored, act, kv, max_pos=s_max)
    x = to_dev(inp["x"], act)
    kc, vc = to_dev(inp["k_cache"], kv), to_dev(inp["v_cache"], kv)
    y_ref = dl.prefill(x, kc, vc, batch, tokens, start_pos, s_max)
    table, n_blocks, max_blocks = make_pages(batch, shape.n_kv_heads, s_max, shape.head_dim, bs,
                                             kv, seed + 7)
    fill = np.array(0x7FC0 if kv != "f32" else np.nan, dtype=STORAGE[kv])
    kp = to_dev(scatter(inp["k_cache"], table, n_blocks, bs, fill), kv)
    vp = to_dev(scatter(inp["v_cache"], table, n_blocks, bs, fill), kv)
    y = torch.full_like(x, float("nan"))
    ws = dl.workspace(batch, tokens, max_blocks * bs)
    B.llama_layer_prefill_paged(dl.cfg, dl.weights, x, y, kp, vp, bs,
                                torch.from_numpy(table).cuda(), batch, tokens, start_pos, ws)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(y), from_dev(y_ref)), f"{label}: paged prefill differs"
    view = torch.int16 if kv != "f32" else torch.float32
    gk = gather(kp.view(view).cpu().numpy().view(STORAGE[kv]), table, s_max)
    gv = gather(vp.view(view).cpu().numpy().view(STORAGE[kv]), table, s_max)
    rk = kc.view(view).cpu().numpy().view(STORAGE[kv])
    rv = vc.view(view).cpu().numpy().view(STORAGE[kv])
    new = slice(start_pos, start_pos + tokens)
    assert np.array_equal(gk[:, :, new], rk[:, :, new]) and np.array_equal(gv[:, :, new],
                                                                            rv[:, :, new])
    assert np.array_equal(gk[:, :, :start_pos], rk[:, :, :start_pos])
    say(f"[{label}] paged prefill == contiguous, bit for bit (output and appended entries)")


def test_paged_prefill_wide_hd128_chunked():
    # MFMA prefill (head_dim 128, DMA key tiles) after 200 cached positions, 2 sequences
    run_paged_prefill_case("paged-prefill-hd128", S.Shape(512, 8, 2, 128, 1032), "bf16", "bf16",
                           2, 300, 200, 512, 32, 170)


def test_paged_prefill_wide_hd64_f16():
    run_paged_prefill_case("paged-prefill-hd64", S.Shape(256, 4, 1, 64, 512), "bf16", "f16", 1,
                           150, 70, 256, 16, 171)


def test_paged_prefill_skinny():
    # 2 x 16 tokens: the token-skinny plan (decode attention kernels in prefill mode)
    run_paged_prefill_case("paged-prefill-16", S.Shape(256, 4, 2, 64, 688), "bf16", "bf16", 2, 16,
                           45, 96, 16, 172)


def test_kv_pages_write():
    r = np.random.default_rng(160)
    batch, nkv, s_max, hd, bs = 3, 2, 200, 128, 32
    for kv in ("bf16", "f32"):
        k = S.to_storage(r.standard_normal((batch, nkv, s_max, hd)).astype(np.float32), kv)
        v = S.to_storage(r.standard_normal((batch, nkv, s_max, hd)).astype(np.float32), kv)
        table, n_blocks, max_blocks = make_pages(batch, nkv, s_max, hd, bs, kv, 161)
        fill = np.array(0, dtype=STORAGE[kv])
        pool_k = np.full((n_blocks, nkv, bs, hd), fill, dtype=STORAGE[kv])
        kp, vp = to_dev(pool_k, kv), to_dev(pool_k.copy(), kv)
        B.llama_kv_pages_write(to_dev(k, kv), to_dev(v, kv), 37, 120, kp, vp, bs,
                               torch.from_numpy(table).cuda(), kv)
        torch.cuda.synchronize()
        # only positions 37..156 moved
        want_k = np.zeros_like(k)
        want_k[:, :, 37:157] = k[:, :, 37:157]
        view = torch.int16 if kv != "f32" else torch.float32
        got_k = gather(kp.view(view).cpu().numpy().view(STORAGE[kv]), table, s_max)
        got_v = gather(vp.view(view).cpu().numpy().view(STORAGE[kv]), table, s_max)
        want_v = np.zeros_like(v)
        want_v[:, :, 37:157] = v[:, :, 37:157]
        assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v), kv


@pytest.mark.parametrize("ctx", [[77], [5, 200, 33]], ids=["1-token", "3-tokens"])
def test_paged_branch_dominant(ctx):
    """x scaled by 2^-8 so the branches dominate the output; paged == contiguous
    bit for bit and the oracle's tolerance with no rounding allowance."""
    run_paged_case("paged-small-x-" + str(len(ctx)), S.Shape(512, 8, 2, 128, 1376), "bf16", "f16",
                   ctx, 256, 32, 190, oracle=True, x_scale=2.0 ** -8)
