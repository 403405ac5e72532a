"""llama_layer_decode_noalloc (built-in device scratch, no workspace argument)
against llama_layer_decode through the C ABI: the same kernels, so outputs
and caches must agree bit for bit.  Two calls in a row, the second smaller
(fewer sequences, shorter contexts), show that the scratch keeps no state a
call depends on; the full-size cases are the 7B batch-1 and 70B batch-32
decodes.  Each result is also held to the oracle's tolerance."""
import numpy as np
import pytest
import torch

from gpu_util import (TOL, DeviceLayer, check_errors, delta_error, from_dev, oracle_cfg,
                      oracle_weights, random_layer, rel_err, to_dev)
from llama2_decoder_layer_amd import binding as B
from llama2_decoder_layer_amd import synth as S
from oracle import llama_ref as R

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _pair(dl, inp, ctx, act, kv, s_max):
    """(noalloc output, caches) and (workspace output, caches) on fresh copies."""
    batch = len(ctx)
    dctx = torch.from_numpy(np.asarray(ctx, np.int32)).cuda()
    x = to_dev(inp["x"], act)
    outs = []
    for which in ("noalloc", "ws"):
        kc, vc = to_dev(inp["k_cache"], kv), to_dev(inp["v_cache"], kv)
        y = torch.full_like(x, float("nan"))
        if which == "noalloc":
            B.llama_layer_decode_noalloc(dl.cfg, dl.weights, x, y, kc, vc, dctx, batch,
                                         int(max(ctx)), s_max)
        else:
            ws = dl.workspace(batch, 1, s_max)
            B.llama_layer_decode(dl.cfg, dl.weights, x, y, kc, vc, dctx, batch, int(max(ctx)),
                                 s_max, ws)
        outs.append((y, kc, vc))
    torch.cuda.synchronize()
    return outs


def _compare(label, dl, stored, inp, ctx, act, kv, s_max, shape, oracle=True):
    (y0, k0, v0), (y1, k1, v1) = _pair(dl, inp, ctx, act, kv, s_max)
    assert torch.equal(y0.view(torch.int16) if act != "f32" else y0,
                       y1.view(torch.int16) if act != "f32" else y1), f"{label}: outputs differ"
    for a, b in ((k0, k1), (v0, v1)):
        assert torch.equal(a.view(torch.int16) if kv != "f32" else a,
                           b.view(torch.int16) if kv != "f32" else b), f"{label}: caches differ"
    say(f"[{label}] noalloc == workspace decode, bit for bit (B={len(ctx)}, max ctx {max(ctx)})")
    if not oracle:
        return
    c = np.asarray(ctx, np.int32)
    x64 = S.to_f64(inp["x"], act)
    want = R.layer_decode(oracle_cfg(shape), oracle_weights(stored, act), x64,
                          S.to_f64(inp["k_cache"], kv), S.to_f64(inp["v_cache"], kv), c)
    got = from_dev(y0)
    d_err, d_allow = delta_error(got, want, x64, act)
    check_errors(label, {"out": rel_err(got, want), "delta": d_err}, TOL[act], {"delta": d_allow})


@pytest.mark.parametrize("act,kv", [("bf16", "f16"), ("f32", "f32")])
def test_noalloc_two_calls_second_smaller(act, kv):
    shape, s_max = S.Shape(512, 8, 2, 128, 1376), 600
    stored = random_layer(shape, act, 200)
    dl = DeviceLayer(shape, stored, act, kv, max_pos=s_max)
    for label, batch, seed, ctx in (("first", 40, 201, None), ("second", 3, 202, [7, 150, 0])):
        if ctx is None:
            ctx = list(np.random.default_rng(seed).integers(0, s_max - 1, batch))
        inp = S.draw_decode_inputs(np.random.SeedSequence(seed), shape, len(ctx), s_max, act, kv,
                                   ctx=0)
        _compare(f"noalloc-{act}-{label}", dl, stored, inp, ctx, act, kv, s_max, shape)


@pytest.mark.parametrize("name", ["decode_7b_b1_ctx4096", "decode_70b_b32_ragged"])
def test_noalloc_full_size(name):
    wl = S.WORKLOADS[name]
    say(f"[{name}] drawing")
    stored, inp = S.workload_layer_and_inputs(name)
    dl = DeviceLayer(wl.shape, stored, wl.act_dtype, wl.kv_dtype, max_pos=wl.s_max)
    _compare(f"noalloc-{name}", dl, stored, inp, list(inp["ctx_len"]), wl.act_dtype, wl.kv_dtype,
             wl.s_max, wl.shape, oracle=False)
    # then a smaller call on the same scratch: at most 2 sequences, shorter contexts
    nb = min(2, wl.batch)
    small = {k: v for k, v in inp.items()}
    small["x"] = inp["x"][:nb].copy()
    small["k_cache"], small["v_cache"] = inp["k_cache"][:nb].copy(), inp["v_cache"][:nb].copy()
    ctx = [100, 37][:nb]
    _compare(f"noalloc-{name}-small", dl, stored, small, ctx, wl.act_dtype, wl.kv_dtype,
             wl.s_max, wl.shape)


def test_noalloc_rejects_beyond_scratch():
    shape = S.L70B
    stored = random_layer(S.Shape(256, 4, 2, 64, 688), "bf16", 203)  # any valid pointers
    dl = DeviceLayer(S.Shape(256, 4, 2, 64, 688), stored, "bf16", "bf16", max_pos=64)
    cfg = B.make_config(shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                        shape.intermediate, shape.eps, shape.rope_theta, "bf16", "f16", 4097)
    batch = 1024
    x = torch.zeros(batch, shape.hidden, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    ctx = torch.zeros(batch, dtype=torch.int32, device="cuda")
    kc = torch.empty(16, dtype=torch.float16, device="cuda")  # never touched: refused first
    with pytest.raises(B.LlamaLayerError, match="LL_ESCRATCH"):
        B.llama_layer_decode_noalloc(cfg, dl.weights, x, y, kc, kc, ctx, batch, 4096, 4097)
