"""GPU parity of weight-only INT4: llama_quantize_w4's packed codes and scales
bit for bit against the oracle's (both decide in float32), then
llama_layer_decode_w4 against the oracle's layer computed with the oracle's own
dequantised weights, at the bf16/f16 tolerance (2e-2) and the float32 one
(1e-4)."""
import numpy as np
import pytest
import torch

from gpu_util import (TOL, check_errors, delta_error, from_dev, oracle_cfg, random_layer,
                      rel_err, scale_stored, to_dev)
from llama2_decoder_layer_amd import binding as B
from llama2_decoder_layer_amd import synth as S
from oracle import llama_ref as R

pytestmark = pytest.mark.gpu

PROJ = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")
SCALE = {"w_q": "s_q", "w_k": "s_k", "w_v": "s_v", "w_o": "s_o", "w_gate": "s_gate",
         "w_up": "s_up", "w_down": "s_down"}


def say(msg):
    print(msg, flush=True)


def unpack_w4(packed: np.ndarray) -> np.ndarray:
    """[rows, cols/2] bytes -> [rows, cols] int8 codes (column 2j in the low
    nibble of byte j, two's complement)."""
    p = packed.astype(np.int16)
    lo, hi = p & 15, p >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((p.shape[0], 2 * p.shape[1]), np.int8)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out


def device_w4_layer(shape, stored, act, max_pos):
    """Upload the layer, quantise its projections on the device, keep the rest."""
    dev = {}
    for k, v in stored.items():
        if k in PROJ:
            w = to_dev(v, act)
            q = torch.empty(w.shape[0], w.shape[1] // 2, dtype=torch.uint8, device="cuda")
            sc = torch.empty(w.shape[0], dtype=torch.float32, device="cuda")
            B.llama_quantize_w4(w, q, sc, act)
            dev[k], dev[SCALE[k]] = q, sc
        else:
            dev[k] = to_dev(v, act)
    half = shape.head_dim // 2
    dev["rope_cos"] = torch.empty(max_pos, half, dtype=torch.float32, device="cuda")
    dev["rope_sin"] = torch.empty(max_pos, half, dtype=torch.float32, device="cuda")
    B.llama_rope_table(dev["rope_cos"], dev["rope_sin"], max_pos, shape.head_dim, shape.rope_theta)
    torch.cuda.synchronize()
    return B.LayerWeightsW4(dev)


def oracle_w4_weights(stored, act):
    """The oracle's own quantisation of the stored weights, dequantised."""
    out = {}
    for k, v in stored.items():
        w = S.to_f64(v, act)
        if k in PROJ:
            q, sc = R.quantize_w4_rows(w.astype(np.float32))
            out[k] = R.dequantize_w4(q, sc)
        else:
            out[k] = w
    return R.LayerWeights(**out)


def run_w4_decode(label, shape, act, kv, ctx_len, s_max, seed, stored=None, inp=None,
                  x_scale=1.0):
    batch = len(ctx_len)
    say(f"[{label}] w4 decode B={batch} ctx={[int(c) for c in ctx_len][:8]} s_max={s_max} "
        f"{act}/{kv} {shape}")
    if stored is None:
        stored = random_layer(shape, act, seed)
    if inp is None:
        inp = S.draw_decode_inputs(np.random.SeedSequence(seed + 1), shape, batch, s_max, act, kv,
                                   ctx=0)
    if x_scale != 1.0:
        inp = dict(inp, x=scale_stored(inp["x"], act, x_scale))
    ctx = np.asarray(ctx_len, dtype=np.int32)
    lw = device_w4_layer(shape, stored, act, s_max)
    cfg = B.make_config(shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                        shape.intermediate, shape.eps, shape.rope_theta, act, kv, s_max)
    x = to_dev(inp["x"], act)
    y = torch.full_like(x, float("nan"))
    kc, vc = to_dev(inp["k_cache"], kv), to_dev(inp["v_cache"], kv)
    ws = torch.full((B.llama_layer_workspace_size(cfg, batch, 1, s_max),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    B.llama_layer_decode_w4(cfg, lw, x, y, kc, vc, torch.from_numpy(ctx).cuda(), batch,
                            int(ctx.max()), s_max, ws)
    torch.cuda.synchronize()
    x64 = S.to_f64(inp["x"], act)
    kc64, vc64 = S.to_f64(inp["k_cache"], kv), S.to_f64(inp["v_cache"], kv)
    want = R.layer_decode(oracle_cfg(shape), oracle_w4_weights(stored, act), x64, kc64, vc64, ctx)
    got = from_dev(y)
    bi = np.arange(batch)
    d_err, d_allow = delta_error(got, want, x64, act)
    errs = {"out": rel_err(got, want), "delta": d_err,
            "k_new": rel_err(from_dev(kc)[bi, :, ctx], kc64[bi, :, ctx]),
            "v_new": rel_err(from_dev(vc)[bi, :, ctx], vc64[bi, :, ctx])}
    check_errors(label, errs, TOL[act], {"delta": d_allow})


@pytest.mark.parametrize("act,rows,cols", [("bf16", 300, 704), ("f16", 129, 1376),
                                           ("f32", 64, 256), ("bf16", 4096, 11008)])
def test_quantize_w4_bit_exact(act, rows, cols):
    r = np.random.default_rng(rows + cols + 4)
    w = (r.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[1] = 0.0                      # zero row
    w[2, :] = 0.0
    w[2, 7] = -0.3                  # a single non-zero weight
    w[3, :cols // 2] = 0.0127       # many equal magnitudes
    stored = S.to_storage(w, act)
    dw = to_dev(stored, act)
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty(rows, dtype=torch.float32, device="cuda")
    B.llama_quantize_w4(dw, q, sc, act)
    torch.cuda.synchronize()
    wq, wsc = R.quantize_w4_rows(S.to_f64(stored, act).astype(np.float32))
    gq, gsc = unpack_w4(q.cpu().numpy()), sc.cpu().numpy()
    say(f"[quantize-w4 {act} {rows}x{cols}] codes differ at {int(np.sum(gq != wq))} places")
    assert np.array_equal(gsc.view(np.uint32), wsc.view(np.uint32))
    assert np.array_equal(gq, wq)


def test_w4_decode_gqa_ragged_groups():
    # 6 sequences: groups of 4 and 2; GQA 4:1, f16 cache, several attention chunks
    run_w4_decode("w4-gqa", S.Shape(512, 8, 2, 128, 1376), "bf16", "f16",
                  [0, 1, 63, 300, 511, 130], 512, 150)


def test_w4_decode_f16_and_f32():
    run_w4_decode("w4-f16", S.Shape(256, 4, 4, 64, 768), "f16", "f16", [10, 129], 160, 151)
    run_w4_decode("w4-f32", S.Shape(256, 4, 2, 64, 704), "f32", "f32", [3, 17, 23], 24, 152)


def test_w4_decode_large_activation_stage():
    # intermediate 28672 (the 70B width): two tokens' down-projection
    # activations take 112 KB of LDS; K = 28672 is 14 chunks of 2048 codes
    run_w4_decode("w4-wide-I", S.Shape(256, 4, 2, 64, 28672), "bf16", "bf16", [5, 40, 77], 96,
                  153)


def test_w4_decode_7b_full():
    """The INT4 benchmark case: the 7B layer at context 4096."""
    name = "decode_7b_b1_ctx4096_w4"
    wl = S.WORKLOADS[name]
    say(f"[{name}] drawing inputs")
    stored, inp = S.workload_layer_and_inputs(name)
    run_w4_decode(name, wl.shape, wl.act_dtype, wl.kv_dtype, list(inp["ctx_len"]), wl.s_max, 0,
                  stored=stored, inp=inp)


@pytest.mark.parametrize("ctx", [[77], [5, 200, 33]], ids=["1-token", "3-tokens"])
def test_w4_decode_branch_dominant(ctx):
    """x scaled by 2^-8: the branches dominate the output, so the output
    tolerance checks the quantised projections with no rounding allowance."""
    run_w4_decode("w4-small-x-" + str(len(ctx)), S.Shape(512, 8, 2, 128, 1376), "bf16", "bf16", ctx,
                  256, 185, x_scale=2.0 ** -8)
