"""The 80-layer 70B-shaped stack on one GPU: a 1024-token prompt prefill, then
128 greedy decode steps, all through the C ABI.

A full fp64 oracle of 80 layers does not fit in host memory, so the run is
checked where the oracle can follow it: on sampled layers (first, middle,
last) the layer's captured input, weights and cache are copied back and the
oracle recomputes that layer's prefill (sampled rows, every K/V entry) and its
first and last decode steps; the final hidden state goes through the oracle's
RMSNorm + LM head + argmax; the embedding of the prompt is checked exactly.
Tolerances as for the single layers (2e-2 in bf16).
"""
import gc

import numpy as np
import pytest
import torch

from gpu_util import TOL, check_errors, delta_error, from_dev, oracle_cfg, rel_err
from llama2_decoder_layer_amd import synth as S
from llama2_decoder_layer_amd.stack import device_stack
from oracle import llama_ref as R

pytestmark = pytest.mark.gpu

SAMPLED = (0, 39, 79)
ROWS = np.array([0, 1, 511, 1022, 1023])


def say(msg):
    print(msg, flush=True)


def layer64(d: dict) -> R.LayerWeights:
    return R.LayerWeights(**{k: from_dev(d[k]) for k in
                             ("attn_norm", "w_q", "w_k", "w_v", "w_o", "ffn_norm", "w_gate",
                              "w_up", "w_down")})


def test_stack_70b_80_layers():
    wl = S.WORKLOADS["stack_70b_80l"]
    s = wl.shape
    free, _ = torch.cuda.mem_get_info()
    if free < 150e9:
        pytest.skip(f"needs ~150 GB of free device memory, {free / 1e9:.0f} GB free")
    say(f"[{wl.name}] drawing {wl.n_layers} layers on the device")
    drawn = S.draw_stack_device(wl)
    stack = device_stack(s, wl.act_dtype, wl.kv_dtype, wl.s_max, drawn)
    prompt = torch.from_numpy(drawn["prompt"]).cuda()
    T, n_new = wl.prompt, wl.new_tokens
    last = n_new - 1
    say(f"[{wl.name}] prefill {T} tokens + {n_new} greedy decode steps")
    g = stack.begin(prompt, n_new, wl.s_max)
    g.prefill(capture=SAMPLED)
    for step in range(n_new):
        g.decode(step, capture=SAMPLED if step in (0, last) else ())
    torch.cuda.synchronize()
    ids = g.ids.cpu().numpy()
    say(f"[{wl.name}] ids[:12]={list(ids[:12])}")

    # embedding gather is exact
    x0 = g.captured[("prefill", 0)][0]
    assert torch.equal(x0, drawn["embed"][prompt.long()])

    cfg = oracle_cfg(s)
    act = wl.act_dtype
    for l in SAMPLED:
        say(f"[{wl.name}] layer {l}: oracle")
        w = layer64(drawn["layers"][l])
        kc_gpu, vc_gpu = (from_dev(c) for c in g.caches[l])
        # prefill: sampled rows of the output, every appended K/V entry
        x_in, y_out = (from_dev(t) for t in g.captured[("prefill", l)])
        kc64 = np.zeros((1, s.n_kv_heads, wl.s_max, s.head_dim))
        vc64 = np.zeros_like(kc64)
        want = R.layer_prefill(cfg, w, x_in[None], kc64, vc64, 0, out_rows=ROWS)[0]
        got = y_out[ROWS]
        d_err, d_allow = delta_error(got, want, x_in[ROWS], act)
        check_errors(f"layer {l} prefill", {
            "out": rel_err(got, want), "delta": d_err,
            "k_all": rel_err(kc_gpu[:, :, :T], kc64[:, :, :T]),
            "v_all": rel_err(vc_gpu[:, :, :T], vc64[:, :, :T])}, TOL[act], {"delta": d_allow})
        # decode steps: the cache before the step is what the GPU holds below its position
        for step in (0, last):
            pos = T + step
            x_in, y_out = (from_dev(t) for t in g.captured[(step, l)])
            kc = kc_gpu.copy()
            vc = vc_gpu.copy()
            kc[:, :, pos:] = 0.0
            vc[:, :, pos:] = 0.0
            want = R.layer_decode(cfg, w, x_in, kc, vc, np.array([pos]))
            d_err, d_allow = delta_error(y_out, want, x_in, act)
            check_errors(f"layer {l} decode step {step}", {
                "out": rel_err(y_out, want), "delta": d_err,
                "k_new": rel_err(kc_gpu[:, :, pos], kc[:, :, pos]),
                "v_new": rel_err(vc_gpu[:, :, pos], vc[:, :, pos])}, TOL[act], {"delta": d_allow})
        del w, kc_gpu, vc_gpu
        gc.collect()

    say(f"[{wl.name}] head")
    h = from_dev(g.last_hidden)
    want_logits = R.lm_head(h, from_dev(drawn["final_norm"]), from_dev(drawn["w_lm"]), s.eps)
    got_logits = from_dev(g.logits[n_new:n_new + 1])
    err = rel_err(got_logits, want_logits)
    srt = np.sort(want_logits[0])
    gap = (srt[-1] - srt[-2]) / np.max(np.abs(want_logits))
    say(f"[{wl.name}] head logits err={err:.2e}, top1-top2 gap={gap:.2e}")
    assert err < TOL[act]
    if gap > 10 * TOL[act]:
        assert int(ids[n_new]) == int(R.greedy(want_logits)[0])
    # every id is the argmax (lowest index on ties) of the logits the GPU produced
    lg = g.logits.cpu().numpy()
    assert np.array_equal(ids, np.argmax(lg, axis=1).astype(np.int32))
    del g, stack, drawn
    gc.collect()
    torch.cuda.empty_cache()
