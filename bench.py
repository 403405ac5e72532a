"""Benchmark of the decoder layer on one MI355X.

Default workload: the 80-layer 70B-shaped stack at batch 1 (1024-token prompt,
then greedy decode).  A step is one decode token through every layer and the
LM head; value = decode tokens/s over exactly --steps steps timed between
synchronisations, with no events in that loop.  The line also carries the
median step and the roofline of the dominant decode kernel (the gate/up GEMV,
timed with HIP events handed to its dispatches), both from a second pass over
the same steps, the stack's algorithmic HBM rate, the prompt prefill's time to
first token and TFLOP/s (median of --prefills runs), HBM read/copy and
bf16 MFMA rates measured on the GPU beside the published peaks, and the fp64
oracle timed on the host's cores (an extrapolation from one layer).

--workload selects a single-layer workload instead (a step is one layer call;
decode: tokens/s per layer; prefill: TFLOP/s) or the sampling head.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s per layer (HBM GB/s %) and prefill TFLOP/s (MFMA %), 1 GPU"
HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA


def layer_weight_elems(s) -> int:
    H, nh, nkv, hd, I = s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate
    return (nh + 2 * nkv) * hd * H + H * nh * hd + 2 * I * H + H * I


def decode_bytes(s, ctx_len, act_b, kv_b, wbits=16) -> dict:
    """Algorithmic HBM bytes of one decode call: each weight once (INT8: one
    byte per weight, INT4 half a byte, and a float32 scale per row), each
    cached K/V entry that is attended once, the new K/V entries, x, y and the
    gains."""
    B = len(ctx_len)
    kv_read = int(np.sum(np.asarray(ctx_len, np.int64) + 1)) * s.n_kv_heads * s.head_dim * 2 * kv_b
    if wbits in (8, 4):
        rows = (s.n_heads + 2 * s.n_kv_heads) * s.head_dim + s.hidden + 2 * s.intermediate + s.hidden
        w = layer_weight_elems(s) * wbits // 8 + 4 * rows
        gate_up = 2 * s.intermediate * s.hidden * wbits // 8 + 4 * 2 * s.intermediate
    else:
        w = layer_weight_elems(s) * act_b
        gate_up = 2 * s.intermediate * s.hidden * act_b
    small = B * s.hidden * act_b * 2 + 2 * s.hidden * act_b + B * 2 * s.n_kv_heads * s.head_dim * kv_b
    gate_up += B * (s.hidden + s.intermediate) * act_b
    return {"total": w + kv_read + small, "weights": w, "kv_read": kv_read, "gemv_gate_up": gate_up,
            "attn_decode": kv_read}


def prefill_flops(s, T) -> dict:
    H, nh, nkv, hd, I = s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate
    f = {"qkv": 2 * T * H * (nh + 2 * nkv) * hd, "o": 2 * T * nh * hd * H,
         "gate_up": 2 * T * H * 2 * I, "down": 2 * T * I * H,
         "attention": 4 * hd * nh * T * (T + 1) // 2}
    f["total"] = sum(f.values())
    return f


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_baseline_decode(wl, stored, inp, budget_s: float) -> dict:
    """The fp64 oracle (as it stands) on the same decode workload, repeated
    until `budget_s` seconds of CPU work have run."""
    from llama2_decoder_layer_amd import synth as S
    from oracle import llama_ref as R
    s = wl.shape
    theta = s.rope_theta
    if "ntk_scale" in wl.extra:
        theta = R.ntk_rope_base(theta, wl.extra["ntk_scale"], s.head_dim)
    cfg = R.LayerConfig(s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.eps,
                        theta)
    w = {k: S.to_f64(v, wl.act_dtype) for k, v in stored.items()}
    if wl.extra.get("w8"):
        for k in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down"):
            w[k] = R.dequantize_w8(*R.quantize_w8_rows(w[k].astype(np.float32)))
    if wl.extra.get("w4"):
        for k in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down"):
            w[k] = R.dequantize_w4(*R.quantize_w4_rows(w[k].astype(np.float32)))
    w = R.LayerWeights(**w)
    B = wl.batch
    nb = B if B <= 4 else 4  # bounded sample: the first sequences of the batch
    kc = S.to_f64(inp["k_cache"][:nb], wl.kv_dtype)
    vc = S.to_f64(inp["v_cache"][:nb], wl.kv_dtype)
    x = S.to_f64(inp["x"][:nb], wl.act_dtype)
    ctx = inp["ctx_len"][:nb]
    n = 0
    t0 = time.perf_counter()
    while True:
        R.layer_decode(cfg, w, x, kc, vc, ctx)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": n * nb / el, "unit": "tokens/s/layer", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{n} oracle decode calls of {nb} sequence(s) of this workload in {el:.1f} s"}


def cpu_baseline_prefill(wl, stored, inp, budget_s: float) -> dict:
    from llama2_decoder_layer_amd import synth as S
    from oracle import llama_ref as R
    s = wl.shape
    cfg = R.LayerConfig(s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.eps,
                        s.rope_theta)
    w = R.LayerWeights(**{k: S.to_f64(v, wl.act_dtype) for k, v in stored.items()})
    T = 64
    while True:  # grow the prompt until one prefill takes a measurable share of the budget
        x = S.to_f64(inp["x"][:1, :T], wl.act_dtype)
        kc = np.zeros((1, s.n_kv_heads, T, s.head_dim))
        vc = np.zeros_like(kc)
        t0 = time.perf_counter()
        R.layer_prefill(cfg, w, x, kc, vc, 0)
        el = time.perf_counter() - t0
        if el > budget_s / 4 or T >= wl.tokens:
            break
        T = min(wl.tokens, T * 2)
    fl = prefill_flops(s, T)["total"]
    return {"value": fl / el / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"one oracle prefill of the first {T} tokens of this workload in {el:.1f} s"}


def cpu_baseline_stack(wl, drawn, budget_s: float) -> dict:
    """The oracle on one layer of the stack (layer 0's weights copied back)
    decoding at the prompt's end, plus the LM head, extrapolated to every layer."""
    from oracle import llama_ref as R
    import torch
    s = wl.shape
    f64 = lambda t: t.detach().to(torch.float64).cpu().numpy()
    cfg = R.LayerConfig(s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.eps,
                        s.rope_theta)
    w = R.LayerWeights(**{k: f64(v) for k, v in drawn["layers"][0].items()})
    rng = np.random.default_rng(0)
    kc = rng.standard_normal((1, s.n_kv_heads, wl.s_max, s.head_dim))
    vc = rng.standard_normal(kc.shape)
    x = rng.standard_normal((1, s.hidden))
    ctx = np.array([wl.prompt])
    n, t0 = 0, time.perf_counter()
    while True:
        R.layer_decode(cfg, w, x, kc, vc, ctx)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    t_layer = el / n
    w_lm, gf = f64(drawn["w_lm"]), f64(drawn["final_norm"])
    t1 = time.perf_counter()
    R.greedy(R.lm_head(x, gf, w_lm, s.eps))
    t_head = time.perf_counter() - t1
    per_tok = wl.n_layers * t_layer + t_head
    return {"value": 1.0 / per_tok, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"extrapolation: {n} oracle decode calls of layer 0 at context {wl.prompt} "
                      f"({t_layer * 1e3:.0f} ms each) x {wl.n_layers} layers + one LM head "
                      f"({t_head * 1e3:.0f} ms)"}


def median(xs):
    return float(np.median(np.asarray(xs, dtype=np.float64)))


class StepEvents:
    """HIP events on torch's current stream (the stream the library launches
    on) between consecutive steps, for the median step time."""

    def __init__(self, n):
        import torch
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        self.i = 0

    def mark(self):
        self.ev[self.i].record()
        self.i += 1

    def times_ms(self):
        return [self.ev[i].elapsed_time(self.ev[i + 1]) for i in range(self.i - 1)]


def measured_peaks() -> dict:
    """HBM read and copy rates and the bf16 MFMA rate measured on this GPU with
    the library's peak kernels (median of 5 runs each), beside the published
    peaks the roofline fractions use."""
    import torch
    from llama2_decoder_layer_amd import binding as B
    gib = 1 << 30
    src = torch.ones(4 * gib // 4, dtype=torch.int32, device="cuda")   # 4 GiB >> the 256 MB MALL
    dst = torch.empty(2 * gib // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    out = torch.empty(131072, dtype=torch.float32, device="cuda")

    def timed(fn, n=5):
        fn()  # warm
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return median(ts)

    read_ms = timed(lambda: B.llama_peak_read(src, sink))
    copy_ms = timed(lambda: B.llama_peak_copy(dst, src[:dst.numel()]))
    iters = 4096
    flops = B.llama_peak_mfma_bf16(out, iters)
    torch.cuda.synchronize()
    mfma_ms = timed(lambda: B.llama_peak_mfma_bf16(out, iters))
    res = {"hbm_read_GBps": 4 * gib / (read_ms / 1e3) / 1e9,
           "hbm_copy_GBps": 2 * 2 * gib / (copy_ms / 1e3) / 1e9,
           "mfma_bf16_TFLOPs": flops / (mfma_ms / 1e3) / 1e12,
           "spec_hbm_GBps": HBM_PEAK_GBPS, "spec_mfma_bf16_TFLOPs": BF16_PEAK_TFLOPS,
           "how": "llama_peak_read (4 GiB), llama_peak_copy (2 GiB each way), "
                  "llama_peak_mfma_bf16 (32x32x16 bf16 chains on registers); median of 5"}
    del src, dst, sink, out
    torch.cuda.empty_cache()
    return res


def bench_stack(args, wl):
    """The 80-layer stack at batch 1.  A warm-up generation (prefill and `warmup`
    decode steps); then the prompt's prefill `--prefills` times (time to first
    token: the median), then exactly `steps` decode steps, timed between
    synchronisations with nothing else on the stream (value = decode
    tokens/s).  A second generation of the same prompt then decodes the same
    positions again with an event between steps (the median step) and the
    gate/up launches bracketed by their own events (the roofline kernel): on
    the 7B layer those events cost ~4% of a step, so they stay out of the
    timed loop."""
    import torch
    from llama2_decoder_layer_amd import binding as B
    from llama2_decoder_layer_amd import synth as S
    from llama2_decoder_layer_amd.profiling import load_traffic
    from llama2_decoder_layer_amd.stack import device_stack
    s = wl.shape
    steps = min(args.steps, wl.new_tokens)
    warm = min(args.warmup, wl.new_tokens)
    print(f"[bench] drawing {wl.n_layers} layers on the device", file=sys.stderr, flush=True)
    drawn = S.draw_stack_device(wl)
    stack = device_stack(s, wl.act_dtype, wl.kv_dtype, wl.s_max, drawn)
    prompt = torch.from_numpy(drawn["prompt"]).cuda()
    print(f"[bench] warm-up: prefill + {warm} decode steps", file=sys.stderr, flush=True)
    g = stack.begin(prompt, wl.new_tokens, wl.s_max)
    g.prefill()
    for i in range(warm):
        g.decode(i)
    torch.cuda.synchronize()
    del g
    g = stack.begin(prompt, wl.new_tokens, wl.s_max)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.prefills} prefills", file=sys.stderr, flush=True)
    pre_ms = []
    for _ in range(args.prefills):  # idempotent: rewrites the prompt's cache entries
        ev = StepEvents(1)
        ev.mark()
        g.prefill()
        ev.mark()
        torch.cuda.synchronize()
        pre_ms += ev.times_ms()
    t_prefill = median(pre_ms) / 1e3
    print(f"[bench] timing {steps} decode steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        g.decode(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(f"[bench] {steps} decode steps again, with events", file=sys.stderr, flush=True)
    g2 = stack.begin(prompt, wl.new_tokens, wl.s_max)
    g2.prefill()
    kid = B.kernel_id("gemv_gate_up")
    B.llama_layer_timer_start(kid, wl.n_layers * steps)
    ev = StepEvents(steps)
    for i in range(steps):
        ev.mark()
        g2.decode(i)
    ev.mark()
    torch.cuda.synchronize()
    kms, kn = B.llama_layer_timer_stop()
    step_ms = ev.times_ms()
    del g2
    ms_tok = el * 1e3 / steps
    act_b = S.DTYPE_BYTES[wl.act_dtype]
    kv_b = S.DTYPE_BYTES[wl.kv_dtype]
    ctx_mean = wl.prompt + (steps - 1) / 2
    per_layer = decode_bytes(s, [ctx_mean], act_b, kv_b)
    head = wl.vocab * s.hidden * act_b + s.hidden * act_b
    tok_bytes = wl.n_layers * per_layer["total"] + head
    gbps = tok_bytes / (ms_tok / 1e3) / 1e9
    kavg_s = kms / 1e3 / max(kn, 1)
    ach = per_layer["gemv_gate_up"] / kavg_s / 1e9
    fl = wl.n_layers * prefill_flops(s, wl.prompt)["total"]
    tr = load_traffic("gemv_gate_up", wl.name)
    out = {"metric": METRIC, "value": steps / el, "unit": "tokens/s", "n_gpus": 1,
           "steps": steps, "warmup": warm, "ms_per_step": ms_tok,
           "ms_per_step_median": median(step_ms), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": wl.act_dtype,
           "data": "synthetic (device-drawn seeded weights; see synth.py)",
           "layer_steps_per_s": wl.n_layers * steps / el,
           "stack_hbm": {"bytes_per_token": int(tok_bytes), "GBps": gbps,
                         "frac_of_peak": gbps / HBM_PEAK_GBPS},
           "prefill": {"tokens": wl.prompt, "time_to_first_token_ms": t_prefill * 1e3,
                       "runs_ms": pre_ms, "flops": fl, "TFLOPs": fl / t_prefill / 1e12,
                       "frac_of_peak": fl / t_prefill / 1e12 / BF16_PEAK_TFLOPS},
           "roofline": {"bound": "hbm", "kernel": "gemv_gate_up", "achieved": ach,
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                        "traffic": None if tr is None else tr["bytes"],
                        "algorithmic_bytes_per_launch": per_layer["gemv_gate_up"],
                        "avg_launch_us": kavg_s * 1e6, "launches_timed": kn},
           "config": {"workload": wl.name, "layers": wl.n_layers, "hidden": s.hidden,
                      "n_heads": s.n_heads, "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                      "intermediate": s.intermediate, "vocab": wl.vocab, "batch": 1,
                      "prompt": wl.prompt, "kv_dtype": wl.kv_dtype},
           "ids_head": [int(i) for i in g.ids[:8].cpu()]}
    del g
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    if not args.no_peaks:
        print("[bench] measuring HBM and MFMA peaks", file=sys.stderr, flush=True)
        out["measured_peaks"] = measured_peaks()
    if args.no_cpu_baseline:
        out["cpu_baseline"] = None
    else:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_stack(wl, drawn, args.cpu_budget)
    print(json.dumps(out), flush=True)


def copy_calibration(mib: int) -> None:
    """Three device-to-device copies of `mib` MiB: the known-size reference
    that scales the HBM byte counters of a counter run."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def paged_pools(inp, bs, seed):
    """The contiguous caches of a decode workload laid out as the blocks of a
    paged cache, in shuffled pool order: (k_pool, v_pool, block_table)."""
    batch, nkv, s_max, hd = inp["k_cache"].shape
    max_blocks = -(-s_max // bs)
    table = np.random.default_rng(seed).permutation(batch * max_blocks).reshape(batch, max_blocks)
    pools = []
    for name in ("k_cache", "v_cache"):
        c = inp[name]
        pool = np.zeros((batch * max_blocks, nkv, bs, hd), dtype=c.dtype)
        for b in range(batch):
            for i in range(max_blocks):
                lo, hi = i * bs, min((i + 1) * bs, s_max)
                pool[table[b, i], :, :hi - lo] = c[b, :, lo:hi]
        pools.append(pool)
    return pools[0], pools[1], table.astype(np.int32)


def bench_sample(args, wl):
    """Sampling after the LM head: one step = one llama_sample call over the
    batch.  The logits come straight from the LM head in a real step, so one
    resident copy is timed (it is 4 MB)."""
    import torch
    from llama2_decoder_layer_amd import binding as B
    from llama2_decoder_layer_amd import synth as S
    e = wl.extra
    inp = S.draw_sample_inputs(wl.name)
    logits = torch.from_numpy(inp["logits"]).cuda()
    hist = torch.from_numpy(inp["history"]).cuda()
    u = torch.from_numpy(inp["u"]).cuda()
    ids = torch.empty(wl.batch, dtype=torch.int32, device="cuda")

    def step():
        B.llama_sample(logits, hist, u, ids, e["temperature"], e["top_k"], e["top_p"], e["penalty"])
    for _ in range(args.warmup):
        step()
    # Timed loop without events, then the same calls with the kernel's own
    # events (the roofline), as for the layer workloads.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    kid = B.kernel_id("sample")
    B.llama_layer_timer_start(kid, args.steps)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kms, kn = B.llama_layer_timer_stop()
    ms_step = el * 1e3 / args.steps
    kavg_s = kms / 1e3 / max(kn, 1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    nbytes = wl.batch * (wl.vocab * 4 + e["n_hist"] * 4 + 4 + 4)
    from llama2_decoder_layer_amd.profiling import load_traffic
    tr = load_traffic("sample", wl.name)
    ach = nbytes / kavg_s / 1e9
    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded; see synth.py)",
           "value": wl.batch / (ms_step / 1e3), "unit": "tokens/s",
           "roofline": {"bound": "hbm", "kernel": "sample", "achieved": ach,
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                        "traffic": None if tr is None else tr["bytes"],
                        "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": kavg_s * 1e6,
                        "launches_timed": kn},
           "config": {"workload": wl.name, "batch": wl.batch, "vocab": wl.vocab, **e}}
    if args.no_cpu_baseline:
        out["cpu_baseline"] = None
    else:
        from oracle import llama_ref as R
        lg = inp["logits"].astype(np.float64)
        u64 = inp["u"].astype(np.float64)
        n, t0 = 0, time.perf_counter()
        while True:
            R.sample(lg, inp["history"], u64, e["temperature"], e["top_k"], e["top_p"],
                     e["penalty"])
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_budget:
                break
        out["cpu_baseline"] = {"value": n * wl.batch / el, "unit": "tokens/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{n} oracle calls over the {wl.batch} rows in {el:.1f} s"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 32 decode tokens for the stack, 200 layer calls)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 4 for the stack, 20 layer calls)")
    ap.add_argument("--workload", default="stack_70b_80l",
                    choices=["decode_7b_b1_ctx4096", "decode_70b_b32_ragged", "prefill_13b_t4096",
                             "stack_70b_80l", "decode_7b_b1_ctx32768_ntk8",
                             "sample_b32_v32000", "decode_7b_b1_ctx4096_w8",
                             "decode_70b_b32_ragged_paged", "decode_70b_b32_ragged_w8",
                             "decode_7b_b1_ctx4096_w4"])
    ap.add_argument("--copies", type=int, default=0,
                    help="distinct weight/cache copies cycled through (0 = enough to exceed the MALL)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured HBM/MFMA peaks (stack workload)")
    ap.add_argument("--time-kernel", default=None, metavar="NAME",
                    help="single-layer workloads: kernel the roofline block times (default: the "
                         "dominant one; names as llama_layer_kernel_name)")
    ap.add_argument("--prefills", type=int, default=3,
                    help="stack workload: prompt prefills timed (time to first token: median)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run 3 device-to-device copies of MIB MiB (the "
                         "known-size reference that scales the HBM byte counters)")
    args = ap.parse_args()
    stack_wl = args.workload == "stack_70b_80l"
    if args.steps is None:
        args.steps = 32 if stack_wl else 200
    if args.warmup is None:
        args.warmup = 4 if stack_wl else 20
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from llama2_decoder_layer_amd import binding as B
    from llama2_decoder_layer_amd import synth as S

    wl = S.WORKLOADS[args.workload]
    if wl.phase == "stack":
        bench_stack(args, wl)
        return
    if wl.phase == "sample":
        bench_sample(args, wl)
        return
    s = wl.shape
    act, kvd = wl.act_dtype, wl.kv_dtype
    act_b, kv_b = S.DTYPE_BYTES[act], S.DTYPE_BYTES[kvd]
    print(f"[bench] drawing {wl.name}", file=sys.stderr, flush=True)
    stored, inp = S.workload_layer_and_inputs(wl.name)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

    def dev(a, dt):
        a = np.ascontiguousarray(a)
        if dt == "f32":
            return torch.from_numpy(a).cuda()
        return torch.from_numpy(a.view(np.int16)).cuda().view(tdt[dt])

    wbits = 8 if wl.extra.get("w8") else 4 if wl.extra.get("w4") else 16
    per_copy = (layer_weight_elems(s) * wbits // 8 if wbits < 16 else
                layer_weight_elems(s) * act_b) + \
        2 * inp["k_cache"].size * kv_b
    copies = args.copies or max(1, min(8, -(-1_500_000_000 // per_copy)))
    max_pos = wl.s_max
    cfg = B.make_config(s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.eps,
                        s.rope_theta, act, kvd, max_pos)
    rc = torch.empty(max_pos, s.head_dim // 2, dtype=torch.float32, device="cuda")
    rs = torch.empty_like(rc)
    ntk = wl.extra.get("ntk_scale")
    if ntk is None:
        B.llama_rope_table(rc, rs, max_pos, s.head_dim, s.rope_theta)
    else:
        B.llama_rope_table_ntk(rc, rs, max_pos, s.head_dim, s.rope_theta, ntk)
    w8 = wbits == 8
    sets, tables = [], []
    for c in range(copies):
        w = {k: dev(v, act) for k, v in stored.items()}
        w["rope_cos"], w["rope_sin"] = rc, rs
        if w8:
            for k in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down"):
                full = w.pop(k)
                q = torch.empty(full.shape, dtype=torch.int8, device="cuda")
                sc = torch.empty(full.shape[0], dtype=torch.float32, device="cuda")
                B.llama_quantize_w8(full, q, sc, act)
                w[k], w["s_" + k[2:]] = q, sc
            torch.cuda.synchronize()
            lw = B.LayerWeightsW8(w)
        elif wbits == 4:
            for k in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down"):
                full = w.pop(k)
                q = torch.empty(full.shape[0], full.shape[1] // 2, dtype=torch.uint8,
                                device="cuda")
                sc = torch.empty(full.shape[0], dtype=torch.float32, device="cuda")
                B.llama_quantize_w4(full, q, sc, act)
                w[k], w["s_" + k[2:]] = q, sc
            torch.cuda.synchronize()
            lw = B.LayerWeightsW4(w)
        else:
            lw = B.LayerWeights(w)
        if wl.extra.get("block_size"):
            kp, vp, table = paged_pools(inp, wl.extra["block_size"], 1000 + c)
            sets.append((lw, dev(kp, kvd), dev(vp, kvd)))
            tables.append(torch.from_numpy(table).cuda())
        else:
            sets.append((lw, dev(inp["k_cache"], kvd), dev(inp["v_cache"], kvd)))
    decode = wl.phase == "decode"
    if decode:
        x = dev(inp["x"], act)
        y = torch.empty_like(x)
        ctx = torch.from_numpy(inp["ctx_len"]).cuda()
        max_ctx = int(inp["ctx_len"].max())
        bsz = wl.extra.get("block_size")
        s_ws = -(-wl.s_max // bsz) * bsz if bsz else wl.s_max  # positions a block table spans
        ws = torch.empty(B.llama_layer_workspace_size(cfg, wl.batch, 1, s_ws), dtype=torch.uint8,
                         device="cuda")

        run = {8: B.llama_layer_decode_w8, 4: B.llama_layer_decode_w4}.get(wbits,
                                                                         B.llama_layer_decode)
        bs = wl.extra.get("block_size")

        def step(i):
            lw, kc, vc = sets[i % copies]
            if bs:
                B.llama_layer_decode_paged(cfg, lw, x, y, kc, vc, bs, tables[i % copies], ctx,
                                           wl.batch, max_ctx, ws)
            else:
                run(cfg, lw, x, y, kc, vc, ctx, wl.batch, max_ctx, wl.s_max, ws)
        # the kernel moving the most bytes: gate/up, or attention at long contexts
        by0 = decode_bytes(s, inp["ctx_len"], act_b, kv_b, wbits)
        dom = "attn_decode" if by0["attn_decode"] > by0["gemv_gate_up"] else "gemv_gate_up"
    else:
        x = dev(inp["x"], act)
        y = torch.empty_like(x)
        ws = torch.empty(B.llama_layer_workspace_size(cfg, wl.batch, wl.tokens, wl.s_max),
                         dtype=torch.uint8, device="cuda")

        def step(i):
            lw, kc, vc = sets[i % copies]
            B.llama_layer_prefill(cfg, lw, x, y, kc, vc, wl.batch, wl.tokens, 0, wl.s_max, ws)
        dom = "gemm_gate_up"

    if args.time_kernel:
        dom = args.time_kernel
    print(f"[bench] {copies} copies, warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    # The timed loop: exactly `steps` calls between synchronisations, nothing
    # else on the stream.  Then the same calls again with an event between
    # steps (the median step) and the dominant kernel's launches bracketed by
    # their own events (the roofline); those events cost ~4% of a 7B step.
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(f"[bench] {args.steps} steps again, with events", file=sys.stderr, flush=True)
    kid = B.kernel_id(dom)
    B.llama_layer_timer_start(kid, args.steps)
    ev = StepEvents(args.steps)
    for i in range(args.steps):
        ev.mark()
        step(i)
    ev.mark()
    torch.cuda.synchronize()
    kms, kn = B.llama_layer_timer_stop()
    ms_step = el * 1e3 / args.steps
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms_step, "ms_per_step_median": median(ev.times_ms()),
           "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": act, "data": "synthetic (seeded; see synth.py)"}
    kavg_s = kms / 1e3 / max(kn, 1)
    # HBM bytes per launch of the dominant kernel from the committed counter
    # summary (None when absent or taken on other kernel sources).
    from llama2_decoder_layer_amd.profiling import load_traffic
    tr = load_traffic(dom, wl.name)
    traffic = None if tr is None else tr["bytes"]
    if decode:
        by = decode_bytes(s, inp["ctx_len"], act_b, kv_b, wbits)
        out.update(value=wl.batch / (ms_step / 1e3), unit="tokens/s/layer")
        layer_gbps = by["total"] / (ms_step / 1e3) / 1e9
        out["layer_hbm"] = {"bytes_per_step": by["total"], "GBps": layer_gbps,
                            "frac_of_peak": layer_gbps / HBM_PEAK_GBPS}
        unit_bytes = by.get(dom)
        ach = unit_bytes / kavg_s / 1e9 if unit_bytes else None
        out["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS if ach else None,
                           "traffic": traffic, "algorithmic_bytes_per_launch": unit_bytes,
                           "avg_launch_us": kavg_s * 1e6, "launches_timed": kn}
    else:
        fl = prefill_flops(s, wl.tokens)
        tflops = fl["total"] / (ms_step / 1e3) / 1e12
        out.update(value=tflops, unit="TFLOP/s")
        out["layer_mfma"] = {"flops_per_step": fl["total"], "TFLOPs": tflops,
                             "frac_of_peak": tflops / BF16_PEAK_TFLOPS}
        unit_flops = fl[{"gemm_qkv": "qkv", "gemm_o": "o", "gemm_gate_up": "gate_up",
                         "gemm_down": "down", "attn_prefill": "attention"}[dom]]
        ach = unit_flops / kavg_s / 1e12
        out["roofline"] = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS, "traffic": traffic,
                           "algorithmic_flops_per_launch": unit_flops,
                           "avg_launch_us": kavg_s * 1e6, "launches_timed": kn}
    out["config"] = {"workload": wl.name, "hidden": s.hidden, "n_heads": s.n_heads,
                     "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                     "intermediate": s.intermediate, "batch": wl.batch,
                     "tokens": wl.tokens if not decode else 1,
                     "ctx": (wl.ctx if wl.ctx else list(wl.ctx_range)) if decode else 0,
                     "kv_dtype": kvd, "rotating_copies": copies}
    if decode and wl.ctx_range:
        out["config"]["ctx_len_sum"] = int(np.sum(inp["ctx_len"]))
    if "ntk_scale" in wl.extra:
        out["config"]["rope_ntk_scale"] = wl.extra["ntk_scale"]
    if wl.extra.get("w8"):
        out["config"]["weights"] = "int8 codes, float32 scale per row"
    if wl.extra.get("w4"):
        out["config"]["weights"] = "int4 codes (two per byte), float32 scale per row"
    if wl.extra.get("block_size"):
        out["config"]["kv_cache"] = f"paged, {wl.extra['block_size']}-position blocks, shuffled pool"
    if args.no_cpu_baseline:
        out["cpu_baseline"] = None
    else:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        if decode:
            out["cpu_baseline"] = cpu_baseline_decode(wl, stored, inp, args.cpu_budget)
        else:
            out["cpu_baseline"] = cpu_baseline_prefill(wl, stored, inp, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
