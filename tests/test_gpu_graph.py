"""The layer calls under HIP graph capture.

The library allocates nothing, sets no memory and synchronises nothing, and
every launch goes to the stream it is given, so a decode or prefill call can
be recorded into a graph (torch.cuda.graph captures on its own stream, which
the binding passes as the current stream) and replayed.  Each case records
one call, replays it three times with eager work and a synchronisation
between replays, and requires every replay to reproduce the eager call's
output and cache contents bit for bit.  (A replay rewrites the same cache
positions with the same values, so the calls are idempotent.)
"""
import numpy as np
import pytest
import torch

from gpu_util import DeviceLayer, random_layer, to_dev
from llama2_decoder_layer_amd import binding as B
from llama2_decoder_layer_amd import synth as S

pytestmark = pytest.mark.gpu

SHAPE = S.Shape(512, 8, 2, 128, 1376)
S_MAX = 320


def say(msg):
    print(msg, flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def _same(a, b):
    return torch.equal(_bits(a), _bits(b))


def _replay_and_check(label, call, outs, inputs):
    """Eager call, then capture it and replay three times against the eager
    result.  `outs` are the written tensors (output and caches); `inputs` are
    (tensor, initial value) pairs restored before every run (the caches, whose
    other positions are read)."""
    def reset():
        for t, init in inputs:
            t.copy_(init)
        for o in outs:
            if not any(o is t for t, _ in inputs):
                o.fill_(float("nan"))

    reset()
    call()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        reset()
        scratch.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert _same(o, w), f"{label}: replay {rep} differs from the eager call (tensor {i})"
    say(f"[{label}] 3 graph replays == eager call, bit for bit")


@pytest.mark.parametrize("act,kv", [("bf16", "f16"), ("f32", "f32")])
def test_decode_graph(act, kv):
    stored = random_layer(SHAPE, act, 300)
    dl = DeviceLayer(SHAPE, stored, act, kv, max_pos=S_MAX)
    ctx = [5, 190, 77, 311]
    inp = S.draw_decode_inputs(np.random.SeedSequence(301), SHAPE, len(ctx), S_MAX, act, kv, ctx=0)
    x = to_dev(inp["x"], act)
    k0, v0 = to_dev(inp["k_cache"], kv), to_dev(inp["v_cache"], kv)
    dctx = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    ws = dl.workspace(len(ctx), 1, S_MAX)
    for which in ("workspace", "noalloc"):
        kc, vc = k0.clone(), v0.clone()
        y = torch.empty_like(x)

        def call():
            if which == "workspace":
                B.llama_layer_decode(dl.cfg, dl.weights, x, y, kc, vc, dctx, len(ctx), max(ctx),
                                     S_MAX, ws)
            else:
                B.llama_layer_decode_noalloc(dl.cfg, dl.weights, x, y, kc, vc, dctx, len(ctx),
                                             max(ctx), S_MAX)

        _replay_and_check(f"decode-{which}-{act}", call, [y, kc, vc], [(kc, k0), (vc, v0)])


def test_prefill_graph():
    act, kv = "bf16", "bf16"
    stored = random_layer(SHAPE, act, 302)
    dl = DeviceLayer(SHAPE, stored, act, kv, max_pos=S_MAX)
    batch, tokens, start = 2, 200, 40
    inp = S.draw_prefill_inputs(np.random.SeedSequence(303), SHAPE, batch, tokens, S_MAX, act, kv,
                                start_pos=start)
    x = to_dev(inp["x"], act)
    k0, v0 = to_dev(inp["k_cache"], kv), to_dev(inp["v_cache"], kv)
    kc, vc = k0.clone(), v0.clone()
    y = torch.empty_like(x)
    ws = dl.workspace(batch, tokens, S_MAX)

    def call():
        B.llama_layer_prefill(dl.cfg, dl.weights, x, y, kc, vc, batch, tokens, start, S_MAX, ws)

    _replay_and_check("prefill-bf16", call, [y, kc, vc], [(kc, k0), (vc, v0)])
