"""The greedy pick of llama_head_argmax on its own ("Llama2架构与推理全解析"
§2.5: the highest logit, ties to the lowest index).

The logits the call returns are the argmax kernel's input, so the ids must be
exactly numpy's argmax of those logits (the first occurrence of the maximum).
Exact ties are made by identical W_lm rows, whose logits are bit-identical;
the rows sit in different 8192-entry windows of the kernel's scan and at the
ends of the vocabulary.
"""
import numpy as np
import pytest
import torch

from llama2_decoder_layer_amd import binding as B

pytestmark = pytest.mark.gpu

HIDDEN = 256


def run(vocab, tie_rows, seed, n=3):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((vocab, HIDDEN)) * 0.02).astype(np.float32)
    if tie_rows:
        top = np.abs(w).max() * 50.0  # a row whose logit dominates every random one
        for r in tie_rows:
            w[r] = top
    h = rng.standard_normal((n, HIDDEN)).astype(np.float32) + 1.0  # positive mean: top row wins
    wd = torch.from_numpy(w).to(torch.bfloat16).cuda()
    hd = torch.from_numpy(h).to(torch.bfloat16).cuda()
    gain = torch.ones(HIDDEN, dtype=torch.bfloat16, device="cuda")
    ids = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    logits = torch.empty(n, vocab, dtype=torch.float32, device="cuda")
    B.llama_head_argmax(gain, wd, hd, ids, logits, n, HIDDEN, vocab, 1e-5, "bf16")
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    got = ids.cpu().numpy()
    want = np.argmax(lg, axis=1)
    assert np.array_equal(got, want), (vocab, tie_rows, got, want)
    if tie_rows:
        assert np.all(got == min(tie_rows)), (got, tie_rows)
    print(f"[argmax] vocab {vocab} ties {tie_rows}: ids {got.tolist()}", flush=True)


@pytest.mark.parametrize("vocab", [1, 5, 1023, 1024, 8192, 8193, 32000])
def test_argmax_random(vocab):
    run(vocab, [], 400 + vocab)


@pytest.mark.parametrize("vocab,ties", [
    (32000, [31999]),                 # the last entry
    (32000, [0, 1, 31999]),           # ties at both ends
    (32000, [8191, 8192, 20000]),     # across a window boundary
    (8193, [8192, 5]),                # the higher index in the second window
    (5, [4, 2]),
])
def test_argmax_ties_lowest_index(vocab, ties):
    run(vocab, ties, 500 + vocab + len(ties))
