"""GPU parity of the fused sampler (llama_sample) against the oracle.

The kernel takes its decisions (top-k membership, the top-p cut, the draw)
on float32 values and sums and the oracle on float64 ones, so a row whose u,
top-p threshold or k-th/(k+1)-th logit gap sits within a hair of a boundary
can legitimately go either way.  float32 puts z = logit / T within 6e-8 of
its value and a sum of at most 1024 terms of the mass within about 1e-6 of
the total, so rows whose mass margins exceed MASS_EPS and whose k-th gap
exceeds GAP_EPS relative have one correct answer and must match exactly;
the others (a few per cent at most with these inputs) must pick a token
that is valid for a slightly wider k and p.
"""
import numpy as np
import pytest
import torch

from llama2_decoder_layer_amd import binding as B
from oracle import llama_ref as R

pytestmark = pytest.mark.gpu

MASS_EPS = 2e-6
GAP_EPS = 1e-6


def say(msg):
    print(msg, flush=True)


def penalised(logits, hist, T, pen):
    z = np.array(logits, np.float64)
    for t in np.unique([h for h in hist if 0 <= h < len(z)]):
        z[t] = z[t] / pen if z[t] > 0 else z[t] * pen
    return z / (T if T > 0 else 1.0)


def row_is_unique(logits, hist, u, T, k, p, pen):
    V = len(logits)
    z = penalised(logits, hist, T, pen)
    zs = np.sort(z)[::-1]
    kk = 1 if T == 0 else min(k, V)
    # an exact tie is ordered by index on both sides; a near tie is not
    if kk < V and 0 < zs[kk - 1] - zs[kk] < GAP_EPS * max(1.0, abs(zs[kk - 1])):
        return False
    if T == 0:
        return True
    ids, q = R.sampling_distribution(logits, hist, T, kk, 1.0, pen)
    before = np.concatenate(([0.0], np.cumsum(q)[:-1]))
    if p < 1.0 and np.min(np.abs(before - p)) < MASS_EPS:
        return False
    ids, q = R.sampling_distribution(logits, hist, T, kk, p, pen)
    return np.min(np.abs(np.cumsum(q) - u)) > MASS_EPS


def run_case(label, n, V, T, k, p, pen, seed, kind="normal", n_hist=64, u=None, given=None):
    r = np.random.default_rng(seed)
    if given is not None:
        logits, hist, u = given["logits"], given["history"], given["u"]
        n_hist = hist.shape[1]
    elif kind == "normal":
        logits = (r.standard_normal((n, V)) * 3.0).astype(np.float32)
    elif kind == "rounded":  # many exact ties
        logits = np.round(r.standard_normal((n, V)) * 2.0).astype(np.float32)
    else:  # all equal
        logits = np.zeros((n, V), np.float32)
    if given is None:
        hist = r.integers(-1, V, (n, n_hist)).astype(np.int32) if n_hist else None
    if u is None:
        u = r.random(n).astype(np.float32)
    u = np.asarray(u, np.float32)
    say(f"[{label}] n={n} V={V} T={T} k={k} p={p} pen={pen} {kind} hist={n_hist}")
    d_log = torch.from_numpy(logits).cuda()
    d_hist = torch.from_numpy(hist).cuda() if n_hist else None
    d_u = torch.from_numpy(u).cuda()
    ids = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    B.llama_sample(d_log, d_hist, d_u, ids, T, k, p, pen)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    h = hist if n_hist else np.zeros((n, 0), np.int32)
    # the kernel sees u as float32; the oracle gets the same value widened
    want = R.sample(logits.astype(np.float64), h, u.astype(np.float64), T, min(k, V), p, pen)
    amb = 0
    for i in range(n):
        if row_is_unique(logits[i].astype(np.float64), h[i], float(u[i]), T, k, p, pen):
            assert got[i] == want[i], (label, i, got[i], want[i])
        else:
            amb += 1
            kk = min((1 if T == 0 else k) + 1, V)
            ok, _ = R.sampling_distribution(logits[i], h[i], T if T else 1.0, kk,
                                            min(1.0, p + 1e-3), pen)
            assert got[i] in set(ok.tolist()), (label, i, got[i], ok[:8])
    say(f"[{label}] {n - amb} rows exact, {amb} near a boundary")
    assert amb <= max(2, n // 20)
    return got


def test_sample_pages_settings():
    # temperature 0.7, top-p 0.9, top-k 50, penalty 1.1 on a 32000-token vocabulary
    run_case("pages", 256, 32000, 0.7, 50, 0.9, 1.1, 1)


def test_sample_bench_workload():
    """The benchmark's inputs and settings (32 rows, 32000 tokens)."""
    from llama2_decoder_layer_amd import synth as S
    wl = S.WORKLOADS["sample_b32_v32000"]
    e = wl.extra
    run_case(wl.name, wl.batch, wl.vocab, e["temperature"], e["top_k"], e["top_p"], e["penalty"],
             0, given=S.draw_sample_inputs(wl.name))


def test_sample_wide_top_k_and_tight_top_p():
    run_case("k1024", 128, 32000, 1.0, 1024, 0.95, 1.0, 2)
    run_case("p0.3", 128, 32000, 1.3, 1024, 0.3, 1.05, 3)


def test_sample_max_vocab_and_small_vocabs():
    run_case("v32768", 64, 32768, 0.3, 8, 1.0, 1.3, 4)
    run_case("v1", 8, 1, 0.7, 50, 0.9, 1.1, 5, n_hist=3)
    run_case("v5", 64, 5, 0.9, 1024, 1.0, 1.2, 6, n_hist=2)
    run_case("v1000-k>V", 64, 1000, 1.1, 1024, 0.8, 1.0, 7, n_hist=0)
    run_case("v1500", 64, 1500, 0.8, 1000, 1.0, 1.1, 8)


def test_sample_greedy_limits():
    # temperature 0 and top-k 1 both return the highest penalised logit
    a = run_case("T0", 128, 32000, 0.0, 50, 0.9, 1.1, 9)
    b = run_case("k1", 128, 32000, 1.0, 1, 0.9, 1.1, 9)
    assert np.array_equal(a, b)


def test_sample_ties_by_lowest_index():
    # all logits equal: top-k keeps ids 0..99, each drawn with mass 1/100 in
    # index order, so u = (j + 0.5) / 100 draws id j
    u = (np.arange(100) + 0.5) / 100.0
    got = run_case("ties", 100, 3000, 1.0, 100, 1.0, 1.0, 10, kind="equal", n_hist=0, u=u)
    assert np.array_equal(got, np.arange(100))
    run_case("rounded", 128, 32000, 0.9, 200, 0.9, 1.1, 11, kind="rounded")


def test_sample_empirical_distribution():
    """One row drawn at 4096 evenly spaced u: each kept token comes up 4096 p
    times to within one (plus the rows near a step), no other token at all."""
    r = np.random.default_rng(12)
    V, N = 32000, 4096
    row = (r.standard_normal(V) * 3.0).astype(np.float32)
    hist = r.integers(0, V, 64).astype(np.int32)
    logits = torch.from_numpy(np.repeat(row[None], N, 0)).cuda()
    h = torch.from_numpy(np.repeat(hist[None], N, 0)).cuda()
    u = torch.from_numpy(((np.arange(N) + 0.5) / N).astype(np.float32)).cuda()
    ids = torch.empty(N, dtype=torch.int32, device="cuda")
    B.llama_sample(logits, h, u, ids, 0.7, 50, 0.9, 1.1)
    torch.cuda.synchronize()
    counts = np.bincount(ids.cpu().numpy(), minlength=V)
    keep, q = R.sampling_distribution(row.astype(np.float64), hist, 0.7, 50, 0.9, 1.1)
    say(f"[empirical] {len(keep)} kept tokens, max |count - N p| "
        f"{np.max(np.abs(counts[keep] - N * q)):.2f}")
    assert counts[keep].sum() == N
    assert np.all(np.abs(counts[keep] - N * q) <= 2.0)


def test_sample_empty_batch():
    # n = 0 launches nothing and leaves every buffer as it was
    ids = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    assert B.lib().llama_sample(B._ptr(ids), None, 0, B._ptr(ids), B._ptr(ids), 0, 100, 0.7, 50,
                                0.9, 1.1, None) == 0
    torch.cuda.synchronize()
    assert torch.all(ids == -7)
