"""Checks that pin the fp64 oracle to facts fixed outside it.

Each ``check_*`` raises AssertionError when the oracle disagrees with a closed
form, an invariant, a brute-force evaluation on a tiny input, a library routine
(torch, transformers) or a value printed on the pages.  test_oracle_pins.py runs
them all; test_oracle_mutations.py plants plausible mistakes in the oracle and
asserts that some check fails for each.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import llama_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rand_cfg(H=64, nh=4, nkv=2, hd=16, I=96, eps=1e-5, theta=10000.0):
    return R.LayerConfig(H, nh, nkv, hd, I, eps, theta)


def rand_weights(cfg, seed=0, std=0.1, gamma_random=True):
    r = _rng(seed)
    H, nh, nkv, hd, I = cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate
    g = (lambda: 1.0 + 0.3 * r.standard_normal(H)) if gamma_random else (lambda: np.ones(H))
    return R.LayerWeights(
        attn_norm=g(),
        w_q=std * r.standard_normal((nh * hd, H)),
        w_k=std * r.standard_normal((nkv * hd, H)),
        w_v=std * r.standard_normal((nkv * hd, H)),
        w_o=std * r.standard_normal((H, nh * hd)),
        ffn_norm=g(),
        w_gate=std * r.standard_normal((I, H)),
        w_up=std * r.standard_normal((I, H)),
        w_down=std * r.standard_normal((H, I)),
    )


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------

def check_rmsnorm_closed_form():
    """gamma = 1: rms(u) = sqrt(ms / (ms + eps)) exactly, for any row."""
    r = _rng(1)
    for eps in (1e-5, 0.05, 0.5):
        x = r.standard_normal((7, 33)) * np.array([[1e-3], [1e-2], [0.1], [1], [3], [10], [0.3]])
        u = R.rmsnorm(x, np.ones(33), eps)
        ms = np.mean(x * x, axis=1)
        got = np.sqrt(np.mean(u * u, axis=1))
        want = np.sqrt(ms / (ms + eps))
        assert np.max(np.abs(got - want)) < 1e-13, (eps, got, want)


def check_rmsnorm_scale_invariance_and_rows():
    """eps -> 0: rmsnorm(c x) = rmsnorm(x); rows are normalised independently."""
    r = _rng(2)
    x = r.standard_normal((5, 40))
    gamma = r.standard_normal(40)
    a = R.rmsnorm(x, gamma, 1e-30)
    b = R.rmsnorm(37.5 * x, gamma, 1e-30)
    assert rel_err(a, b) < 1e-13
    x2 = x.copy()
    x2[3] *= 1000.0
    x2[1] = r.standard_normal(40)
    c = R.rmsnorm(x2, gamma, 1e-30)
    for i in (0, 2, 4):
        assert np.array_equal(c[i], a[i])


def check_rmsnorm_torch():
    r = _rng(3)
    x = r.standard_normal((6, 48))
    gamma = r.standard_normal(48)
    for eps in (1e-5, 1e-6, 0.1):
        want = F.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(gamma), eps).numpy()
        assert rel_err(R.rmsnorm(x, gamma, eps), want) < 1e-13


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def check_rope_complex_hd2():
    """head_dim = 2: the pair (a, b) is the complex number a + ib multiplied
    by e^{i m theta_0} with theta_0 = 1 for any base."""
    r = _rng(4)
    z = r.standard_normal((9, 3, 2))
    pos = np.array([0, 1, 2, 5, 17, 100, 1000, 4095, 16383])
    got = R.rope(z, pos, 10000.0)
    c = (z[..., 0] + 1j * z[..., 1]) * np.exp(1j * pos)[:, None]
    assert np.max(np.abs(got[..., 0] - c.real)) < 1e-9
    assert np.max(np.abs(got[..., 1] - c.imag)) < 1e-9


def check_rope_norm_identity_relative():
    r = _rng(5)
    hd = 32
    z = r.standard_normal((6, 2, hd))
    pos = np.array([0, 3, 11, 250, 4000, 4096])
    out = R.rope(z, pos, 10000.0)
    # norm of every pair is preserved
    pa = z[..., 0::2] ** 2 + z[..., 1::2] ** 2
    pb = out[..., 0::2] ** 2 + out[..., 1::2] ** 2
    assert np.max(np.abs(pa - pb)) < 1e-12
    # identity at m = 0
    assert np.array_equal(R.rope(z[:1], np.array([0]), 10000.0), z[:1])
    # <R_m q, R_n k> depends only on m - n
    q = r.standard_normal((1, 1, hd))
    k = r.standard_normal((1, 1, hd))
    for m, n in ((5, 2), (40, 1), (700, 699), (3, 3)):
        base = np.sum(R.rope(q, np.array([m]), 1e4) * R.rope(k, np.array([n]), 1e4))
        for s in (1, 17, 1000, 3000):
            sh = np.sum(R.rope(q, np.array([m + s]), 1e4) * R.rope(k, np.array([n + s]), 1e4))
            assert abs(sh - base) < 1e-9 * max(1.0, abs(base)), (m, n, s, sh, base)


def adjacent_to_half_perm(hd):
    """Row order taking the adjacent-pair layout (2i, 2i+1) to the half-split
    layout (i, i + hd/2) used by transformers' rotate_half."""
    return np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])


def check_rope_transformers():
    """transformers' apply_rotary_pos_emb with its own inverse frequencies,
    after mapping adjacent pairs to its half-split layout."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    r = _rng(6)
    hd, T, nh = 64, 40, 3
    cfg = LlamaConfig(hidden_size=nh * hd, num_attention_heads=nh, num_key_value_heads=nh,
                      head_dim=hd, rope_theta=10000.0, max_position_embeddings=4096)
    rot = LlamaRotaryEmbedding(cfg)
    pos = np.sort(r.choice(4096, T, replace=False))
    q = r.standard_normal((T, nh, hd))
    perm = adjacent_to_half_perm(hd)
    qt = torch.from_numpy(q[..., perm]).permute(1, 0, 2)[None]  # [1, nh, T, hd]
    cos, sin = rot(qt.float(), torch.from_numpy(pos)[None])
    got_hf, _ = apply_rotary_pos_emb(qt, qt, cos.double(), sin.double())
    got_hf = got_hf[0].permute(1, 0, 2).numpy()
    ours = R.rope(q, pos, 10000.0)[..., perm]
    # transformers forms its angles in float32, hence the looser bound
    assert np.max(np.abs(ours - got_hf)) < 2e-3 * np.max(np.abs(q)), np.max(np.abs(ours - got_hf))
    # low positions, where float32 angles are accurate to ~1e-6
    sel = pos < 64
    if sel.any():
        assert np.max(np.abs(ours[sel] - got_hf[sel])) < 1e-5


def check_rope_ntk_scaling():
    """NTK-aware base scaling: scale 1 is plain RoPE; the fastest pair keeps
    its frequency and the slowest turns exactly `scale` times slower, so with
    the pages' example (scale 8, a 4K context stretched to 32K) the slowest
    pair's angle at position 8m equals the unscaled angle at m; every pair
    lies between no scaling and full position interpolation."""
    for hd in (64, 128):
        plain = R.rope_inv_freq(hd, 10000.0)
        assert R.ntk_rope_base(10000.0, 1.0, hd) == 10000.0
        for scale in (2.0, 8.0, 16.0):
            f = R.rope_inv_freq(hd, R.ntk_rope_base(10000.0, scale, hd))
            assert f[0] == plain[0] == 1.0
            assert abs(f[-1] * scale / plain[-1] - 1.0) < 1e-13, (hd, scale)
            assert np.all(f <= plain * (1 + 1e-15)) and np.all(f >= plain / scale * (1 - 1e-13))
            assert np.all(np.diff(f / plain) < 0)
    hd, m = 128, np.array([1, 7, 512, 4095])
    z = np.zeros((4, 1, hd))
    z[..., -2] = 1.0  # only the slowest pair: angle = atan2 of the rotated pair
    a_ntk = R.rope(z, 8 * m, R.ntk_rope_base(10000.0, 8.0, hd))
    a_plain = R.rope(z, m, 10000.0)
    assert np.max(np.abs(a_ntk - a_plain)) < 1e-12


def check_rope_ntk_transformers():
    """transformers' dynamic-NTK base at a sequence length where its factor
    works out to a fixed scale: factor 2 at 4.5x the trained length gives
    2 * 4.5 - (2 - 1) = 8."""
    from transformers import LlamaConfig
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    hd = 128
    cfg = LlamaConfig(hidden_size=32 * hd, num_attention_heads=32, num_key_value_heads=32,
                      head_dim=hd, rope_theta=10000.0, max_position_embeddings=4096,
                      rope_scaling={"rope_type": "dynamic", "factor": 2.0})
    inv, _ = ROPE_INIT_FUNCTIONS["dynamic"](cfg, "cpu", seq_len=int(4.5 * 4096))
    ours = R.rope_inv_freq(hd, R.ntk_rope_base(10000.0, 8.0, hd))
    assert np.max(np.abs(inv.double().numpy() / ours - 1.0)) < 1e-6


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _brute_attention(q, k, v, q_pos):
    T, nh, hd = q.shape
    S, nkv, _ = k.shape
    o = np.zeros_like(q)
    for t in range(T):
        for h in range(nh):
            j = h // (nh // nkv)
            w = []
            for tau in range(S):
                if tau <= q_pos[t]:
                    w.append(np.exp(sum(q[t, h, d] * k[tau, j, d] for d in range(hd)) / np.sqrt(hd)))
                else:
                    w.append(0.0)
            tot = sum(w)
            for tau in range(S):
                o[t, h] += (w[tau] / tot) * v[tau, j]
    return o


def check_attention_bruteforce():
    r = _rng(7)
    for (T, S, nh, nkv, hd, start) in ((5, 5, 2, 1, 4, 0), (3, 7, 4, 2, 3, 4), (1, 6, 3, 3, 2, 5)):
        q = r.standard_normal((T, nh, hd))
        k = r.standard_normal((S, nkv, hd))
        v = r.standard_normal((S, nkv, hd))
        qp = start + np.arange(T)
        assert rel_err(R.causal_gqa_attention(q, k, v, qp), _brute_attention(q, k, v, qp)) < 1e-12


def check_attention_invariants():
    r = _rng(8)
    T, nh, nkv, hd = 6, 4, 2, 8
    q = r.standard_normal((T, nh, hd)) * 3
    k = r.standard_normal((T, nkv, hd))
    v = r.standard_normal((T, nkv, hd))
    qp = np.arange(T)
    o = R.causal_gqa_attention(q, k, v, qp)
    # position 0 sees one key: output is exactly v_0 of its KV head
    for h in range(nh):
        assert np.allclose(o[0, h], v[0, h // (nh // nkv)], rtol=0, atol=1e-15)
    # perturbing later tokens leaves earlier outputs bit-identical
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[4:] += 5.0
    v2[4:] -= 7.0
    q2[4:] *= -2.0
    o2 = R.causal_gqa_attention(q2, k2, v2, qp)
    assert np.array_equal(o[:4], o2[:4])
    # constant V rows give that constant (weights sum to one)
    ones = np.full_like(v, 2.5)
    assert np.max(np.abs(R.causal_gqa_attention(q, k, ones, qp) - 2.5)) < 1e-13


def check_attention_torch_sdpa():
    r = _rng(9)
    for (T, nh, nkv, hd) in ((9, 4, 2, 16), (7, 8, 1, 8), (5, 3, 3, 4)):
        q = r.standard_normal((T, nh, hd))
        k = r.standard_normal((T, nkv, hd))
        v = r.standard_normal((T, nkv, hd))
        want = F.scaled_dot_product_attention(
            torch.from_numpy(q).transpose(0, 1)[None], torch.from_numpy(k).transpose(0, 1)[None],
            torch.from_numpy(v).transpose(0, 1)[None], is_causal=True, enable_gqa=True)
        want = want[0].transpose(0, 1).numpy()
        assert rel_err(R.causal_gqa_attention(q, k, v, np.arange(T)), want) < 1e-12


def check_gqa_reductions():
    """GQA equals MHA over K/V heads replicated in contiguous groups; with
    n_kv_heads = n_heads it is plain multi-head attention, with one KV head MQA."""
    r = _rng(10)
    T, nh, hd = 6, 8, 4
    q = r.standard_normal((T, nh, hd))
    for nkv in (1, 2, 4, 8):
        k = r.standard_normal((T, nkv, hd))
        v = r.standard_normal((T, nkv, hd))
        g = nh // nkv
        kr = np.repeat(k, g, axis=1)
        vr = np.repeat(v, g, axis=1)
        a = R.causal_gqa_attention(q, k, v, np.arange(T))
        b = R.causal_gqa_attention(q, kr, vr, np.arange(T))
        assert np.max(np.abs(a - b)) < 1e-14
        # per-head single-head attention, written independently as MHA
        for h in range(nh):
            oh = R.causal_gqa_attention(q[:, h:h + 1], kr[:, h:h + 1], vr[:, h:h + 1], np.arange(T))
            assert np.max(np.abs(oh[:, 0] - a[:, h])) < 1e-14


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------

def check_silu_closed_forms():
    assert R.silu(np.array([0.0]))[0] == 0.0
    assert abs(R.silu(np.array([1.0]))[0] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
    assert abs(R.silu(np.array([-1.0]))[0] + 1.0 / (1.0 + np.e)) < 1e-15
    assert abs(R.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(R.silu(np.array([-40.0]))[0]) < 1e-15
    z = np.linspace(-8, 8, 101)
    assert rel_err(R.silu(z), F.silu(torch.from_numpy(z)).numpy()) < 1e-15


def check_swiglu_special_cases():
    cfg = rand_cfg()
    w = rand_weights(cfg, seed=11)
    u = _rng(12).standard_normal((5, cfg.hidden))
    w.w_gate = np.zeros_like(w.w_gate)
    assert np.max(np.abs(R.swiglu_ffn(u, w))) == 0.0
    w = rand_weights(cfg, seed=11)
    w.w_up = np.zeros_like(w.w_up)
    assert np.max(np.abs(R.swiglu_ffn(u, w))) == 0.0


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def transformers_layer(cfg, w):
    """transformers' LlamaDecoderLayer in float64 carrying the same weights
    (W_q / W_k rows permuted from adjacent pairs to the half-split layout)."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaDecoderLayer
    hc = LlamaConfig(hidden_size=cfg.hidden, intermediate_size=cfg.intermediate,
                     num_attention_heads=cfg.n_heads, num_key_value_heads=cfg.n_kv_heads,
                     head_dim=cfg.head_dim, rms_norm_eps=cfg.eps, rope_theta=cfg.rope_theta,
                     max_position_embeddings=8192, attention_bias=False, mlp_bias=False,
                     hidden_act="silu")
    hc._attn_implementation = "eager"
    layer = LlamaDecoderLayer(hc, layer_idx=0).to(torch.float64).eval()
    hd = cfg.head_dim
    perm = adjacent_to_half_perm(hd)
    rows_q = (np.arange(cfg.n_heads)[:, None] * hd + perm[None, :]).ravel()
    rows_k = (np.arange(cfg.n_kv_heads)[:, None] * hd + perm[None, :]).ravel()
    sd = {
        "self_attn.q_proj.weight": w.w_q[rows_q], "self_attn.k_proj.weight": w.w_k[rows_k],
        "self_attn.v_proj.weight": w.w_v, "self_attn.o_proj.weight": w.w_o,
        "mlp.gate_proj.weight": w.w_gate, "mlp.up_proj.weight": w.w_up,
        "mlp.down_proj.weight": w.w_down, "input_layernorm.weight": w.attn_norm,
        "post_attention_layernorm.weight": w.ffn_norm,
    }
    layer.load_state_dict({k: torch.from_numpy(np.ascontiguousarray(v)) for k, v in sd.items()})
    return layer


def run_transformers_layer(layer, cfg, x, pos):
    """x: [T, H] at positions pos; fp64 angles for the half-split layout."""
    T = x.shape[0]
    inv = cfg.rope_theta ** (-2.0 * np.arange(cfg.head_dim // 2) / cfg.head_dim)
    ang = pos[:, None].astype(np.float64) * inv[None]
    emb = np.concatenate([ang, ang], axis=-1)
    cos = torch.from_numpy(np.cos(emb))[None]
    sin = torch.from_numpy(np.sin(emb))[None]
    mask = torch.full((T, T), float("-inf"), dtype=torch.float64).triu(1)[None, None]
    with torch.no_grad():
        y = layer(torch.from_numpy(x)[None], attention_mask=mask,
                  position_ids=torch.from_numpy(pos)[None], position_embeddings=(cos, sin))
    y = y[0] if isinstance(y, tuple) else y
    return y[0].numpy()


def check_layer_transformers():
    """transformers runs its RMSNorm and eager softmax in float32 even for
    float64 inputs, so agreement is bounded near 1e-7 rather than 1e-15."""
    for (H, nh, nkv, hd, I, T, seed, eps) in ((64, 4, 2, 16, 96, 11, 13, 1e-5),
                                              (48, 3, 3, 16, 80, 7, 14, 0.05),
                                              (64, 8, 1, 8, 72, 6, 15, 1e-6)):
        cfg = rand_cfg(H, nh, nkv, hd, I, eps=eps)
        w = rand_weights(cfg, seed=seed)
        x = _rng(seed + 100).standard_normal((1, T, H))
        kc = np.zeros((1, nkv, T, hd))
        vc = np.zeros((1, nkv, T, hd))
        ours = R.layer_prefill(cfg, w, x, kc, vc, 0)[0]
        hf = run_transformers_layer(transformers_layer(cfg, w), cfg, x[0], np.arange(T))
        assert rel_err(ours, hf) < 1e-6, rel_err(ours, hf)
        assert rel_err(ours - x[0], hf - x[0]) < 1e-6


def check_layer_cached_decode_equals_recompute():
    cfg = rand_cfg(64, 4, 2, 16, 96)
    w = rand_weights(cfg, seed=16)
    T, k, B, S = 7, 4, 2, 16
    x = _rng(17).standard_normal((B, T + k, cfg.hidden))
    kc_full = np.zeros((B, cfg.n_kv_heads, S, cfg.head_dim))
    vc_full = np.zeros_like(kc_full)
    full = R.layer_prefill(cfg, w, x, kc_full, vc_full, 0)
    kc = np.zeros_like(kc_full)
    vc = np.zeros_like(kc_full)
    R.layer_prefill(cfg, w, x[:, :T], kc, vc, 0)
    for i in range(k):
        out = R.layer_decode(cfg, w, x[:, T + i], kc, vc, np.full(B, T + i))
        assert rel_err(out, full[:, T + i]) < 1e-12
    assert rel_err(kc[:, :, :T + k], kc_full[:, :, :T + k]) < 1e-13
    assert rel_err(vc[:, :, :T + k], vc_full[:, :, :T + k]) < 1e-13
    # chunked prefill (start_pos > 0) equals one prefill
    kc2 = np.zeros_like(kc_full)
    vc2 = np.zeros_like(kc_full)
    R.layer_prefill(cfg, w, x[:, :5], kc2, vc2, 0)
    part = R.layer_prefill(cfg, w, x[:, 5:], kc2, vc2, 5)
    assert rel_err(part, full[:, 5:]) < 1e-12
    # out_rows restriction returns the same rows
    kc3 = np.zeros_like(kc_full)
    vc3 = np.zeros_like(kc_full)
    rows = np.array([0, 3, T + k - 1])
    sub = R.layer_prefill(cfg, w, x, kc3, vc3, 0, out_rows=rows)
    assert rel_err(sub, full[:, rows]) < 1e-14


def check_layer_ragged_batch():
    """Batched decode with different lengths equals per-sequence decode."""
    cfg = rand_cfg(64, 4, 2, 16, 96)
    w = rand_weights(cfg, seed=18)
    r = _rng(19)
    B, S = 3, 12
    kc = r.standard_normal((B, cfg.n_kv_heads, S, cfg.head_dim))
    vc = r.standard_normal((B, cfg.n_kv_heads, S, cfg.head_dim))
    x = r.standard_normal((B, cfg.hidden))
    ctx = np.array([2, 9, 5])
    kcb, vcb = kc.copy(), vc.copy()
    outb = R.layer_decode(cfg, w, x, kcb, vcb, ctx)
    for b in range(B):
        k1, v1 = kc[b:b + 1].copy(), vc[b:b + 1].copy()
        o1 = R.layer_decode(cfg, w, x[b:b + 1], k1, v1, ctx[b:b + 1])
        assert np.array_equal(o1[0], outb[b])
        assert np.array_equal(k1[0], kcb[b])


# --------------------------------------------------------------------------
# Stack and greedy
# --------------------------------------------------------------------------

def check_greedy_ties():
    assert int(R.greedy(np.array([1.0, 3.0, 3.0, 2.0]))) == 1
    assert int(R.greedy(np.array([-1.0, -1.0]))) == 0
    assert list(R.greedy(np.array([[0.0, 5.0, 5.0], [7.0, 7.0, 1.0]]))) == [1, 0]


def check_embed_one_hot():
    """Embedding lookup is the one-hot row vector of each id times the table."""
    r = _rng(23)
    table = r.standard_normal((11, 6))
    ids = np.array([0, 10, 3, 3, 7])
    onehot = np.zeros((len(ids), 11))
    onehot[np.arange(len(ids)), ids] = 1.0
    assert np.array_equal(R.embed(table, ids), onehot @ table)


def check_lm_head_worked_example():
    """A hand-worked output head ("Llama2架构与推理全解析" §2.3: final RMSNorm,
    then the untied LM head; "Llama2架构全景解析" §2.2 step 2).

    hidden 2, eps 3.5, gain (2, -1).  Row (3, 4): mean square 12.5, so
    sqrt(12.5 + 3.5) = 4 and the normalised row is (0.75, 1) * (2, -1) =
    (1.5, -1).  Row (-3, 4): (-0.75, 1) * (2, -1) = (-1.5, -1).  With W_lm
    rows (1, 0), (0, 1), (1, 1), (-2, 0.5) the logits are (1.5, -1, 0.5, -3.5)
    and (-1.5, -1, -2.5, 2.5): greedy ids 0 and 3.
    """
    h = np.array([[3.0, 4.0], [-3.0, 4.0]])
    gain = np.array([2.0, -1.0])
    w_lm = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-2.0, 0.5]])
    lg = R.lm_head(h, gain, w_lm, 3.5)
    want = np.array([[1.5, -1.0, 0.5, -3.5], [-1.5, -1.0, -2.5, 2.5]])
    assert np.max(np.abs(lg - want)) < 1e-15, lg
    assert list(R.greedy(lg)) == [0, 3]


def check_lm_head_torch():
    """lm_head equals torch's rms_norm followed by a linear layer, in float64,
    with a learned final gain and a large eps (so its place shows)."""
    r = _rng(24)
    H, V = 48, 37
    h = r.standard_normal((5, H)) * np.array([[0.05], [0.3], [1.0], [4.0], [0.01]])
    gain = 1.0 + 0.3 * r.standard_normal(H)
    w_lm = r.standard_normal((V, H))
    for eps in (1e-5, 0.05):
        want = F.linear(F.rms_norm(torch.from_numpy(h), (H,), torch.from_numpy(gain), eps),
                        torch.from_numpy(w_lm)).numpy()
        assert rel_err(R.lm_head(h, gain, w_lm, eps), want) < 1e-13


def check_generate_head_leg():
    """With no layers, greedy generation is the head alone: the first id comes
    from the prompt's last token, each later one from the previous id, through
    the final RMSNorm (learned gain) and W_lm, not the embedding table
    ("Llama2架构与推理全解析" §2.3, §2.5).  Evaluated with torch."""
    r = _rng(25)
    H, V = 16, 29
    emb = r.standard_normal((V, H))
    w_lm = r.standard_normal((V, H))
    gain = 1.0 + 0.3 * r.standard_normal(H)
    eps = 0.05
    cfg = rand_cfg(H, 2, 1, 8, 24, eps=eps)
    prompt = np.array([3, 17, 8, 21])

    def head(i):
        x = torch.from_numpy(emb[i][None])
        return F.linear(F.rms_norm(x, (H,), torch.from_numpy(gain), eps),
                        torch.from_numpy(w_lm)).numpy()[0]

    ids, logits = R.generate_greedy(cfg, [], emb, gain, w_lm, prompt, 5, 16)
    prev = int(prompt[-1])
    for step in range(6):
        want = head(prev)
        assert rel_err(logits[step], want) < 1e-13, step
        assert ids[step] == int(np.argmax(want))
        prev = int(ids[step])


def check_stack_cached_equals_recompute():
    """Greedy generation with the KV cache picks the same ids as running the
    whole sequence again from scratch at every step."""
    cfg = rand_cfg(32, 2, 1, 16, 48)
    layers = [rand_weights(cfg, seed=20 + i, std=0.3) for i in range(2)]
    r = _rng(22)
    V = 50
    emb = r.standard_normal((V, cfg.hidden))
    wlm = r.standard_normal((V, cfg.hidden))
    fn = np.ones(cfg.hidden)
    prompt = r.integers(0, V, 5)
    ids, logits = R.generate_greedy(cfg, layers, emb, fn, wlm, prompt, 4, 16)
    seq = list(prompt)
    for step in range(5):
        h = R.embed(emb, seq)[None]
        for w in layers:
            S = len(seq)
            h = R.layer_prefill(cfg, w, h, np.zeros((1, 1, S, 16)), np.zeros((1, 1, S, 16)), 0)
        lg = R.lm_head(h[0, -1], fn, wlm, cfg.eps)
        assert rel_err(lg, logits[step]) < 1e-12
        assert int(np.argmax(lg)) == ids[step]
        seq.append(ids[step])


# --------------------------------------------------------------------------
# Sizes printed on the pages
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# Weight-only INT8
# --------------------------------------------------------------------------

def check_quantize_w8():
    """Round to nearest per row: every weight within half a step of its code
    times the scale, each row's largest magnitude on +-127, codes of -w are
    minus the codes of w, dequantised rows quantise back to themselves, a
    zero row stays zero, and a hand-worked row."""
    r = _rng(30)
    w = (r.standard_normal((64, 300)) * 0.02).astype(np.float32)
    w[5] = 0.0
    w[7, :] = 0.0
    w[7, 3] = -0.5
    q, sc = R.quantize_w8_rows(w)
    assert q.dtype == np.int8 and sc.dtype == np.float32
    assert np.all(np.abs(q.astype(int)) <= 127)
    err = np.abs(w.astype(np.float64) - R.dequantize_w8(q, sc))
    assert np.all(err <= sc.astype(np.float64)[:, None] * (0.5 + 1e-6))
    nz = sc > 0
    assert np.all(np.max(np.abs(q[nz].astype(int)), axis=1) == 127)
    assert sc[5] == 0 and not np.any(q[5])
    assert q[7, 3] == -127 and np.count_nonzero(q[7]) == 1
    qn, scn = R.quantize_w8_rows(-w)
    assert np.array_equal(qn, -q) and np.array_equal(scn, sc)
    back = R.dequantize_w8(q, sc).astype(np.float32)
    q2, sc2 = R.quantize_w8_rows(back)
    assert np.array_equal(q2, q) and np.allclose(sc2, sc, rtol=1e-6, atol=0)
    # by hand: max 1.27 -> scale 0.01; -0.64 -> -64, 0.015 -> 1.5 (just above
    # in float32) -> 2, 0.0051 -> 0.51 -> 1
    q, sc = R.quantize_w8_rows(np.array([[1.27, -0.64, 0.015, 0.0051, -1.27]], np.float32))
    assert abs(sc[0] - 0.01) < 1e-9 and list(q[0]) == [127, -64, 2, 1, -127]


def check_quantize_w4():
    """The same properties with 4-bit codes: every weight within half a step,
    each row's largest magnitude on +-7, odd symmetry, dequantised rows
    quantise back to themselves, a zero row stays zero, and a hand-worked row."""
    r = _rng(31)
    w = (r.standard_normal((64, 300)) * 0.02).astype(np.float32)
    w[5] = 0.0
    w[7, :] = 0.0
    w[7, 3] = 0.5
    q, sc = R.quantize_w4_rows(w)
    assert q.dtype == np.int8 and sc.dtype == np.float32
    assert np.all(np.abs(q.astype(int)) <= 7)
    err = np.abs(w.astype(np.float64) - R.dequantize_w4(q, sc))
    assert np.all(err <= sc.astype(np.float64)[:, None] * (0.5 + 1e-6))
    nz = sc > 0
    assert np.all(np.max(np.abs(q[nz].astype(int)), axis=1) == 7)
    assert sc[5] == 0 and not np.any(q[5])
    assert q[7, 3] == 7 and np.count_nonzero(q[7]) == 1
    qn, scn = R.quantize_w4_rows(-w)
    assert np.array_equal(qn, -q) and np.array_equal(scn, sc)
    back = R.dequantize_w4(q, sc).astype(np.float32)
    q2, sc2 = R.quantize_w4_rows(back)
    assert np.array_equal(q2, q) and np.allclose(sc2, sc, rtol=1e-6, atol=0)
    # by hand: max 0.7 -> scale 0.1; -0.33 -> -3.3 -> -3, 0.26 -> 2.6 -> 3,
    # 0.04 -> 0.4 -> 0, 0.68 -> 6.8 -> 7
    q, sc = R.quantize_w4_rows(np.array([[0.7, -0.33, 0.26, 0.04, 0.68, -0.7]], np.float32))
    assert abs(sc[0] - 0.1) < 1e-8 and list(q[0]) == [7, -3, 3, 0, 7, -7]


# --------------------------------------------------------------------------
# Sampling
# --------------------------------------------------------------------------

def check_sampling_worked_example():
    """Four tokens with logits log(1..4): probabilities 0.1..0.4 at T = 1,
    worked out by hand from the definitions."""
    l = np.log([1.0, 2.0, 3.0, 4.0])
    ids, p = R.sampling_distribution(l, [], 1.0, 4, 1.0, 1.0)
    assert list(ids) == [3, 2, 1, 0] and np.allclose(p, [0.4, 0.3, 0.2, 0.1], rtol=1e-14)
    # top-k 3 renormalises over the three largest
    ids, p = R.sampling_distribution(l, [], 1.0, 3, 1.0, 1.0)
    assert list(ids) == [3, 2, 1] and np.allclose(p, [4 / 9, 3 / 9, 2 / 9], rtol=1e-14)
    # top-p 0.6: 0.4 < 0.6, 0.4 + 0.3 reaches it -> two tokens, 4/7 and 3/7
    ids, p = R.sampling_distribution(l, [], 1.0, 4, 0.6, 1.0)
    assert list(ids) == [3, 2] and np.allclose(p, [4 / 7, 3 / 7], rtol=1e-14)
    # top-p 0.35: the first token alone already reaches it
    ids, _ = R.sampling_distribution(l, [], 1.0, 4, 0.35, 1.0)
    assert list(ids) == [3]
    # T = 2: probabilities proportional to sqrt(1..4)
    ids, p = R.sampling_distribution(l, [], 2.0, 4, 1.0, 1.0)
    w = np.sqrt([4.0, 3.0, 2.0, 1.0])
    assert list(ids) == [3, 2, 1, 0] and np.allclose(p, w / w.sum(), rtol=1e-14)
    # penalty 2 on token 3 (seen twice, penalised once): log 4 / 2 = log 2, so
    # the weights are 1, 2, 3, 2 and the tie between tokens 1 and 3 goes to 1
    ids, p = R.sampling_distribution(l, [3, 3, -1], 1.0, 4, 1.0, 2.0)
    assert list(ids) == [2, 1, 3, 0] and np.allclose(p, [3 / 8, 2 / 8, 2 / 8, 1 / 8], rtol=1e-14)
    # a negative logit is multiplied: logits (-1, 0) with token 0 penalised by 3
    ids, p = R.sampling_distribution(np.array([-1.0, 0.0]), [0], 1.0, 2, 1.0, 3.0)
    assert list(ids) == [1, 0] and np.isclose(p[1] / p[0], np.exp(-3.0), rtol=1e-14)
    # inverse CDF over (0.4, 0.7, 0.9, 1.0)
    for u, want in ((0.0, 3), (0.39, 3), (0.41, 2), (0.69, 2), (0.71, 1), (0.95, 0), (0.999, 0)):
        assert R.sample(l[None], [[]], [u], 1.0, 4, 1.0, 1.0)[0] == want, u


def check_sampling_inverse_cdf_counts():
    """Over a grid of N evenly spaced u, every kept token is drawn N * p times
    to within one, and no other token is drawn."""
    r = _rng(21)
    V, N = 300, 20000
    logits = r.standard_normal(V) * 2.0
    hist = r.integers(0, V, 40)
    ids, p = R.sampling_distribution(logits, hist, 0.8, 120, 0.85, 1.3)
    u = (np.arange(N) + 0.5) / N
    got = R.sample(np.repeat(logits[None], N, 0), np.repeat(hist[None], N, 0), u, 0.8, 120, 0.85,
                   1.3)
    counts = np.bincount(got, minlength=V)
    assert np.all(np.abs(counts[ids] - N * p) <= 1.0 + 1e-9)
    assert counts.sum() == counts[ids].sum() == N
    assert abs(np.sum(p) - 1.0) < 1e-12 and len(ids) <= 120


def check_sampling_greedy_limits():
    """T = 0, top-k = 1 and a vanishing temperature all pick the highest
    penalised logit; ties go to the lowest index."""
    r = _rng(22)
    for _ in range(20):
        V = int(r.integers(2, 500))
        l = r.standard_normal(V)
        hist = r.integers(0, V, 5)
        pen = np.array(l)
        for t in np.unique(hist):
            pen[t] = pen[t] / 1.2 if pen[t] > 0 else pen[t] * 1.2
        want = int(np.argmax(pen))
        u = [float(r.random())]
        assert R.sample(l[None], [hist], u, 0.0, 50, 0.9, 1.2)[0] == want
        assert R.sample(l[None], [hist], u, 1.0, 1, 0.9, 1.2)[0] == want
        top2 = np.sort(pen)[-2:]
        if top2[1] - top2[0] > 1e-3:
            assert R.sample(l[None], [hist], u, 1e-6, V, 1.0, 1.2)[0] == want
    tie = np.array([0.5, 2.0, 2.0, 1.0])
    assert R.sample(tie[None], [[]], [0.9], 0.0, 4, 1.0, 1.0)[0] == 1
    assert R.sample(tie[None], [[]], [0.9], 1.0, 1, 1.0, 1.0)[0] == 1


def check_sampling_transformers():
    """transformers' repetition-penalty, temperature, top-k and top-p
    processors, applied in the same order, keep the same tokens with the same
    probabilities."""
    from transformers.generation.logits_process import (RepetitionPenaltyLogitsProcessor,
                                                        TemperatureLogitsWarper,
                                                        TopKLogitsWarper, TopPLogitsWarper)
    r = _rng(23)
    for T, k, tp, pen in ((0.7, 50, 0.9, 1.1), (1.0, 300, 0.5, 1.5), (0.3, 8, 1.0, 1.0)):
        V = 1000
        l = r.standard_normal(V) * 3.0
        hist = r.integers(0, V, 64)
        ids, p = R.sampling_distribution(l, hist, T, k, tp, pen)
        x = torch.from_numpy(l)[None]
        h = torch.from_numpy(hist)[None]
        x = RepetitionPenaltyLogitsProcessor(pen)(h, x)
        x = TemperatureLogitsWarper(T)(h, x)
        x = TopKLogitsWarper(k)(h, x)
        if tp < 1.0:
            x = TopPLogitsWarper(tp)(h, x)
        q = torch.softmax(x, -1)[0].numpy()
        kept = np.nonzero(q)[0]
        assert set(kept) == set(ids), (T, k, tp, pen)
        assert np.max(np.abs(q[ids] - p)) < 1e-12


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def check_sizes_golden():
    g = load_golden("page_sizes.json")
    tab = g["config_table"]["values"]
    for name, row in tab.items():
        cfg = R.LayerConfig(row["hidden"], row["heads"], row["kv_heads"],
                            row["hidden"] // row["heads"], row["intermediate"], 1e-5, 1e4)
        # weight memory in fp16 (2 bytes per parameter)
        gb = R.model_param_count(cfg, row["layers"], row["vocab"]) * 2 / 1e9
        want = g["weights_fp16_GB"]["values"][name]
        assert abs(gb - want) / want < 0.05, (name, gb, want)
    # KV cache, 7B at 4096 positions in fp16 ("about 2 GB")
    r7 = tab["7B"]
    kv = R.kv_cache_bytes(r7["layers"], r7["kv_heads"], r7["hidden"] // r7["heads"], 4096, 2)
    assert kv == 2 * 32 * 32 * 128 * 4096 * 2
    assert abs(kv / 1e9 - g["kv_cache_fp16_4096_GB"]["values"]["7B"]) < 0.25
    # GQA saving for 70B (64 query heads, 8 KV heads)
    r70 = tab["70B"]
    gq = g["gqa_70b"]["values"]
    assert r70["heads"] == gq["q_heads"] and r70["kv_heads"] == gq["kv_heads"]
    hd = r70["hidden"] // r70["heads"]
    saving = 1 - R.kv_cache_bytes(80, r70["kv_heads"], hd, 4096, 2) / R.kv_cache_bytes(80, r70["heads"], hd, 4096, 2)
    assert abs(100 * saving - gq["kv_saving_pct"]) < 1e-9
    # int8 7B ~ 7 GB (one byte per parameter)
    c7 = R.LayerConfig(4096, 32, 32, 128, 11008, 1e-5, 1e4)
    assert abs(R.model_param_count(c7, 32, 32000) / 1e9 - g["weights_int8_7B_GB"]["value"]) < 0.5


ALL_CHECKS = [
    check_rmsnorm_closed_form, check_rmsnorm_scale_invariance_and_rows, check_rmsnorm_torch,
    check_rope_complex_hd2, check_rope_norm_identity_relative, check_rope_transformers,
    check_rope_ntk_scaling, check_rope_ntk_transformers,
    check_attention_bruteforce, check_attention_invariants, check_attention_torch_sdpa,
    check_gqa_reductions, check_silu_closed_forms, check_swiglu_special_cases,
    check_layer_transformers, check_layer_cached_decode_equals_recompute,
    check_layer_ragged_batch, check_greedy_ties, check_embed_one_hot, check_lm_head_worked_example,
    check_lm_head_torch, check_generate_head_leg, check_stack_cached_equals_recompute,
    check_sizes_golden, check_quantize_w8, check_quantize_w4, check_sampling_worked_example, check_sampling_inverse_cdf_counts,
    check_sampling_greedy_limits, check_sampling_transformers,
]
