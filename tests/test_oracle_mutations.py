"""Plant plausible mistakes in the oracle and require that a pin catches each.

Every mutant below is a deliberately wrong variant of one oracle function (a
dropped term, a wrong sign or index, a transposed operand, a wrong scale).  It
is patched into ``oracle.llama_ref`` for the duration of one test, and the pins
of oracle_pins.py are run until one fails.  A mutant that passes every pin
would mean the pins cannot tell that mistake from the truth.
"""
import numpy as np
import pytest

import oracle_pins as P
from oracle import llama_ref as R

F64 = np.float64


def _rmsnorm_eps_outside(x, gamma, eps):
    x = np.asarray(x, F64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * gamma


def _rmsnorm_no_gamma(x, gamma, eps):
    x = np.asarray(x, F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _rmsnorm_across_tokens(x, gamma, eps):
    x = np.asarray(x, F64)
    return x / np.sqrt(np.mean(x * x) + eps) * gamma


def _rope_generic(sign=1.0, half=False, freq_div=1.0):
    def rope(z, positions, rope_theta):
        z = np.asarray(z, F64)
        hd = z.shape[-1]
        i = np.arange(hd // 2, dtype=F64)
        inv = np.power(F64(rope_theta), -2.0 * i / hd / freq_div)
        ang = sign * np.asarray(positions, F64)[:, None] * inv[None, :]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        out = np.empty_like(z)
        if half:
            a, b = z[..., :hd // 2], z[..., hd // 2:]
            out[..., :hd // 2] = a * c - b * s
            out[..., hd // 2:] = a * s + b * c
        else:
            a, b = z[..., 0::2], z[..., 1::2]
            out[..., 0::2] = a * c - b * s
            out[..., 1::2] = a * s + b * c
        return out
    return rope


def _attention_generic(scale="sqrt", strict=False, mod_map=False, normalise=True):
    def attn(q, k, v, q_pos):
        q, k, v = (np.asarray(a, F64) for a in (q, k, v))
        T, nh, hd = q.shape
        S, nkv, _ = k.shape
        g = nh // nkv
        kp = np.arange(S)
        vis = (kp[None, :] < np.asarray(q_pos)[:, None]) if strict else (kp[None, :] <= np.asarray(q_pos)[:, None])
        o = np.empty((T, nh, hd))
        for h in range(nh):
            j = (h % nkv) if mod_map else (h // g)
            s = q[:, h, :] @ k[:, j, :].T
            s = s / {"sqrt": np.sqrt(F64(hd)), "none": 1.0, "lin": F64(hd)}[scale]
            s = np.where(vis, s, -np.inf)
            e = np.exp(s - np.max(s, axis=-1, keepdims=True))
            p = e / np.sum(e, axis=-1, keepdims=True) if normalise else e
            o[:, h, :] = p @ v[:, j, :]
        return o
    return attn


def _sigmoid_not_silu(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, F64)))


def _greedy_last_tie(logits):
    a = np.asarray(logits)
    return a.shape[-1] - 1 - np.argmax(a[..., ::-1], axis=-1)


def _layer_generic(drop_attn_residual=False, rotate_v=False, wo_transposed=False,
                   cache_pre_rope=False, swap_gate_up=False, drop_ffn_residual=False):
    def layer(cfg, w, x, k_cache, v_cache, start_pos, out_rows=None):
        x = np.asarray(x, F64)
        T = x.shape[0]
        nh, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
        pos = start_pos + np.arange(T)
        u = R.rmsnorm(x, w.attn_norm, cfg.eps)
        q = (u @ w.w_q.T).reshape(T, nh, hd)
        k = (u @ w.w_k.T).reshape(T, nkv, hd)
        v = (u @ w.w_v.T).reshape(T, nkv, hd)
        q = R.rope(q, pos, cfg.rope_theta)
        kr = R.rope(k, pos, cfg.rope_theta)
        if rotate_v:
            v = R.rope(v, pos, cfg.rope_theta)
        k_cache[:, pos, :] = (k if cache_pre_rope else kr).transpose(1, 0, 2)
        v_cache[:, pos, :] = v.transpose(1, 0, 2)
        rows = np.arange(T) if out_rows is None else np.asarray(out_rows)
        S = start_pos + T
        o = R.causal_gqa_attention(q[rows], k_cache[:, :S].transpose(1, 0, 2),
                                   v_cache[:, :S].transpose(1, 0, 2), pos[rows])
        wo = w.w_o.T if wo_transposed else w.w_o
        attn = o.reshape(len(rows), nh * hd) @ wo.T
        h1 = attn if drop_attn_residual else x[rows] + attn
        u2 = R.rmsnorm(h1, w.ffn_norm, cfg.eps)
        if swap_gate_up:
            f = (R.silu(u2 @ w.w_up.T) * (u2 @ w.w_gate.T)) @ w.w_down.T
        else:
            f = R.swiglu_ffn(u2, w)
        return f if drop_ffn_residual else h1 + f
    return layer


def _ntk_exponent(num_off=0.0, den_off=-2.0):
    def base(rope_theta, ntk_scale, head_dim):
        d = F64(head_dim)
        return F64(rope_theta) * np.power(F64(ntk_scale), (d + num_off) / (d + den_off))
    return base


def _sampling_generic(pen_inverted=False, pen_per_occurrence=False, temp_mul=False,
                      top_p_exclusive=False, top_k_extra=0):
    def dist(logits, history, temperature, top_k, top_p, penalty):
        z = np.array(logits, dtype=F64)
        hist = [int(t) for t in np.asarray(history).ravel() if 0 <= int(t) < z.shape[0]]
        for t in (hist if pen_per_occurrence else np.unique(hist)):
            if pen_inverted:
                z[t] = z[t] * penalty if z[t] > 0 else z[t] / penalty
            else:
                z[t] = z[t] / penalty if z[t] > 0 else z[t] * penalty
        z = z * temperature if temp_mul else z / temperature
        order = np.lexsort((np.arange(z.shape[0]), -z))[:top_k + top_k_extra]
        e = np.exp(z[order] - z[order[0]])
        p = e / np.sum(e)
        if top_p_exclusive:
            keep = np.cumsum(p) < top_p
            keep[0] = True
        else:
            keep = np.concatenate(([0.0], np.cumsum(p)[:-1])) < top_p
        return order[keep], p[keep] / np.sum(p[keep])
    return dist


def _sample_index_order(logits, history, u, temperature, top_k, top_p, penalty):
    logits = np.asarray(logits, dtype=F64)
    out = np.empty(logits.shape[0], dtype=np.int64)
    for r in range(logits.shape[0]):
        ids, p = R.sampling_distribution(logits[r], history[r] if history is not None else [],
                                         temperature if temperature else 1.0,
                                         top_k if temperature else 1, top_p, penalty)
        o = np.argsort(ids)  # walks the kept tokens by index instead of by probability
        i = int(np.searchsorted(np.cumsum(p[o]), float(u[r]), side="right"))
        out[r] = ids[o][min(i, len(ids) - 1)]
    return out


def _w8_generic(levels=127.0, rounding=np.rint, per_column=False, clip=127):
    def quant(w):
        w32 = np.asarray(w, dtype=np.float32)
        amax = np.max(np.abs(w32), axis=0 if per_column else 1)
        scale = (amax / np.float32(levels)).astype(np.float32)
        safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
        q = rounding(w32 / (safe[None, :] if per_column else safe[:, None]))
        q = np.clip(q, -clip, clip)
        return q.astype(np.int8), (scale if not per_column else scale[:w32.shape[0]])
    return quant


def _lm_head_no_final_norm(h, final_norm, w_lm, eps):
    return np.asarray(h, F64) @ np.asarray(w_lm, F64).T


def _lm_head_eps_outside(h, final_norm, w_lm, eps):
    h = np.asarray(h, F64)
    u = h / (np.sqrt(np.mean(h * h, axis=-1, keepdims=True)) + eps) * final_norm
    return u @ np.asarray(w_lm, F64).T


def _lm_head_no_gain(h, final_norm, w_lm, eps):
    h = np.asarray(h, F64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) @ np.asarray(w_lm, F64).T


def _generate_generic(tied=False, first_position=False):
    """generate_greedy with the head tied to the embedding table, or applied to
    the prompt's first position instead of its last."""
    def gen(cfg, layers, embed_table, final_norm, w_lm, prompt_ids, n_new, s_max):
        head_w = embed_table if tied else w_lm
        prompt_ids = np.asarray(prompt_ids, dtype=np.int64)
        T = prompt_ids.shape[0]
        caches = [(np.zeros((1, cfg.n_kv_heads, s_max, cfg.head_dim)),
                   np.zeros((1, cfg.n_kv_heads, s_max, cfg.head_dim))) for _ in layers]
        h = R.embed(embed_table, prompt_ids)[None]
        for w, (kc, vc) in zip(layers, caches):
            h = R.layer_prefill(cfg, w, h, kc, vc, 0)
        logits = [R.lm_head(h[0, 0 if first_position else -1], final_norm, head_w, cfg.eps)]
        ids = [int(R.greedy(logits[-1]))]
        for step in range(n_new):
            h = R.embed(embed_table, [ids[-1]])
            ctx = np.array([T + step])
            for w, (kc, vc) in zip(layers, caches):
                h = R.layer_decode(cfg, w, h, kc, vc, ctx)
            logits.append(R.lm_head(h[0], final_norm, head_w, cfg.eps))
            ids.append(int(R.greedy(logits[-1])))
        return np.array(ids), np.stack(logits)
    return gen


def _embed_off_by_one(table, ids):
    t = np.asarray(table, F64)
    return t[(np.asarray(ids, dtype=np.int64) + 1) % t.shape[0]]


MUTANTS = {
    "lm_head_drops_final_norm": ("lm_head", _lm_head_no_final_norm),
    "lm_head_eps_outside_sqrt": ("lm_head", _lm_head_eps_outside),
    "lm_head_drops_gain": ("lm_head", _lm_head_no_gain),
    "generate_tied_head": ("generate_greedy", _generate_generic(tied=True)),
    "generate_head_on_first_position": ("generate_greedy", _generate_generic(first_position=True)),
    "embed_off_by_one": ("embed", _embed_off_by_one),
    "rmsnorm_eps_outside_sqrt": ("rmsnorm", _rmsnorm_eps_outside),
    "rmsnorm_drops_gamma": ("rmsnorm", _rmsnorm_no_gamma),
    "rmsnorm_across_tokens": ("rmsnorm", _rmsnorm_across_tokens),
    "rope_wrong_sign": ("rope", _rope_generic(sign=-1.0)),
    "rope_half_split_pairs": ("rope", _rope_generic(half=True)),
    "rope_wrong_frequencies": ("rope", _rope_generic(freq_div=2.0)),
    "ntk_base_scaled_linearly": ("ntk_rope_base", _ntk_exponent(den_off=0.0)),
    "ntk_exponent_d_over_d_minus_1": ("ntk_rope_base", _ntk_exponent(den_off=-1.0)),
    "ntk_exponent_d_over_d_plus_2": ("ntk_rope_base", _ntk_exponent(den_off=2.0)),
    "sampling_penalty_inverted": ("sampling_distribution", _sampling_generic(pen_inverted=True)),
    "sampling_penalty_per_occurrence": ("sampling_distribution",
                                        _sampling_generic(pen_per_occurrence=True)),
    "sampling_temperature_multiplies": ("sampling_distribution", _sampling_generic(temp_mul=True)),
    "sampling_top_p_drops_crossing_token": ("sampling_distribution",
                                            _sampling_generic(top_p_exclusive=True)),
    "sampling_top_k_off_by_one": ("sampling_distribution", _sampling_generic(top_k_extra=1)),
    "sampling_walks_index_order": ("sample", _sample_index_order),
    "w8_scale_over_128": ("quantize_w8_rows", _w8_generic(levels=128.0)),
    "w8_truncates": ("quantize_w8_rows", _w8_generic(rounding=np.trunc)),
    "w8_column_scales": ("quantize_w8_rows", _w8_generic(per_column=True)),
    "w4_scale_over_8": ("quantize_w4_rows", _w8_generic(levels=8.0, clip=7)),
    "w4_truncates": ("quantize_w4_rows", _w8_generic(levels=7.0, rounding=np.trunc, clip=7)),
    "w4_codes_to_8": ("quantize_w4_rows", _w8_generic(levels=7.5, clip=8)),
    "attention_no_scale": ("causal_gqa_attention", _attention_generic(scale="none")),
    "attention_scale_1_over_d": ("causal_gqa_attention", _attention_generic(scale="lin")),
    "attention_mask_excludes_self": ("causal_gqa_attention", _attention_generic(strict=True)),
    "gqa_head_modulo_mapping": ("causal_gqa_attention", _attention_generic(mod_map=True)),
    "softmax_unnormalised": ("causal_gqa_attention", _attention_generic(normalise=False)),
    "silu_is_sigmoid": ("silu", _sigmoid_not_silu),
    "greedy_last_index_on_tie": ("greedy", _greedy_last_tie),
    "layer_drops_attention_residual": ("_layer_one_sequence", _layer_generic(drop_attn_residual=True)),
    "layer_drops_ffn_residual": ("_layer_one_sequence", _layer_generic(drop_ffn_residual=True)),
    "layer_rotates_v": ("_layer_one_sequence", _layer_generic(rotate_v=True)),
    "layer_wo_transposed": ("_layer_one_sequence", _layer_generic(wo_transposed=True)),
    "layer_caches_k_before_rope": ("_layer_one_sequence", _layer_generic(cache_pre_rope=True)),
    "layer_swaps_gate_and_up": ("_layer_one_sequence", _layer_generic(swap_gate_up=True)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(R, attr, fn)
    caught = []
    for check in P.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, IndexError) as e:
            caught.append((check.__name__, type(e).__name__))
            break
    assert caught, f"mutant {name} passed every pin"
