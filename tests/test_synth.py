"""The seeded input generators: storage rounding and reproducibility (CPU)."""
import numpy as np
import torch

from llama2_decoder_layer_amd import synth as S


def test_bf16_rounding_matches_torch():
    r = np.random.Generator(np.random.PCG64(5))
    a = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -1e-40], np.float32)])
    ours = S.f32_to_bf16_bits(a)
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, want)
    back = S.to_f64(ours, "bf16")
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).double().numpy())


def test_f16_rounding_matches_torch():
    a = np.random.Generator(np.random.PCG64(6)).standard_normal(50000).astype(np.float32) * 100
    ours = S.f32_to_f16_bits(a)
    want = torch.from_numpy(a).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, want)
    assert np.array_equal(S.to_f64(ours, "f16"), torch.from_numpy(a).half().double().numpy())


def test_draws_are_seeded():
    a = S.draw_layer(S.weights_seed(7), S.TINY, "bf16")
    b = S.draw_layer(S.weights_seed(7), S.TINY, "bf16")
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["w_q"].shape == (S.TINY.n_heads * S.TINY.head_dim, S.TINY.hidden)
    w = S.to_f64(a["w_q"], "bf16")
    assert abs(w.std() - 0.02) < 1e-3 and abs(w.mean()) < 1e-3


def test_workload_shapes_follow_size_table():
    import oracle_pins as P
    tab = P.load_golden("page_sizes.json")["config_table"]["values"]
    for wl, row in (("decode_7b_b1_ctx4096", "7B"), ("prefill_13b_t4096", "13B"),
                    ("decode_70b_b32_ragged", "70B"), ("stack_70b_80l", "70B")):
        s = S.WORKLOADS[wl].shape
        t = tab[row]
        assert (s.hidden, s.n_heads, s.n_kv_heads, s.intermediate) == \
            (t["hidden"], t["heads"], t["kv_heads"], t["intermediate"])
        assert s.n_heads * s.head_dim == s.hidden


def test_ragged_lengths_in_range():
    w = S.WORKLOADS["decode_70b_b32_ragged"]
    d = S.draw_decode_inputs(S.inputs_seed(w.index), S.Shape(64, 4, 2, 16, 32), w.batch, 8,
                             "bf16", "f16", ctx_range=w.ctx_range)
    assert d["ctx_len"].min() >= 512 and d["ctx_len"].max() <= 4096 and len(set(d["ctx_len"])) > 10


def test_chunked_draw_independent_of_threads(monkeypatch):
    a = S.normal(np.random.SeedSequence(3), (S.CHUNK * 2 + 17,), 0.5, "bf16")
    monkeypatch.setattr(S, "_workers", lambda: 1)
    b = S.normal(np.random.SeedSequence(3), (S.CHUNK * 2 + 17,), 0.5, "bf16")
    assert np.array_equal(a, b)
    assert abs(S.to_f64(a, "bf16").std() - 0.5) < 1e-3
