"""Helpers for the GPU parity tests: move seeded workloads to the device, run
the C ABI through the binding, and evaluate the fp64 oracle on the same values.

Error measure: for a tensor, max|got - want| / max|want| (an element-wise
relative error blows up near zero).  It is applied to the layer output, to
the branch delta out - x (a residual can hide an error in the branches), and to
the K/V entries the call appended.  The branch delta gets an allowance for the
rounding of the stored output (see delta_error).
"""
from __future__ import annotations

import numpy as np
import torch

from llama2_decoder_layer_amd import binding as B
from llama2_decoder_layer_amd import synth as S
from oracle import llama_ref as R

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if dtype == "f32":
        return torch.from_numpy(a).cuda()
    return torch.from_numpy(a.view(np.int16)).cuda().view(TORCH[dtype])


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def rel_err(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))


def oracle_cfg(shape: S.Shape, ntk_scale=None) -> R.LayerConfig:
    theta = shape.rope_theta
    if ntk_scale is not None:
        theta = R.ntk_rope_base(theta, ntk_scale, shape.head_dim)
    return R.LayerConfig(shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                         shape.intermediate, shape.eps, theta)


def oracle_weights(stored: dict, dtype: str) -> R.LayerWeights:
    return R.LayerWeights(**{k: S.to_f64(v, dtype) for k, v in stored.items()})


class DeviceLayer:
    """One layer on the device: config, weights and RoPE tables."""

    def __init__(self, shape: S.Shape, stored: dict, act: str, kv: str, max_pos: int,
                 ntk_scale=None):
        self.shape, self.act, self.kv, self.max_pos = shape, act, kv, max_pos
        dev = {k: to_dev(v, act) for k, v in stored.items()}
        half = shape.head_dim // 2
        dev["rope_cos"] = torch.empty(max_pos, half, dtype=torch.float32, device="cuda")
        dev["rope_sin"] = torch.empty(max_pos, half, dtype=torch.float32, device="cuda")
        if ntk_scale is None:
            B.llama_rope_table(dev["rope_cos"], dev["rope_sin"], max_pos, shape.head_dim,
                               shape.rope_theta)
        else:
            B.llama_rope_table_ntk(dev["rope_cos"], dev["rope_sin"], max_pos, shape.head_dim,
                                   shape.rope_theta, ntk_scale)
        self.cfg = B.make_config(shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                                 shape.intermediate, shape.eps, shape.rope_theta, act, kv, max_pos)
        self.weights = B.LayerWeights(dev)

    def workspace(self, batch, tokens, s_max, poison=True):
        n = B.llama_layer_workspace_size(self.cfg, batch, tokens, s_max)
        assert n > 0
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        if poison:
            ws.fill_(0xFF)  # NaN in every float format
        return ws

    def prefill(self, x, kc, vc, batch, tokens, start_pos, s_max):
        y = torch.full_like(x, float("nan"))
        ws = self.workspace(batch, tokens, s_max)
        B.llama_layer_prefill(self.cfg, self.weights, x, y, kc, vc, batch, tokens, start_pos,
                              s_max, ws)
        return y

    def decode(self, x, kc, vc, ctx_len, batch, max_ctx, s_max):
        y = torch.full_like(x, float("nan"))
        ws = self.workspace(batch, 1, s_max)
        B.llama_layer_decode(self.cfg, self.weights, x, y, kc, vc, ctx_len, batch, max_ctx,
                             s_max, ws)
        return y


def random_layer(shape: S.Shape, act: str, seed: int, learned_gains: bool = True) -> dict:
    """A parity case's layer: N(0, 0.02) weights and learned RMSNorm gains
    (1 + 0.3 N(0, 1), a different draw for attn_norm and ffn_norm), so that a
    kernel that ignored a gain or swapped the two would fail."""
    return S.draw_layer(np.random.SeedSequence(seed), shape, act, learned_gains=learned_gains)


def scale_stored(a, dtype, factor):
    """Multiply stored values by a power of two (exact in every format)."""
    return S.to_storage((S.to_f64(a, dtype) * factor).astype(np.float32), dtype)


# Half an ulp, relative to the value, of the format the layer stores out and
# h1 in (8, 11 and 24 significant bits): each stored tensor carries up to that
# much rounding whatever the kernels compute.
STORE_ULP = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def delta_error(got, want, x, act: str):
    """(error, allowance) of the branch delta out - x.  out and h1 are stored
    in `act`, so each carries up to half an ulp of |out| of rounding that is no
    branch error; the allowance adds those two half-ulps (STORE_ULP is one
    half-ulp relative to the value), relative to the branch scale."""
    dg = np.asarray(got) - x
    dw = np.asarray(want) - x
    scale = max(np.max(np.abs(dw)), 1e-30)
    err = rel_err(dg, dw)
    return err, 2.0 * STORE_ULP[act] * np.max(np.abs(want)) / scale


def check_errors(label: str, errs: dict, tol: float, allow: dict | None = None) -> None:
    """errs: name -> relative error; allow: name -> extra allowance on top of tol."""
    allow = allow or {}
    bad = {k: v for k, v in errs.items() if not v <= tol + allow.get(k, 0.0)}
    print(f"[{label}] " + ", ".join(
        f"{k}={v:.2e}" + (f" (bound {tol + allow[k]:.2e})" if k in allow else "")
        for k, v in errs.items()), flush=True)
    assert not bad, f"{label}: errors above {tol}: {bad}"
