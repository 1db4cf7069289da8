"""Seeded synthetic inputs for the denoise path: weights, token ids, KV caches, hidden states.

This module only draws random numbers. It holds none of the method's arithmetic, so the
independent CPU oracle and the HIP path can both be fed from it without sharing any code.

Two backends with the same shapes and distributions:

* ``numpy`` (CPU, the default): every tensor has its own stream,
  ``SeedSequence([master, layer, tensor_id])``, so any one tensor can be regenerated alone.
  Values are drawn in float32 and rounded once to bfloat16 (round-to-nearest-even); the
  returned arrays are float32 holding bf16-exact values.
* ``torch`` (device RNG): the same recipe drawn with ``torch.Generator`` on a device, for
  model sizes that would take minutes to draw on the host.  The two backends give different
  numbers for the same seed; a run uses one backend for everything it compares.

Distributions (the synthetic stand-in for a trained checkpoint, which is not available):
matrices are N(0, sigma = 1/sqrt(fan_in)); the embedding is N(0, 1); norm gains are 1.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

MASTER_SEED = 20260610

# tensor ids inside a layer's SeedSequence
_T_ATTN_NORM, _T_WQ, _T_WK, _T_WV, _T_WO, _T_FFN_NORM, _T_ROUTER = range(7)
_T_GATE, _T_UP, _T_DOWN, _T_SGATE, _T_SUP, _T_SDOWN = range(7, 13)
# global tensors use layer id = -1 → mapped to a large constant to stay non-negative
_GLOBAL = 1 << 20
_T_EMBED, _T_FINAL_NORM, _T_HEAD = 0, 1, 2
# non-weight inputs
_DATA = 1 << 21


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    d_ff_expert: int
    d_ff_shared: int  # 0 = no shared dense FFN
    vocab: int
    canvas: int = 256
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    expert_fp8: bool = False  # routed experts quantized to OCP E4M3 (per-channel scales)


# The shapes of the workloads this path is measured and checked on.
TINY = ModelShape(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                  n_experts=8, top_k=2, d_ff_expert=512, d_ff_shared=0, vocab=1024)
MID_LAYER = ModelShape(n_layers=1, d_model=2048, n_q_heads=16, n_kv_heads=8, head_dim=128,
                       n_experts=64, top_k=4, d_ff_expert=768, d_ff_shared=0, vocab=65536)
FULL = ModelShape(n_layers=12, d_model=2048, n_q_heads=16, n_kv_heads=8, head_dim=128,
                  n_experts=64, top_k=4, d_ff_expert=768, d_ff_shared=4096, vocab=65536)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32 (new array)."""
    out = np.array(x, dtype=np.float32, copy=True, order="C")
    u = out.view(np.uint32)
    nan = np.isnan(out)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    lsb += np.uint32(0x7FFF)
    u += lsb          # finite values: no uint32 overflow (|x| <= max float)
    u &= np.uint32(0xFFFF0000)
    if nan.any():
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def _normal(shape, sigma: float, *key: int) -> np.ndarray:
    x = _rng(*key).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return bf16_round(x)


def layer_weights(shape: ModelShape, layer: int, seed: int = MASTER_SEED) -> Dict[str, np.ndarray]:
    d, Hq, Hkv, D = shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    E, F, Fs = shape.n_experts, shape.d_ff_expert, shape.d_ff_shared
    s = lambda fan_in: 1.0 / np.sqrt(fan_in)
    w = {
        "attn_norm": np.ones(d, np.float32),
        "wq": _normal((Hq * D, d), s(d), seed, layer, _T_WQ),
        "wk": _normal((Hkv * D, d), s(d), seed, layer, _T_WK),
        "wv": _normal((Hkv * D, d), s(d), seed, layer, _T_WV),
        "wo": _normal((d, Hq * D), s(Hq * D), seed, layer, _T_WO),
        "ffn_norm": np.ones(d, np.float32),
        "w_router": _normal((E, d), s(d), seed, layer, _T_ROUTER),
        "w_gate": _normal((E, F, d), s(d), seed, layer, _T_GATE),
        "w_up": _normal((E, F, d), s(d), seed, layer, _T_UP),
        "w_down": _normal((E, d, F), s(F), seed, layer, _T_DOWN),
    }
    if Fs:
        w["ws_gate"] = _normal((Fs, d), s(d), seed, layer, _T_SGATE)
        w["ws_up"] = _normal((Fs, d), s(d), seed, layer, _T_SUP)
        w["ws_down"] = _normal((d, Fs), s(Fs), seed, layer, _T_SDOWN)
    return w


def global_weights(shape: ModelShape, seed: int = MASTER_SEED) -> Dict[str, np.ndarray]:
    d, V = shape.d_model, shape.vocab
    return {
        "embed": _normal((V, d), 1.0, seed, _GLOBAL, _T_EMBED),
        "final_norm": np.ones(d, np.float32),
        "lm_head": _normal((V, d), 1.0 / np.sqrt(d), seed, _GLOBAL, _T_HEAD),
    }


def model_weights(shape: ModelShape, seed: int = MASTER_SEED) -> Dict[str, object]:
    """All weights as float32 arrays holding bf16 values: {'layers': [...], 'embed', ...}."""
    g = global_weights(shape, seed)
    g["layers"] = [layer_weights(shape, l, seed) for l in range(shape.n_layers)]
    return g


def tokens(n: int, vocab: int, seed: int, tag: int = 0) -> np.ndarray:
    """n uniform token ids in [0, vocab)."""
    return _rng(seed, _DATA, 1, tag).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def hidden(rows: int, d: int, seed: int, tag: int = 0) -> np.ndarray:
    """A residual-stream state N(0, 1), float32 (not rounded)."""
    return _rng(seed, _DATA, 2, tag).standard_normal(size=(rows, d), dtype=np.float32)


def bf16_normal(shape, seed: int, tag: int = 0, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma) rounded to bf16, float32 storage (synthetic K/V, normed hidden states)."""
    return _normal(tuple(shape), sigma, seed, _DATA, 3, tag)


def uniform(shape, lo: float, hi: float, seed: int, tag: int = 0) -> np.ndarray:
    return _rng(seed, _DATA, 4, tag).uniform(lo, hi, size=shape).astype(np.float32)


def ragged_lengths(batch: int, mean: int, spread: float, seed: int, multiple: int = 1) -> List[int]:
    """Per-request prefix lengths round(mean * (1 + U(-spread, spread)))."""
    u = _rng(seed, _DATA, 5).uniform(-spread, spread, size=batch)
    out = [int(round(mean * (1.0 + x))) for x in u]
    if multiple > 1:
        out = [max(multiple, (v // multiple) * multiple) for v in out]
    return out


# ----------------------------------------------------------------------------------------------
# torch device backend (large shapes).  Same recipe, device RNG; returns bf16 tensors.
# ----------------------------------------------------------------------------------------------

def torch_model_weights(shape: ModelShape, device, seed: int = MASTER_SEED):
    import torch

    gen = torch.Generator(device=device)

    def normal(shp, sigma, *key):
        gen.manual_seed(int(np.random.SeedSequence([seed, *key]).generate_state(1, np.uint64)[0] >> 1))
        t = torch.empty(shp, dtype=torch.float32, device=device)
        t.normal_(0.0, float(sigma), generator=gen)
        return t.to(torch.bfloat16)

    d, Hq, Hkv, D = shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    E, F, Fs, V = shape.n_experts, shape.d_ff_expert, shape.d_ff_shared, shape.vocab
    s = lambda fan_in: 1.0 / np.sqrt(fan_in)
    layers = []
    for l in range(shape.n_layers):
        w = {
            "attn_norm": torch.ones(d, dtype=torch.float32, device=device),
            "wq": normal((Hq * D, d), s(d), l, _T_WQ),
            "wk": normal((Hkv * D, d), s(d), l, _T_WK),
            "wv": normal((Hkv * D, d), s(d), l, _T_WV),
            "wo": normal((d, Hq * D), s(Hq * D), l, _T_WO),
            "ffn_norm": torch.ones(d, dtype=torch.float32, device=device),
            "w_router": normal((E, d), s(d), l, _T_ROUTER),
            "w_gate": normal((E, F, d), s(d), l, _T_GATE),
            "w_up": normal((E, F, d), s(d), l, _T_UP),
            "w_down": normal((E, d, F), s(F), l, _T_DOWN),
        }
        if Fs:
            w["ws_gate"] = normal((Fs, d), s(d), l, _T_SGATE)
            w["ws_up"] = normal((Fs, d), s(d), l, _T_SUP)
            w["ws_down"] = normal((d, Fs), s(Fs), l, _T_SDOWN)
        layers.append(w)
    return {
        "embed": normal((V, d), 1.0, _GLOBAL, _T_EMBED),
        "final_norm": torch.ones(d, dtype=torch.float32, device=device),
        "lm_head": normal((V, d), s(d), _GLOBAL, _T_HEAD),
        "layers": layers,
    }


def torch_bf16_normal(shape, device, seed: int, tag: int = 0, sigma: float = 1.0):
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([seed, _DATA, 3, tag]).generate_state(1, np.uint64)[0] >> 1))
    t = torch.empty(tuple(shape), dtype=torch.float32, device=device)
    t.normal_(0.0, float(sigma), generator=gen)
    return t.to(torch.bfloat16)
