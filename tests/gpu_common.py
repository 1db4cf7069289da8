"""Shared helpers for the GPU parity tests (imported only by tests marked `gpu`)."""
import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import synth

# Parity bar for continuous outputs (attention, FFN, logits) against the float64 oracle with
# bf16 weights: max-abs 2e-2 and relative L2 1e-2.
MAX_ABS = 2e-2
REL_L2 = 1e-2
# Token decisions are compared bit-exactly except where the oracle's own top-2 margin is
# below this (the two sides' logits differ by accumulation order, ~1e-5).
MARGIN = 1e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_discrete_diffusion_amd import dg  # noqa: F401  (raises if libdg.so is missing)
    return dg


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def np_bf16_dev(x) -> torch.Tensor:
    from block_discrete_diffusion_amd import dg
    return dg.to_device_bf16(x, "cuda")


def close(got, want, max_abs=MAX_ABS, rel_l2=REL_L2, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    rl = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    assert mx <= max_abs and rl <= rel_l2, f"{what}: max-abs {mx:.3g} rel-L2 {rl:.3g}"
    return mx, rl


def topk_margin(logits: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest router logit per row (inf when k == E)."""
    s = np.sort(logits, axis=1)[:, ::-1]
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


# Router inputs on the two sides differ by the attention block's bf16-level error (within the
# parity bar), so experts whose logits lie within that bar of the k-th may legitimately swap.
ROUTER_BOUND = 2e-2


def check_topk(gpu_idx: np.ndarray, oracle_logits: np.ndarray, k: int, bound: float = ROUTER_BOUND):
    """Expert choices: identical where the oracle's k-th/(k+1)-th logit gap is >= bound; elsewhere
    every GPU pick must lie within `bound` of the oracle's k-th logit.  Returns the mask of rows
    whose choice is unique (safe to compare downstream values on)."""
    o_idx = np.argsort(-oracle_logits, axis=1, kind="stable")[:, :k]
    margin = topk_margin(oracle_logits, k)
    safe = margin >= bound
    same = np.all(np.sort(gpu_idx, 1) == np.sort(o_idx, 1), axis=1)
    assert same[safe].all(), f"expert choice differs on {int((~same[safe]).sum())} rows with a clear margin"
    kth = np.sort(oracle_logits, axis=1)[:, ::-1][:, k - 1]
    picked = np.take_along_axis(oracle_logits, gpu_idx.astype(np.int64), 1)
    assert np.all(picked[~same] >= kth[~same, None] - bound), "GPU picked an expert far below the k-th"
    # order inside the k picks follows the logits (desc); only near-equal picks may swap
    return safe & same


def oracle_cfg(cfg):
    """Oracle sampler config from the exact float32 values the library receives."""
    from oracle import sampler
    return sampler.SamplerConfig(max_steps=cfg.max_steps, temp_start=float(np.float32(cfg.temp_start)),
                                 temp_end=float(np.float32(cfg.temp_end)), commit_per_step=cfg.commit_per_step,
                                 renoise_conf=float(np.float32(cfg.renoise_conf)), stable_steps=cfg.stable_steps,
                                 entropy_stop=float(np.float32(cfg.entropy_stop)),
                                 renoise_committed=bool(cfg.renoise_committed), seed=cfg.seed)


def random_cache(shape, L: int, cap: int, seed: int, batch: int = 1):
    """Synthetic bf16 prefix K/V (N(0,1)) for every layer: numpy [n_layers, batch, Hkv, cap, D]."""
    k = np.zeros((shape.n_layers, batch, shape.n_kv_heads, cap, shape.head_dim), np.float32)
    v = np.zeros_like(k)
    k[:, :, :, :L] = synth.bf16_normal((shape.n_layers, batch, shape.n_kv_heads, L, shape.head_dim), seed, 1)
    v[:, :, :, :L] = synth.bf16_normal((shape.n_layers, batch, shape.n_kv_heads, L, shape.head_dim), seed, 2)
    return k, v


def load_cache(kv, k: np.ndarray, v: np.ndarray, lens):
    kv.k.copy_(np_bf16_dev(k))
    kv.v.copy_(np_bf16_dev(v))
    kv.set_lengths(lens)
