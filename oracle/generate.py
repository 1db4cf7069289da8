"""Block-autoregressive generation: prefill, then canvases denoised to completion and committed.

[GUIDE] "Arquitetura em Detalhes" (prompt prefilled causally into the KV cache; a 256-token block
is refined bidirectionally, committed to the cache when finished, and the next block starts);
[NEWS] second paragraph (the same, plus the new canvas conditions on the committed history);
[DOCS] feature list (multi-canvas block-autoregressive sampling).

One canvas: x = uniform tokens; for s = 0..: forward → row stats → sample/commit → stop?  When
the loop ends on a step that changed the canvas (only possible at the step cap), the K/V of the
last forward pass belong to an older canvas, so the forward runs once more without the head on
the final tokens before the K/V are appended.

Parity: composed from pinned parts; the composition itself is "parity unpinned" against the
pages (they print no worked example).  tests/test_oracle_generate.py checks its invariants
(determinism, resume equals uninterrupted run, cache growth and contents).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from . import model, sampler


def new_cache(shape, cap: int):
    z = lambda: np.zeros((shape.n_kv_heads, cap, shape.head_dim), np.float64)
    return [z() for _ in range(shape.n_layers)], [z() for _ in range(shape.n_layers)]


def denoise_canvas(weights: Dict, shape, cache_k, cache_v, prefix_len: int,
                   cfg: sampler.SamplerConfig, b: int = 0, tokens: Optional[np.ndarray] = None,
                   committed: Optional[np.ndarray] = None, stable_run: int = 0,
                   start_step: int = 0, max_step: Optional[int] = None):
    """Run the sampling loop on one canvas.  Returns a dict with the final tokens, the per-step
    trace and the canvas K/V matching the final tokens."""
    C = shape.canvas
    positions = prefix_len + np.arange(C)
    x = sampler.canvas_init(cfg.seed, b, positions, shape.vocab) if tokens is None else np.array(tokens, np.int32)
    com = np.zeros(C, bool) if committed is None else np.array(committed, bool)
    trace = []
    last = None
    step = start_step
    end = cfg.max_steps if max_step is None else min(cfg.max_steps, max_step)
    status = None
    while step < end:
        fw = model.denoise_forward(weights, shape, x, cache_k, cache_v, prefix_len)
        T = sampler.temperature(cfg, step)
        st = sampler.row_stats(fw["logits"], x, T, cfg.seed, b, positions, step)
        x, com, stable_run, status = sampler.sample_commit(st, x, com, stable_run, cfg, step, b,
                                                           positions, shape.vocab)
        last = fw
        trace.append({"step": step, "tokens": x.copy(), "committed": com.copy(), **{
            k: v for k, v in status.items() if k != "selected"}})
        step += 1
        if status["stop"]:
            break
    return {"tokens": x, "committed": com, "stable_run": stable_run, "trace": trace,
            "last_forward": last, "steps": len(trace), "next_step": step,
            "stopped": bool(status and status["stop"]),
            "last_changed": bool(status and status["changed"])}


def finish_block(weights: Dict, shape, cache_k, cache_v, prefix_len: int, result: Dict) -> int:
    """Append the canvas K/V of the final tokens to the cache; return the new length."""
    fw = result["last_forward"]
    if fw is None or result["last_changed"]:
        fw = model.denoise_forward(weights, shape, result["tokens"], cache_k, cache_v, prefix_len,
                                   with_head=False)
    return model.commit_block(cache_k, cache_v, fw["canvas_k"], fw["canvas_v"], prefix_len)


def generate(weights: Dict, shape, prefix_tokens: Sequence[int], n_blocks: int,
             cfg: sampler.SamplerConfig, b: int = 0):
    """Prefill `prefix_tokens`, then denoise and commit `n_blocks` canvases."""
    L = len(prefix_tokens)
    cap = L + n_blocks * shape.canvas
    ck, cv = new_cache(shape, cap)
    model.prefill(weights, shape, prefix_tokens, ck, cv, 0)
    blocks = []
    for _ in range(n_blocks):
        res = denoise_canvas(weights, shape, ck, cv, L, cfg, b)
        L = finish_block(weights, shape, ck, cv, L, res)
        blocks.append(res)
    return {"blocks": blocks, "cache_k": ck, "cache_v": cv, "length": L}
