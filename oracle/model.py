"""Forward pass of the denoiser, float64, written out as its plain definition.

The backbone is a pre-norm decoder stack whose blocks are attention followed by a top-k routed
mixture-of-experts FFN ([DOCS] feature list: sparse MoE backbone; [NEWS] second paragraph: the
diffusion head sits on the same backbone and reuses its prefill).  Two ways of running it:

* causal prefill ([GUIDE] "Arquitetura em Detalhes", block-autoregressive bullet list; [NEWS]
  second paragraph; [DOCS] feature list, autoregressive encoder): prompt tokens at positions
  0..L-1, each attending to itself and earlier positions; every layer's K (after RoPE) and V
  are written to the KV cache, which stores bfloat16.
* denoise forward ([GUIDE] "Arquitetura em Detalhes", uniform-state diffusion; [GUIDE] Sudoku
  demo, bidirectional context; [NEWS] second paragraph; [RANK] "Pontos-chave"; [DOCS] feature
  list): the 256 canvas tokens at positions L..L+255 attend, with no mask at all, to the cached
  prefix and to every canvas position; the canvas K/V of each layer are returned (kept in
  float64 here) so they can be appended to the cache when the block is finished.

Readings where the pages are silent:
RMSNorm x * rsqrt(mean(x^2) + eps) * gain; RoPE rotate-half with theta 10000 at absolute
positions, K cached after rotation; attention scale 1/sqrt(head_dim), query head h reads KV head
h // (Hq/Hkv); router logits are a plain linear map, top-k by (logit descending, index
ascending), gates = softmax over the k selected logits, no capacity limit; experts and the
optional shared FFN are SwiGLU, silu(x Wg^T) * (x Wu^T) then W_down; the shared FFN sees the
same normed input and is added with weight 1; untied LM head.

Parity: pinned by tests/test_oracle_model.py (brute-force attention loops on tiny shapes,
closed-form special cases, invariants; see that file for the list).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

F64 = np.float64


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), returned as float64.

    Used where the method stores bfloat16: the KV cache."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    keep = ((bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    out = (keep << np.uint64(16)).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)


def rmsnorm(x, gain, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(gain, F64)


def rope(x: np.ndarray, positions: Sequence[int], theta: float) -> np.ndarray:
    """Rotate-half RoPE.  x: [heads, n, D]; positions: n absolute positions."""
    if theta == 0:
        return np.asarray(x, F64)
    x = np.asarray(x, F64)
    D = x.shape[-1]
    half = D // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=F64) / D)
    ang = np.asarray(positions, F64)[:, None] * inv_freq[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    s = np.asarray(s, F64)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              allowed: Optional[np.ndarray] = None) -> np.ndarray:
    """Grouped-query attention.  q [Hq, n, D]; k, v [Hkv, m, D]; allowed: bool [n, m] or None
    (None = every query sees every key, the canvas case).  Returns [Hq, n, D]."""
    Hq, n, D = q.shape
    Hkv = k.shape[0]
    group = Hq // Hkv
    out = np.empty((Hq, n, D), F64)
    for h in range(Hq):
        g = h // group
        s = (np.asarray(q[h], F64) @ np.asarray(k[g], F64).T) / np.sqrt(D)
        if allowed is not None:
            s = np.where(allowed, s, -np.inf)
        out[h] = softmax(s) @ np.asarray(v[g], F64)
    return out


def silu(x):
    return x / (1.0 + np.exp(-x))


def swiglu(x, w_gate, w_up, w_down):
    x = np.asarray(x, F64)
    return (silu(x @ np.asarray(w_gate, F64).T) * (x @ np.asarray(w_up, F64).T)) @ np.asarray(w_down, F64).T


def router_topk(logits: np.ndarray, k: int):
    """Top-k experts per row by (logit desc, index asc) and softmax gates over those k."""
    logits = np.asarray(logits, F64)
    idx = np.argsort(-logits, axis=-1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, idx, axis=-1)
    return idx.astype(np.int64), softmax(sel, axis=-1)


def moe(b: np.ndarray, lw: Dict[str, np.ndarray], top_k: int):
    """Routed experts (+ shared FFN if present) on normed input b [n, d].
    Returns (output [n, d], expert ids [n, k], gates [n, k], router logits [n, E])."""
    b = np.asarray(b, F64)
    logits = b @ np.asarray(lw["w_router"], F64).T
    idx, gates = router_topk(logits, top_k)
    out = np.zeros_like(b)
    n_exp = lw["w_gate"].shape[0]
    for e in range(n_exp):
        rows, slots = np.nonzero(idx == e)
        if rows.size == 0:
            continue
        y = swiglu(b[rows], lw["w_gate"][e], lw["w_up"][e], lw["w_down"][e])
        np.add.at(out, rows, gates[rows, slots][:, None] * y)
    if "ws_gate" in lw:
        out = out + swiglu(b, lw["ws_gate"], lw["ws_up"], lw["ws_down"])
    return out, idx, gates, logits


def layer(h: np.ndarray, lw: Dict[str, np.ndarray], shape, positions: Sequence[int],
          k_prefix: np.ndarray, v_prefix: np.ndarray, allowed: Optional[np.ndarray]):
    """One decoder layer on rows h [n, d] at absolute positions.

    k_prefix, v_prefix: [Hkv, L, D] keys/values already in the cache (post-RoPE).
    allowed: [n, L + n] mask, or None for the unmasked canvas.
    Returns (h_out, k_new [Hkv, n, D], v_new [Hkv, n, D], debug dict)."""
    Hq, Hkv, D = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    h = np.asarray(h, F64)
    n = h.shape[0]
    a = rmsnorm(h, lw["attn_norm"], shape.rms_eps)
    q = (a @ np.asarray(lw["wq"], F64).T).reshape(n, Hq, D).transpose(1, 0, 2)
    k = (a @ np.asarray(lw["wk"], F64).T).reshape(n, Hkv, D).transpose(1, 0, 2)
    v = (a @ np.asarray(lw["wv"], F64).T).reshape(n, Hkv, D).transpose(1, 0, 2)
    q = rope(q, positions, shape.rope_theta)
    k = rope(k, positions, shape.rope_theta)
    K = np.concatenate([np.asarray(k_prefix, F64), k], axis=1)
    V = np.concatenate([np.asarray(v_prefix, F64), v], axis=1)
    o = attention(q, K, V, allowed).transpose(1, 0, 2).reshape(n, Hq * D)
    h_mid = h + o @ np.asarray(lw["wo"], F64).T
    b = rmsnorm(h_mid, lw["ffn_norm"], shape.rms_eps)
    f, idx, gates, logits = moe(b, lw, shape.top_k)
    h_out = h_mid + f
    dbg = {"attn_in": a, "q": q, "attn_out": o, "h_mid": h_mid, "ffn_in": b,
           "router_logits": logits, "expert_idx": idx, "gates": gates, "ffn_out": f}
    return h_out, k, v, dbg


def denoise_forward(weights: Dict, shape, canvas_tokens: Sequence[int],
                    cache_k: List[np.ndarray], cache_v: List[np.ndarray], prefix_len: int,
                    hidden_in: Optional[np.ndarray] = None, with_head: bool = True,
                    keep_debug: bool = False):
    """Denoise forward for one request's canvas.

    cache_k/cache_v: per layer [Hkv, >=prefix_len, D] (bf16 values); only [:prefix_len] is read.
    hidden_in: optional residual-stream input [C, d] that replaces the token embedding.
    Returns dict with 'logits' [C, V] (if with_head), 'hidden' (final residual), 'canvas_k' /
    'canvas_v' (per layer [Hkv, C, D], float64) and, if keep_debug, per-layer debug dicts."""
    if hidden_in is None:
        h = np.asarray(weights["embed"], F64)[np.asarray(canvas_tokens, dtype=np.int64)]
    else:
        h = np.asarray(hidden_in, F64)
    n = h.shape[0]
    positions = prefix_len + np.arange(n)
    ks, vs, dbgs = [], [], []
    for l, lw in enumerate(weights["layers"]):
        kp = np.asarray(cache_k[l], F64)[:, :prefix_len]
        vp = np.asarray(cache_v[l], F64)[:, :prefix_len]
        h, k, v, dbg = layer(h, lw, shape, positions, kp, vp, None)
        ks.append(k)
        vs.append(v)
        if keep_debug:
            dbgs.append(dbg)
    out = {"hidden": h, "canvas_k": ks, "canvas_v": vs}
    if keep_debug:
        out["debug"] = dbgs
    if with_head:
        f = rmsnorm(h, weights["final_norm"], shape.rms_eps)
        out["final_normed"] = f
        out["logits"] = f @ np.asarray(weights["lm_head"], F64).T
    return out


def head_logits(f: np.ndarray, lm_head: np.ndarray) -> np.ndarray:
    """Vocab projection of already-normed final states f [n, d] → logits [n, V]."""
    return np.asarray(f, F64) @ np.asarray(lm_head, F64).T


def prefill(weights: Dict, shape, tokens: Sequence[int], cache_k: List[np.ndarray],
            cache_v: List[np.ndarray], start: int = 0):
    """Causal prefill of `tokens` at positions start..start+n-1 into the bf16 caches (in place).

    cache_k/cache_v: per layer float64 arrays [Hkv, cap, D]; positions < start must already hold
    earlier keys.  Each query attends to cached keys at positions <= its own."""
    tok = np.asarray(tokens, dtype=np.int64)
    n = tok.shape[0]
    h = np.asarray(weights["embed"], F64)[tok]
    positions = start + np.arange(n)
    key_pos = np.arange(start + n)
    allowed = key_pos[None, :] <= positions[:, None]
    for l, lw in enumerate(weights["layers"]):
        a = rmsnorm(h, lw["attn_norm"], shape.rms_eps)
        Hq, Hkv, D = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
        q = (a @ np.asarray(lw["wq"], F64).T).reshape(n, Hq, D).transpose(1, 0, 2)
        k = (a @ np.asarray(lw["wk"], F64).T).reshape(n, Hkv, D).transpose(1, 0, 2)
        v = (a @ np.asarray(lw["wv"], F64).T).reshape(n, Hkv, D).transpose(1, 0, 2)
        q = rope(q, positions, shape.rope_theta)
        k = rope(k, positions, shape.rope_theta)
        cache_k[l][:, start:start + n] = to_bf16(k)
        cache_v[l][:, start:start + n] = to_bf16(v)
        K = cache_k[l][:, :start + n]
        V = cache_v[l][:, :start + n]
        o = attention(q, K, V, allowed).transpose(1, 0, 2).reshape(n, Hq * D)
        h = h + o @ np.asarray(lw["wo"], F64).T
        b = rmsnorm(h, lw["ffn_norm"], shape.rms_eps)
        f, _, _, _ = moe(b, lw, shape.top_k)
        h = h + f
    return h


def commit_block_causal(weights: Dict, shape, canvas_tokens: Sequence[int], cache_k: List[np.ndarray],
                        cache_v: List[np.ndarray], prefix_len: int) -> int:
    """The other way to commit a finished canvas: re-encode its tokens causally as a continuation
    of the prompt ([DOCS] feature list: the model also runs as an autoregressive encoder), i.e.
    the causal prefill of the canvas at positions L..L+C-1.  Returns the new length."""
    prefill(weights, shape, canvas_tokens, cache_k, cache_v, prefix_len)
    return prefix_len + len(canvas_tokens)


def commit_block(cache_k: List[np.ndarray], cache_v: List[np.ndarray],
                 canvas_k: List[np.ndarray], canvas_v: List[np.ndarray], prefix_len: int) -> int:
    """Append a finished canvas's K/V (rounded to the cache's bf16) at [L, L+C); return new L.

    [GUIDE] "Arquitetura em Detalhes" and [NEWS] second paragraph: a finished block goes into the
    KV cache and the next canvas conditions on it."""
    C = canvas_k[0].shape[1]
    for l in range(len(cache_k)):
        cache_k[l][:, prefix_len:prefix_len + C] = to_bf16(canvas_k[l])
        cache_v[l][:, prefix_len:prefix_len + C] = to_bf16(canvas_v[l])
    return prefix_len + C
