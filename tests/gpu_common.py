"""Shared helpers for the GPU parity tests (imported only by tests marked `gpu`)."""
import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import synth
from oracle import model as omodel

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


# Values the GPU stores as bfloat16 (K/V cache entries, attention output) can land one bf16 ulp
# (at most 2^-7 of the value) further from the float64 oracle than the value before rounding.
BF16_ULP = 2.0 ** -7


def close(got, want, max_abs=MAX_ABS, rel_l2=REL_L2, what="", bf16_out=False):
    """Element-wise |got - want| <= max_abs (plus one bf16 ulp of want for bf16-stored values)
    and relative L2 error <= rel_l2."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    bound = max_abs + (BF16_ULP * np.abs(want) if bf16_out else 0.0)
    excess = float((err - bound).max()) if err.size else 0.0
    mx = float(err.max()) if err.size else 0.0
    rl = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    assert excess <= 0.0 and rl <= rel_l2, f"{what}: max-abs {mx:.3g} (bound excess {excess:.3g}) rel-L2 {rl:.3g}"
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
                                 renoise_committed=bool(cfg.renoise_committed), seed=cfg.seed,
                                 select_mode=cfg.select_mode,
                                 entropy_budget=float(np.float32(cfg.entropy_budget)))


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


def layer_debug(dg, m, shape, rows, n_layers, batch=1):
    HD = shape.n_q_heads * shape.head_dim
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt, device="cuda")
    return {
        "hidden_out": z(rows, shape.d_model),
        "attn_out": z(n_layers, rows, HD, dt=torch.bfloat16),
        "h_mid": z(n_layers, rows, shape.d_model),
        "expert_idx": z(n_layers, rows, shape.top_k, dt=torch.int32),
        "gates": z(n_layers, rows, shape.top_k),
        "canvas_k": z(n_layers, batch, shape.n_kv_heads, 256, shape.head_dim, dt=torch.bfloat16),
        "canvas_v": z(n_layers, batch, shape.n_kv_heads, 256, shape.head_dim, dt=torch.bfloat16),
        "layer_out": z(n_layers, rows, shape.d_model),
    }


def check_layer(dg, m, w, shape, Lp, seed, cap, min_safe=0.75):
    """One layer from a synthetic residual state: attention, FFN and canvas K/V vs the oracle."""
    kv = dg.KV(shape, 1, cap)
    k, v = random_cache(shape, Lp, cap, seed)
    load_cache(kv, k, v, [Lp])
    h = synth.hidden(256, shape.d_model, seed, 5)
    dbg = layer_debug(dg, m, shape, 256, shape.n_layers)
    m.denoise_step(None, kv, None, 0, None, flags=dg.DG_STEP_HIDDEN_IN | dg.DG_STEP_NO_HEAD,
                   hidden_in=torch.from_numpy(h).cuda(), debug=dbg)
    torch.cuda.synchronize()
    pos = Lp + np.arange(256)
    h_out, ok_k, ok_v, od = omodel.layer(h, w["layers"][0], shape, pos, k[0, 0, :, :Lp], v[0, 0, :, :Lp], None)
    close(bf16_to_np(dbg["attn_out"][0]), od["attn_out"], what="attention output", bf16_out=True)
    close(dbg["h_mid"][0].cpu().numpy(), od["h_mid"], what="h after attention")
    close(bf16_to_np(dbg["canvas_k"][0, 0]), ok_k, what="canvas K", bf16_out=True)
    close(bf16_to_np(dbg["canvas_v"][0, 0]), ok_v, what="canvas V", bf16_out=True)
    gi = dbg["expert_idx"][0].cpu().numpy()
    safe = check_topk(gi, od["router_logits"], shape.top_k)
    assert safe.mean() > min_safe, safe.mean()
    order_ok = np.all(gi == od["expert_idx"], axis=1) & safe
    close(dbg["gates"][0].cpu().numpy()[order_ok], od["gates"][order_ok], max_abs=1e-2, what="gates")
    close(dbg["hidden_out"].cpu().numpy()[safe], h_out[safe], what="layer output")
    close((dbg["hidden_out"].cpu().numpy() - dbg["h_mid"][0].cpu().numpy())[safe], od["ffn_out"][safe],
          what="FFN output")


def check_layers_teacher_forced(w, shape, dbg, b, tokens, cache_k, cache_v, Lb, min_safe=0.7):
    """Every layer of request b's canvas against the oracle layer fed the GPU's own input to that
    layer (the token embedding for layer 0, the GPU's previous layer output after that), over
    the same cached prefix.  A router near-tie that flips an expert only moves that row's FFN
    output inside its layer; feeding each layer the GPU's input keeps it from reaching the other
    rows through the next layer's attention.  Compares the canvas K/V, the attention output and
    residual (all rows), the expert choice, and the layer output on rows with a clear choice.

    dbg: the layer_debug buffers of a denoise step; cache_k/cache_v: per layer [Hkv, >=Lb, D]."""
    sl = slice(b * 256, (b + 1) * 256)
    pos = Lb + np.arange(256)
    h_in = np.asarray(w["embed"], np.float64)[np.asarray(tokens, np.int64)]
    n_safe = []
    for l in range(shape.n_layers):
        if l > 0:
            h_in = dbg["layer_out"][l - 1][sl].cpu().numpy().astype(np.float64)
        h_out, k, v, od = omodel.layer(h_in, w["layers"][l], shape, pos, cache_k[l][:, :Lb],
                                       cache_v[l][:, :Lb], None)
        tag = f"request {b} layer {l}"
        close(bf16_to_np(dbg["canvas_k"][l, b]), k, what=f"canvas K {tag}", bf16_out=True)
        close(bf16_to_np(dbg["canvas_v"][l, b]), v, what=f"canvas V {tag}", bf16_out=True)
        close(bf16_to_np(dbg["attn_out"][l][sl]), od["attn_out"], what=f"attention {tag}", bf16_out=True)
        close(dbg["h_mid"][l][sl].cpu().numpy(), od["h_mid"], what=f"residual after attention {tag}")
        safe = check_topk(dbg["expert_idx"][l][sl].cpu().numpy(), od["router_logits"], shape.top_k)
        assert safe.mean() > min_safe, (tag, safe.mean())
        close(dbg["layer_out"][l][sl].cpu().numpy()[safe], h_out[safe], what=f"layer output {tag}")
        n_safe.append(int(safe.sum()))
    return n_safe
