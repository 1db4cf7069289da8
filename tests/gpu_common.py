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


# Values the GPU stores as bfloat16 (K/V cache entries, attention output) are rounded to the
# nearest bf16 value, which moves them by at most half a bf16 step, 2^-8 of the value's magnitude.
BF16_ULP = 2.0 ** -8


def close(got, want, max_abs=MAX_ABS, rel_l2=REL_L2, what="", bf16_out=False):
    """Element-wise |got - want| <= max_abs (plus half a bf16 step of want for bf16-stored values)
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


# End to end (tokens through every layer, no teacher forcing) the router inputs on the two sides
# differ by the attention blocks' bf16-level error, so experts whose logits lie within this bound
# of the k-th may legitimately swap there.
ROUTER_BOUND = 2e-2


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
        "route_offs": z(n_layers, shape.n_experts + 1, dt=torch.int32),
        "route_perm": z(n_layers, rows * shape.top_k, dt=torch.int32),
        "route_inv": z(n_layers, rows * shape.top_k, dt=torch.int32),
    }


def check_ffn_teacher_forced(lw, shape, h_mid, gpu_idx, gpu_gates, gpu_out, tag=""):
    """The FFN sub-block (norm, router, top-k, gates, routed experts, shared FFN, residual) of the
    oracle fed the GPU's own residual after attention, so both sides start from identical values.
    Expert sets must be equal wherever the oracle's k-th/(k+1)-th router logit gap is >= MARGIN
    (the two sides' logits then differ only by accumulation order); inside that gap the GPU's
    picks must be a valid top-k within MARGIN.  Gates, the FFN output and the layer output are
    compared on every row outside the gap.  Returns the mask of those rows."""
    h_mid = np.asarray(h_mid, np.float64)
    b = omodel.rmsnorm(h_mid, lw["ffn_norm"], shape.rms_eps)
    f, o_idx, o_gates, logits = omodel.moe(b, lw, shape.top_k)
    k = shape.top_k
    clear = topk_margin(logits, k) >= MARGIN
    gi = np.asarray(gpu_idx, np.int64)
    same = np.all(np.sort(gi, 1) == np.sort(o_idx, 1), axis=1)
    assert same[clear].all(), f"{tag}: expert set differs on {int((~same[clear]).sum())} rows with a clear margin"
    kth = np.sort(logits, axis=1)[:, ::-1][:, k - 1]
    picked = np.take_along_axis(logits, gi, 1)
    assert np.all(picked[~same] >= kth[~same, None] - MARGIN), f"{tag}: GPU picked an expert below the k-th"
    assert np.all(np.diff(np.sort(gi, 1), axis=1) != 0), f"{tag}: an expert picked twice in one row"
    # gates paired with their experts (the order inside the k picks may differ at equal logits)
    og = np.take_along_axis(o_gates, np.argsort(o_idx, 1), 1)
    gg = np.take_along_axis(np.asarray(gpu_gates, np.float64), np.argsort(gi, 1), 1)
    close(gg[clear], og[clear], max_abs=1e-4, rel_l2=1e-4, what=f"gates {tag}")
    gpu_out = np.asarray(gpu_out, np.float64)
    close((gpu_out - h_mid)[clear], f[clear], what=f"FFN output {tag}")
    close(gpu_out[clear], (h_mid + f)[clear], what=f"layer output {tag}")
    return clear


def check_layer(dg, m, w, shape, Lp, seed, cap, cache=None):
    """One layer from a synthetic residual state: attention, canvas K/V and the residual after
    attention against the oracle layer on the same input; the FFN sub-block teacher-forced on the
    GPU's residual after attention (every row outside the router's tie gap).  cache: the prefix
    (k, v) as numpy [n_layers, 1, Hkv, cap, D] bf16 values (default: random_cache)."""
    kv = dg.KV(shape, 1, cap)
    k, v = random_cache(shape, Lp, cap, seed) if cache is None else cache
    load_cache(kv, k, v, [Lp])
    h = synth.hidden(256, shape.d_model, seed, 5)
    dbg = layer_debug(dg, m, shape, 256, shape.n_layers)
    m.denoise_step(None, kv, None, 0, None, flags=dg.DG_STEP_HIDDEN_IN | dg.DG_STEP_NO_HEAD,
                   hidden_in=torch.from_numpy(h).cuda(), debug=dbg)
    torch.cuda.synchronize()
    pos = Lp + np.arange(256)
    _, ok_k, ok_v, od = omodel.layer(h, w["layers"][0], shape, pos, k[0, 0, :, :Lp], v[0, 0, :, :Lp], None)
    close(bf16_to_np(dbg["attn_out"][0]), od["attn_out"], what="attention output", bf16_out=True)
    close(dbg["h_mid"][0].cpu().numpy(), od["h_mid"], what="h after attention")
    close(bf16_to_np(dbg["canvas_k"][0, 0]), ok_k, what="canvas K", bf16_out=True)
    close(bf16_to_np(dbg["canvas_v"][0, 0]), ok_v, what="canvas V", bf16_out=True)
    clear = check_ffn_teacher_forced(w["layers"][0], shape, dbg["h_mid"][0].cpu().numpy(),
                                     dbg["expert_idx"][0].cpu().numpy(), dbg["gates"][0].cpu().numpy(),
                                     dbg["hidden_out"].cpu().numpy(), "layer 0")
    check_routes(dbg, shape, 256, 0)
    return clear


def check_routes(dbg, shape, rows, l):
    """Route tables of layer l (when dumped): the permutation is the stable sort of the routes
    r = row * top_k + j by their expert, bit for bit; offsets and the inverse follow from it."""
    if "route_perm" not in dbg:
        return
    k, E = shape.top_k, shape.n_experts
    idx = dbg["expert_idx"][l].cpu().numpy().reshape(-1).astype(np.int64)
    assert idx.size == rows * k
    want_perm = np.argsort(idx, kind="stable")
    want_offs = np.searchsorted(idx[want_perm], np.arange(E + 1), side="left")
    want_offs[E] = rows * k
    perm = dbg["route_perm"][l][:rows * k].cpu().numpy()
    inv = dbg["route_inv"][l][:rows * k].cpu().numpy()
    offs = dbg["route_offs"][l].cpu().numpy()
    assert np.array_equal(offs, want_offs), f"layer {l}: expert offsets"
    assert np.array_equal(perm, want_perm), f"layer {l}: route permutation"
    want_inv = np.empty_like(want_perm)
    want_inv[want_perm] = np.arange(want_perm.size)
    assert np.array_equal(inv, want_inv), f"layer {l}: inverse permutation"


def check_layers_teacher_forced(w, shape, dbg, b, tokens, cache_k, cache_v, Lb, h0=None):
    """Every layer of request b's canvas against the oracle layer fed the GPU's own input to that
    layer (the token embedding for layer 0, the GPU's previous layer output after that), over
    the same cached prefix; inside each layer the FFN sub-block is fed the GPU's own residual
    after attention.  Compares the canvas K/V, the attention output and the residual after
    attention (all rows), the expert choice, gates, FFN and layer output (every row outside the
    router's tie gap).  A router near-tie that flips an expert then cannot move any other row or
    layer's inputs.

    dbg: the layer_debug buffers of a denoise step; cache_k/cache_v: per layer [Hkv, >=Lb, D];
    h0: the request's [256, d] residual input when the step ran on a given hidden state
    (DG_STEP_HIDDEN_IN) instead of token embeddings."""
    sl = slice(b * 256, (b + 1) * 256)
    pos = Lb + np.arange(256)
    if h0 is not None:
        h_in = np.asarray(h0, np.float64)
    else:
        h_in = np.asarray(w["embed"], np.float64)[np.asarray(tokens, np.int64)]
    n_clear = []
    for l in range(shape.n_layers):
        if l > 0:
            h_in = dbg["layer_out"][l - 1][sl].cpu().numpy().astype(np.float64)
        _, k, v, od = omodel.layer(h_in, w["layers"][l], shape, pos, cache_k[l][:, :Lb], cache_v[l][:, :Lb], None)
        tag = f"request {b} layer {l}"
        close(bf16_to_np(dbg["canvas_k"][l, b]), k, what=f"canvas K {tag}", bf16_out=True)
        close(bf16_to_np(dbg["canvas_v"][l, b]), v, what=f"canvas V {tag}", bf16_out=True)
        close(bf16_to_np(dbg["attn_out"][l][sl]), od["attn_out"], what=f"attention {tag}", bf16_out=True)
        close(dbg["h_mid"][l][sl].cpu().numpy(), od["h_mid"], what=f"residual after attention {tag}")
        clear = check_ffn_teacher_forced(w["layers"][l], shape, dbg["h_mid"][l][sl].cpu().numpy(),
                                         dbg["expert_idx"][l][sl].cpu().numpy(), dbg["gates"][l][sl].cpu().numpy(),
                                         dbg["layer_out"][l][sl].cpu().numpy(), tag)
        n_clear.append(int(clear.sum()))
    return n_clear
