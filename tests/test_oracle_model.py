"""Pins for the oracle's forward pass: brute force, library routines, closed forms, invariants."""
import dataclasses
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model
from block_discrete_diffusion_amd import synth


def _rng(s=0):
    return np.random.default_rng(s)


# ---------------------------------------------------------------- bf16 rounding, norms, silu

def test_to_bf16_matches_torch():
    x = _rng(1).standard_normal(20000).astype(np.float32) * 10
    # exact ties: the 17th bit set, lower bits zero
    ties = (np.arange(1, 200, dtype=np.uint32) << 16) | (1 << 15)
    x = np.concatenate([x, ties.view(np.float32), np.array([0.0, -0.0, 1e-40, 3e38], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(model.to_bf16(x), want)


def test_rmsnorm_matches_torch_and_unit_rms():
    x = _rng(2).standard_normal((7, 64)) * 3
    g = _rng(3).uniform(0.5, 2, 64)
    want = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(model.rmsnorm(x, g, 1e-6), want, atol=1e-12)
    y = model.rmsnorm(x, np.ones(64), 1e-6)
    assert np.allclose(np.sqrt(np.mean(y * y, -1)), 1.0, atol=1e-6)


def test_silu_closed_form():
    x = np.array([-3.0, 0.0, 1.0, 5.0])
    assert np.allclose(model.silu(x), F.silu(torch.from_numpy(x)).numpy(), atol=1e-15)
    assert model.silu(0.0) == 0.0


def test_softmax_rows_sum_to_one():
    s = _rng(4).standard_normal((9, 33)) * 20
    p = model.softmax(s)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-12)
    assert np.allclose(p, torch.softmax(torch.from_numpy(s), -1).numpy(), atol=1e-14)


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    x = _rng(5).standard_normal((3, 1, 16))
    assert np.array_equal(model.rope(x, [0], 10000.0), x)


def test_rope_preserves_norm_and_is_relative():
    D = 32
    q = _rng(6).standard_normal((1, 1, D))
    k = _rng(7).standard_normal((1, 1, D))
    for m, n in [(5, 2), (105, 102), (40000, 39997)]:
        qm = model.rope(q, [m], 10000.0)
        kn = model.rope(k, [n], 10000.0)
        assert np.isclose(np.linalg.norm(qm), np.linalg.norm(q))
        ref = (model.rope(q, [3], 10000.0) * model.rope(k, [0], 10000.0)).sum()
        assert np.isclose((qm * kn).sum(), ref, atol=1e-9)


def test_rope_matches_complex_rotation():
    """Rotate-half RoPE = multiply (x_j + i x_{j+D/2}) by exp(i pos theta^(-2j/D))."""
    D, pos = 16, 37
    x = _rng(8).standard_normal((2, 1, D))
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    w = np.exp(1j * pos * 10000.0 ** (-2.0 * np.arange(D // 2) / D))
    r = z * w
    want = np.concatenate([r.real, r.imag], -1)
    assert np.allclose(model.rope(x, [pos], 10000.0), want, atol=1e-12)


# ---------------------------------------------------------------- attention

def _attn_bruteforce(q, k, v, allowed):
    Hq, n, D = q.shape
    Hkv, m, _ = k.shape
    out = np.zeros((Hq, n, D))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(n):
            sc = []
            for j in range(m):
                if allowed is None or allowed[i][j]:
                    sc.append((j, sum(q[h, i, d] * k[g, j, d] for d in range(D)) / math.sqrt(D)))
            mx = max(s for _, s in sc)
            w = [(j, math.exp(s - mx)) for j, s in sc]
            tot = sum(e for _, e in w)
            for d in range(D):
                out[h, i, d] = sum(e * v[g, j, d] for j, e in w) / tot
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_attention_bruteforce_gqa(causal):
    Hq, Hkv, D, L, C = 4, 2, 8, 5, 7
    r = _rng(9)
    q = r.standard_normal((Hq, C, D))
    k = r.standard_normal((Hkv, L + C, D))
    v = r.standard_normal((Hkv, L + C, D))
    allowed = None
    if causal:
        allowed = np.arange(L + C)[None, :] <= (L + np.arange(C))[:, None]
    got = model.attention(q, k, v, allowed)
    assert np.allclose(got, _attn_bruteforce(q, k, v, allowed), atol=1e-12)


def test_attention_matches_torch_sdpa():
    Hq, Hkv, D, L, C = 8, 2, 16, 40, 24
    r = _rng(10)
    q, k, v = r.standard_normal((Hq, C, D)), r.standard_normal((Hkv, L + C, D)), r.standard_normal((Hkv, L + C, D))
    kk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, 0)
    vv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, 0)
    want = F.scaled_dot_product_attention(torch.from_numpy(q)[None], kk[None], vv[None])[0].numpy()
    assert np.allclose(model.attention(q, k, v), want, atol=1e-12)


def test_attention_special_cases():
    r = _rng(11)
    D = 8
    q = r.standard_normal((2, 3, D))
    # identical keys → mean of V
    k = np.repeat(r.standard_normal((1, 1, D)), 6, axis=1)
    v = r.standard_normal((1, 6, D))
    assert np.allclose(model.attention(q, k, v), np.broadcast_to(v.mean(1, keepdims=True), (2, 3, D)))
    # one key → that value
    k1, v1 = r.standard_normal((1, 1, D)), r.standard_normal((1, 1, D))
    assert np.allclose(model.attention(q, k1, v1), np.broadcast_to(v1, (2, 3, D)))
    # causal first query → first value
    kc, vc = r.standard_normal((1, 3, D)), r.standard_normal((1, 3, D))
    allowed = np.tril(np.ones((3, 3), bool))
    assert np.allclose(model.attention(q, kc, vc, allowed)[:, 0], np.broadcast_to(vc[0, 0], (2, D)))


# ---------------------------------------------------------------- router / MoE

def test_router_topk_is_stable_full_sort():
    r = _rng(12)
    logits = np.round(r.standard_normal((50, 16)), 1)  # many ties
    idx, gates = model.router_topk(logits, 4)
    for t in range(50):
        order = sorted(range(16), key=lambda e: (-logits[t, e], e))[:4]
        assert list(idx[t]) == order
    assert np.allclose(gates.sum(-1), 1.0)
    sel = np.take_along_axis(logits, idx, -1)
    assert np.allclose(gates, np.exp(sel) / np.exp(sel).sum(-1, keepdims=True))


def _tiny_moe(E, k, d=16, Fd=24, shared=False, seed=13):
    r = _rng(seed)
    lw = {"w_router": r.standard_normal((E, d)), "w_gate": r.standard_normal((E, Fd, d)) * 0.3,
          "w_up": r.standard_normal((E, Fd, d)) * 0.3, "w_down": r.standard_normal((E, d, Fd)) * 0.3}
    if shared:
        lw.update(ws_gate=r.standard_normal((20, d)) * .3, ws_up=r.standard_normal((20, d)) * .3,
                  ws_down=r.standard_normal((d, 20)) * .3)
    return lw, r.standard_normal((9, d))


def test_moe_bruteforce_per_token():
    lw, b = _tiny_moe(6, 2, shared=True)
    out, idx, gates, _ = model.moe(b, lw, 2)
    for t in range(b.shape[0]):
        logits = [float(b[t] @ lw["w_router"][e]) for e in range(6)]
        top = sorted(range(6), key=lambda e: (-logits[e], e))[:2]
        z = sum(math.exp(logits[e]) for e in top)
        acc = np.zeros(b.shape[1])
        for e in top:
            g = b[t] @ lw["w_gate"][e].T
            u = b[t] @ lw["w_up"][e].T
            acc += math.exp(logits[e]) / z * ((g / (1 + np.exp(-g)) * u) @ lw["w_down"][e].T)
        g = b[t] @ lw["ws_gate"].T
        acc += (g / (1 + np.exp(-g)) * (b[t] @ lw["ws_up"].T)) @ lw["ws_down"].T
        assert np.allclose(out[t], acc, atol=1e-12)


def test_moe_k_equals_e_is_dense_mixture():
    lw, b = _tiny_moe(4, 4)
    out, _, _, logits = model.moe(b, lw, 4)
    p = model.softmax(logits)
    want = sum(p[:, e:e + 1] * model.swiglu(b, lw["w_gate"][e], lw["w_up"][e], lw["w_down"][e]) for e in range(4))
    assert np.allclose(out, want, atol=1e-12)


def test_moe_single_expert_is_plain_swiglu():
    lw, b = _tiny_moe(1, 1)
    out, _, gates, _ = model.moe(b, lw, 1)
    assert np.all(gates == 1.0)
    assert np.allclose(out, model.swiglu(b, lw["w_gate"][0], lw["w_up"][0], lw["w_down"][0]), atol=1e-12)


# ---------------------------------------------------------------- layer / forward / prefill

SMALL = synth.ModelShape(n_layers=2, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8,
                         n_experts=4, top_k=2, d_ff_expert=24, d_ff_shared=16, vocab=50, canvas=6)


def _weights(shape, seed=1):
    return synth.model_weights(shape, seed)


def test_canvas_attention_is_unmasked_permutation_equivariant():
    """Without positions, permuting the canvas permutes the output: no causal mask inside."""
    shape = dataclasses.replace(SMALL, rope_theta=0.0)
    w = _weights(shape)
    ck, cv = [np.zeros((2, 8, 8)) for _ in range(2)], [np.zeros((2, 8, 8)) for _ in range(2)]
    r = _rng(14)
    for l in range(2):
        ck[l][:, :3] = r.standard_normal((2, 3, 8))
        cv[l][:, :3] = r.standard_normal((2, 3, 8))
    toks = np.array([3, 9, 1, 40, 22, 7])
    perm = np.array([5, 2, 0, 4, 1, 3])
    a = model.denoise_forward(w, shape, toks, ck, cv, 3)["logits"]
    b = model.denoise_forward(w, shape, toks[perm], ck, cv, 3)["logits"]
    assert np.allclose(a[perm], b, atol=1e-10)
    # and a later canvas token does influence an earlier one (not causal)
    toks2 = toks.copy()
    toks2[-1] = 11
    c = model.denoise_forward(w, shape, toks2, ck, cv, 3)["logits"]
    assert not np.allclose(a[0], c[0])


def test_prefill_is_causal_and_chunkable():
    w = _weights(SMALL)
    toks = synth.tokens(10, SMALL.vocab, 3)
    ck1, cv1 = [np.zeros((2, 10, 8)) for _ in range(2)], [np.zeros((2, 10, 8)) for _ in range(2)]
    h1 = model.prefill(w, SMALL, toks, ck1, cv1, 0)
    # chunked prefill gives the same cache
    ck2, cv2 = [np.zeros((2, 10, 8)) for _ in range(2)], [np.zeros((2, 10, 8)) for _ in range(2)]
    model.prefill(w, SMALL, toks[:4], ck2, cv2, 0)
    h2 = model.prefill(w, SMALL, toks[4:], ck2, cv2, 4)
    for l in range(2):
        assert np.allclose(ck1[l], ck2[l], atol=1e-2) and np.allclose(cv1[l], cv2[l], atol=1e-2)
    assert np.allclose(h1[4:], h2, atol=1e-2)
    # changing a later token leaves earlier positions' cache untouched
    toks3 = toks.copy()
    toks3[7] = (toks3[7] + 1) % SMALL.vocab
    ck3, cv3 = [np.zeros((2, 10, 8)) for _ in range(2)], [np.zeros((2, 10, 8)) for _ in range(2)]
    model.prefill(w, SMALL, toks3, ck3, cv3, 0)
    for l in range(2):
        assert np.array_equal(ck1[l][:, :7], ck3[l][:, :7])
        assert not np.array_equal(ck1[l][:, 7:], ck3[l][:, 7:])


def test_cache_holds_bf16_values():
    w = _weights(SMALL)
    ck, cv = [np.zeros((2, 10, 8)) for _ in range(2)], [np.zeros((2, 10, 8)) for _ in range(2)]
    model.prefill(w, SMALL, synth.tokens(10, SMALL.vocab, 4), ck, cv, 0)
    for a in ck + cv:
        assert np.array_equal(a, model.to_bf16(a))


def test_layer_mha_when_kv_heads_equal_q_heads():
    """GQA with Hkv == Hq is plain multi-head attention: each head reads its own K/V."""
    shape = dataclasses.replace(SMALL, n_kv_heads=4, n_layers=1)
    w = _weights(shape)
    h = synth.hidden(6, 32, 5).astype(np.float64)
    out, k, v, dbg = model.layer(h, w["layers"][0], shape, np.arange(6), np.zeros((4, 0, 8)),
                                 np.zeros((4, 0, 8)), None)
    q = dbg["q"]
    for hh in range(4):
        s = q[hh] @ k[hh].T / math.sqrt(8)
        p = np.exp(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        assert np.allclose(dbg["attn_out"][:, hh * 8:(hh + 1) * 8], p @ v[hh], atol=1e-12)


def test_commit_block_appends_rounded_kv():
    ck, cv = [np.zeros((2, 9, 8))], [np.zeros((2, 9, 8))]
    r = _rng(15)
    k, v = [r.standard_normal((2, 3, 8))], [r.standard_normal((2, 3, 8))]
    L = model.commit_block(ck, cv, k, v, 4)
    assert L == 7
    assert np.array_equal(ck[0][:, 4:7], model.to_bf16(k[0]))
    assert np.array_equal(cv[0][:, 4:7], model.to_bf16(v[0]))
    assert not ck[0][:, :4].any() and not ck[0][:, 7:].any()
