"""GPU vs oracle parity on the small configuration (2 layers, d 256, 4/2 heads, D 64, 8 experts
top-2, F 512, V 1024, prefix 64, one 256-token canvas).  Every call goes through the C ABI."""
import dataclasses

import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import synth
from oracle import fp8 as ofp8
from oracle import model as omodel
from oracle import sampler as osampler
from tests.gpu_common import (MARGIN, ROUTER_BOUND, bf16_to_np, check_layer, close, layer_debug,
                              load_cache, need_gpu, np_bf16_dev, oracle_cfg, random_cache, topk_margin)

pytestmark = pytest.mark.gpu

SHAPE = synth.TINY
L = 64
SEED = 20260610


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    w = synth.model_weights(SHAPE, SEED)
    m = dg.Model(SHAPE, w, max_batch=2, max_prefill_rows=512)
    yield dg, w, m
    m.close()


def _kv(dg, cap=L + 512, batch=1, seed=7):
    kv = dg.KV(SHAPE, batch, cap)
    k, v = random_cache(SHAPE, L, cap, seed, batch)
    load_cache(kv, k, v, [L] * batch)
    return kv, k, v


def test_canvas_init_bitexact(env):
    dg, w, m = env
    kv, _, _ = _kv(dg, batch=2)
    kv.set_lengths([L, L + 256])
    st = dg.Canvas(2, 256)
    cfg = dg.sampler_cfg(seed=123456789012345)
    m.canvas_init(st, kv, cfg)
    torch.cuda.synchronize()
    for b, Lb in enumerate([L, L + 256]):
        want = osampler.canvas_init(cfg.seed, b, Lb + np.arange(256), SHAPE.vocab)
        assert np.array_equal(st.tokens[b].cpu().numpy(), want)
    assert not st.committed.any() and not st.stable_run.any() and not st.stopped.any()


@pytest.mark.parametrize("step", [0, 17, 47])
def test_head_decisions_and_stats(env, step):
    """Teacher-forced head: identical bf16 final states f and W_out on both sides."""
    dg, w, m = env
    kv, _, _ = _kv(dg)
    f = synth.bf16_normal((256, SHAPE.d_model), SEED, 30 + step)
    x = synth.tokens(256, SHAPE.vocab, SEED, 31 + step)
    cfg = dg.sampler_cfg(seed=99 + step)
    stats = dg.Stats(1, 256)
    logits = torch.zeros((256, SHAPE.vocab), dtype=torch.float32, device="cuda")
    tok = torch.from_numpy(x).cuda()
    m.denoise_step(tok, kv, cfg, step, stats, flags=dg.DG_STEP_HEAD_ONLY, hidden_in=np_bf16_dev(f),
                   debug={"logits": logits})
    torch.cuda.synchronize()
    oc = oracle_cfg(cfg)
    z = omodel.head_logits(f, w["lm_head"])
    close(logits.cpu().numpy(), z, what="logits")
    T = osampler.temperature(oc, step)
    assert np.float32(dg.temperature(cfg, step)) == T
    want = osampler.row_stats(z, x, T, cfg.seed, 0, L + np.arange(256), step)
    got_cand = stats.cand.cpu().numpy()[0]
    ok = want["margin"] >= MARGIN
    assert ok.mean() > 0.9
    assert np.array_equal(got_cand[ok], want["cand"][ok])
    for k in ("t_cand", "t_cur", "lse"):
        close(getattr(stats, k).cpu().numpy()[0][ok], want[k][ok], max_abs=1e-3, rel_l2=1e-5, what=k)
    close(stats.entropy.cpu().numpy()[0], want["entropy"], max_abs=1e-3, rel_l2=1e-4, what="entropy")


@pytest.mark.parametrize("select_mode", [0, 1])
def test_sampler_bitexact_over_steps(env, select_mode):
    """dg_sample_commit on identical float32 row statistics is bit-exact against the oracle,
    under both selection rules (top-m by confidence; entropy-bounded)."""
    dg, w, m = env
    kv, _, _ = _kv(dg, batch=2)
    kv.set_lengths([L, 3 * L])
    cfg = dg.sampler_cfg(seed=4242, max_steps=12, commit_per_step=16, select_mode=select_mode)
    oc = oracle_cfg(cfg)
    st = dg.Canvas(2, 256)
    m.canvas_init(st, kv, cfg)
    torch.cuda.synchronize()
    o_state = []
    for b, Lb in enumerate([L, 3 * L]):
        o_state.append([osampler.canvas_init(cfg.seed, b, Lb + np.arange(256), SHAPE.vocab),
                        np.zeros(256, bool), 0])
    stats = dg.Stats(2, 256)
    status = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    for s in range(cfg.max_steps):
        # confidences spread around log(0.1) so commit, keep and re-noise all occur
        rs = {
            "cand": synth.tokens(512, SHAPE.vocab, s, 1).reshape(2, 256),
            "t_cand": synth.uniform((2, 256), -4.0, 0.5, s, 2),
            "t_cur": synth.uniform((2, 256), -4.0, 0.5, s, 3),
            "lse": synth.uniform((2, 256), 0.0, 0.5, s, 4),
            "entropy": synth.uniform((2, 256), 0.0, 3.0, s, 5),
        }
        rs["t_cand"][:, ::7] = rs["t_cand"][:, 3:4]  # exact ties in the ranking
        if select_mode == 1:
            # a low-entropy third so that the budget admits several slots per step; values on a
            # 1/4096 grid give exact ties and zeros
            low = synth.uniform((2, 256), 0.0, 0.03, s, 6)
            pick = synth.uniform((2, 256), 0.0, 1.0, s, 7) < 0.33
            rs["entropy"] = np.where(pick, np.floor(low * 4096) / 4096, rs["entropy"]).astype(np.float32)
        for k, v in rs.items():
            getattr(stats, k).copy_(torch.from_numpy(np.ascontiguousarray(v)))
        m.sample_commit(st, stats, cfg, s, kv, status)
        torch.cuda.synchronize()
        got = dg.status_dict(status)
        for b, Lb in enumerate([L, 3 * L]):
            ost = {k: rs[k][b] for k in rs}
            x, com, sr, ostatus = osampler.sample_commit(ost, o_state[b][0], o_state[b][1], o_state[b][2],
                                                        oc, s, b, Lb + np.arange(256), SHAPE.vocab)
            o_state[b] = [x, com, sr]
            assert np.array_equal(st.tokens[b].cpu().numpy(), x), (s, b)
            assert np.array_equal(st.committed[b].cpu().numpy().astype(bool), com), (s, b)
            assert int(st.stable_run[b]) == sr
            for k in ("changed", "n_committed", "n_new", "n_renoised", "stable_run", "stop"):
                assert got[b][k] == ostatus[k], (s, b, k)
            assert abs(got[b]["mean_entropy"] - ostatus["mean_entropy"]) < 1e-5
        if all(g["stop"] for g in got):
            break


def test_single_layer_parity(env):
    dg, w, _ = env
    shape = dataclasses.replace(SHAPE, n_layers=1)
    w1 = dict(w)
    w1["layers"] = w["layers"][:1]
    m1 = dg.Model(shape, w1, max_batch=1)
    try:
        check_layer(dg, m1, w1, shape, L, SEED, L + 256)
        check_layer(dg, m1, w1, shape, 0, SEED + 1, 256)       # no prefix: pure canvas attention
        check_layer(dg, m1, w1, shape, 1000, SEED + 2, 1300)   # ragged prefix, several key tiles
    finally:
        m1.close()


@pytest.mark.parametrize("cols", [2048, 768, 1000, 1])
def test_quantize_e4m3_rows_bitexact(cols):
    """dg_quantize_e4m3_rows gives the oracle's bytes and scales exactly: rows over six orders
    of magnitude (so that small weights fall in the subnormal codes), an all-zero row, a row
    with a single non-zero entry."""
    dg = need_gpu()
    rows = 64
    r = np.random.default_rng(cols)
    w = r.standard_normal((rows, cols)) * np.logspace(-4, 2, rows)[:, None]
    w[5] = 0.0
    w[6] = 0.0
    w[6, cols // 2] = -3.0
    w[7] *= np.where(r.random(cols) < 0.5, 1e-4, 1.0)  # wide range inside one row
    wd = np_bf16_dev(w.reshape(rows, cols))
    wq = bf16_to_np(wd)
    q = torch.zeros((rows, cols), dtype=torch.uint8, device="cuda")
    sc = torch.zeros(rows, dtype=torch.float32, device="cuda")
    dg.quantize_e4m3_rows(wd, q, sc)
    torch.cuda.synchronize()
    want_q, want_s = ofp8.quantize_rows(wq)
    assert np.array_equal(sc.cpu().numpy(), want_s)
    got = q.cpu().numpy()
    bad = np.argwhere(got != want_q)
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])] if bad.size else None)
    assert np.any(((want_q & 0x78) == 0) & ((want_q & 7) != 0)) or cols == 1  # subnormal codes were exercised


def test_fp8_expert_layer_parity(env):
    """Routed experts as E4M3 bytes with per-channel scales, quantized by dg_create: one layer
    against the oracle layer whose experts are the oracle's own E4M3 round trip of the same
    weights (attention, router and norms as in bf16)."""
    dg, w, _ = env
    shape = dataclasses.replace(SHAPE, n_layers=1, expert_fp8=True)
    w1 = dict(w)
    w1["layers"] = w["layers"][:1]
    m1 = dg.Model(shape, w1, max_batch=1)
    try:
        wo = dict(w1)
        wo["layers"] = [ofp8.dequantize_experts({k: np.asarray(v) for k, v in w1["layers"][0].items()})]
        check_layer(dg, m1, wo, shape, L, SEED + 11, L + 256)
        check_layer(dg, m1, wo, shape, 300, SEED + 12, 600)
    finally:
        m1.close()


def _peaked_stats(V, target, T, seed, pos, step, x):
    z = np.zeros((256, V))
    z[np.arange(256), target] = 50.0
    return osampler.row_stats(z, x, T, seed, 0, pos, step)


@pytest.mark.parametrize("select_mode", [0, 1])
def test_entropy_stop_on_peaked_logits(env, select_mode):
    """DiffusionGemma docs, table "Configuração de exibição recomendada", adaptive-stop row: with
    the mean-entropy stop on (0.005), the peaked-logits fixture (z = 50 onehot(target): every
    draw is the target, entropy ~0) ends after exactly two steps, one step before the stable-run
    rule would, under both selection rules.  The GPU sampler is fed the oracle's row statistics
    of the same fixture each step and must follow the oracle's trajectory bit for bit."""
    dg, w, m = env
    V = SHAPE.vocab
    kv, _, _ = _kv(dg)
    cfg = dg.sampler_cfg(seed=31, select_mode=select_mode, entropy_stop=0.005)
    oc = oracle_cfg(cfg)
    target = synth.tokens(256, V, SEED, 60)
    pos = L + np.arange(256)
    st = dg.Canvas(1, 256)
    m.canvas_init(st, kv, cfg)
    stats = dg.Stats(1, 256)
    status = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    x, com, sr = osampler.canvas_init(cfg.seed, 0, pos, V), np.zeros(256, bool), 0
    n_steps = 0
    for s in range(cfg.max_steps):
        rs = _peaked_stats(V, target, osampler.temperature(oc, s), cfg.seed, pos, s, x)
        for k in ("cand", "t_cand", "t_cur", "lse", "entropy"):
            getattr(stats, k)[0].copy_(torch.from_numpy(np.ascontiguousarray(rs[k])))
        m.sample_commit(st, stats, cfg, s, kv, status)
        torch.cuda.synchronize()
        x, com, sr, ost = osampler.sample_commit(rs, x, com, sr, oc, s, 0, pos, V)
        got = dg.status_dict(status)[0]
        assert np.array_equal(st.tokens[0].cpu().numpy(), x), s
        assert np.array_equal(st.committed[0].cpu().numpy().astype(bool), com), s
        for k in ("changed", "n_committed", "n_new", "n_renoised", "stable_run", "stop"):
            assert got[k] == ost[k], (s, k)
        n_steps += 1
        if got["stop"]:
            break
    assert n_steps == 2
    assert np.array_equal(x, target)


def test_entropy_stop_decision_around_the_threshold(env):
    """Mean entropies just below and just above the 0.005 threshold: the GPU's float32 sum in
    a fixed tree and the oracle's float64 mean take the same stop decision wherever the oracle's
    mean is more than 1e-7 (2e-5 relative) from the threshold; the reported mean agrees to
    1e-6 relative.  Candidates equal the current tokens at full confidence, so no step changes
    the canvas and only the entropy condition can stop it (stable-run limit set out of reach)."""
    dg, w, m = env
    V = SHAPE.vocab
    kv, _, _ = _kv(dg)
    cfg = dg.sampler_cfg(seed=32, entropy_stop=0.005, stable_steps=1000)
    oc = oracle_cfg(cfg)
    pos = L + np.arange(256)
    stats = dg.Stats(1, 256)
    status = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    decided = 0
    for i, rel in enumerate([0.5, 0.99, 0.9999, 1.0001, 1.01, 2.0, 0.99995, 1.00005]):
        st = dg.Canvas(1, 256)
        m.canvas_init(st, kv, cfg)
        torch.cuda.synchronize()
        x = st.tokens[0].cpu().numpy()
        ent = synth.uniform((256,), 0.0, 2.0, SEED, 80 + i)
        ent = (ent * np.float32(0.005 * rel / float(np.mean(ent.astype(np.float64))))).astype(np.float32)
        rs = {"cand": x.astype(np.int32), "t_cand": np.zeros(256, np.float32), "t_cur": np.zeros(256, np.float32),
              "lse": np.zeros(256, np.float32), "entropy": ent}
        for k, val in rs.items():
            getattr(stats, k)[0].copy_(torch.from_numpy(np.ascontiguousarray(val)))
        m.sample_commit(st, stats, cfg, 3, kv, status)
        torch.cuda.synchronize()
        _, _, _, ost = osampler.sample_commit(rs, x, np.zeros(256, bool), 0, oc, 3, 0, pos, V)
        got = dg.status_dict(status)[0]
        assert got["changed"] == 0 == ost["changed"]
        assert abs(got["mean_entropy"] - ost["mean_entropy"]) <= 1e-6 * ost["mean_entropy"]
        if abs(ost["mean_entropy"] - 0.005) > 1e-7:
            assert got["stop"] == ost["stop"] == int(rel < 1), (rel, got, ost["mean_entropy"])
            decided += 1
    assert decided >= 6


def test_full_step_parity(env):
    """Tokens → 2 layers → head: continuous row statistics within the parity bar; decisions
    compared where the oracle margin is safely away from a tie."""
    dg, w, m = env
    kv, k, v = _kv(dg)
    x = synth.tokens(256, SHAPE.vocab, SEED, 40)
    cfg = dg.sampler_cfg(seed=5)
    stats = dg.Stats(1, 256)
    logits = torch.zeros((256, SHAPE.vocab), dtype=torch.float32, device="cuda")
    m.denoise_step(torch.from_numpy(x).cuda(), kv, cfg, 3, stats, debug={"logits": logits})
    torch.cuda.synchronize()
    fw = omodel.denoise_forward(w, SHAPE, x, [k[l, 0] for l in range(2)], [v[l, 0] for l in range(2)], L,
                                keep_debug=True)
    # rows whose expert choice is unique in every layer (no near-tie in the oracle's router)
    safe = np.ones(256, bool)
    for dl in fw["debug"]:
        safe &= topk_margin(dl["router_logits"], SHAPE.top_k) >= ROUTER_BOUND
    assert safe.mean() > 0.75, safe.mean()
    # each sub-block meets the 2e-2 bar on identical inputs; end to end the per-block errors
    # add up over the n_layers + 1 blocks on the path (rel-L2 keeps the 1e-2 bar)
    close(logits.cpu().numpy()[safe], fw["logits"][safe], max_abs=2e-2 * (SHAPE.n_layers + 1),
          what="logits (end to end)")
    oc = oracle_cfg(cfg)
    want = osampler.row_stats(fw["logits"], x, osampler.temperature(oc, 3), cfg.seed, 0, L + np.arange(256), 3)
    close(stats.lse.cpu().numpy()[0][safe], want["lse"][safe], max_abs=2e-2, what="lse")
    close(stats.t_cur.cpu().numpy()[0][safe], want["t_cur"][safe], max_abs=5e-2, what="t_cur")
    agree = (stats.cand.cpu().numpy()[0] == want["cand"])
    clear = safe & (want["margin"] >= 0.1)
    assert agree[clear].mean() > 0.97, agree[clear].mean()


def test_prefill_matches_oracle(env):
    dg, w, m = env
    toks = synth.tokens(L, SHAPE.vocab, SEED, 50)
    kv = dg.KV(SHAPE, 1, L + 256)
    m.prefill(torch.from_numpy(toks).cuda(), [L], kv)
    torch.cuda.synchronize()
    assert kv.lengths == [L]
    ck = [np.zeros((2, L + 256, 64)) for _ in range(2)]
    cv = [np.zeros((2, L + 256, 64)) for _ in range(2)]
    omodel.prefill(w, SHAPE, toks, ck, cv, 0)
    for l in range(2):
        close(bf16_to_np(kv.k[l, 0, :, :L]), ck[l][:, :L], what=f"prefill K layer {l}", bf16_out=True)
        close(bf16_to_np(kv.v[l, 0, :, :L]), cv[l][:, :L], what=f"prefill V layer {l}", bf16_out=True)


def test_prefill_chunked_equals_whole(env):
    dg, w, m = env
    toks = synth.tokens(200, SHAPE.vocab, SEED, 51)
    a = dg.KV(SHAPE, 1, 512)
    m.prefill(torch.from_numpy(toks).cuda(), [200], a)
    b = dg.KV(SHAPE, 1, 512)
    m.prefill(torch.from_numpy(toks[:72]).cuda(), [72], b)
    m.prefill(torch.from_numpy(toks[72:]).cuda(), [128], b)
    torch.cuda.synchronize()
    assert a.lengths == b.lengths == [200]
    close(bf16_to_np(a.k[:, :, :, :200]), bf16_to_np(b.k[:, :, :, :200]), max_abs=2e-2, rel_l2=2e-3,
          what="chunked prefill", bf16_out=True)


def test_commit_block_bitexact_with_canaries(env):
    dg, w, m = env
    kv = dg.KV(SHAPE, 2, 1024, fill=None)
    canary_k = synth.bf16_normal(tuple(kv.k.shape), 1, 60)
    canary_v = synth.bf16_normal(tuple(kv.v.shape), 1, 61)
    kv.k.copy_(np_bf16_dev(canary_k))
    kv.v.copy_(np_bf16_dev(canary_v))
    kv.set_lengths([L, 300])
    src_k = synth.bf16_normal((2, 2, 2, 256, 64), 2, 62)
    src_v = synth.bf16_normal((2, 2, 2, 256, 64), 2, 63)
    m.set_canvas_kv(np_bf16_dev(src_k), np_bf16_dev(src_v), 2)
    m.commit_block(None, kv, refresh=False)
    torch.cuda.synchronize()
    assert kv.lengths == [L + 256, 556]
    want_k = [[canary_k[l, b] for b in range(2)] for l in range(2)]
    ok = [[c.copy() for c in row] for row in want_k]
    for l in range(2):
        for b, Lb in enumerate([L, 300]):
            ck = [canary_k[l, b].astype(np.float64)]
            cv = [canary_v[l, b].astype(np.float64)]
            omodel.commit_block(ck, cv, [src_k[l, b]], [src_v[l, b]], Lb)
            assert np.array_equal(bf16_to_np(kv.k[l, b]), ck[0])
            assert np.array_equal(bf16_to_np(kv.v[l, b]), cv[0])


def test_commit_after_denoise_appends_the_step_kv(env):
    dg, w, m = env
    kv, k, v = _kv(dg, cap=L + 256)
    x = torch.from_numpy(synth.tokens(256, SHAPE.vocab, SEED, 70)).cuda()
    dbg = layer_debug(dg, m, SHAPE, 256, 2)
    cfg = dg.sampler_cfg(seed=1)
    m.denoise_step(x, kv, cfg, 0, dg.Stats(1, 256), debug={"canvas_k": dbg["canvas_k"], "canvas_v": dbg["canvas_v"]})
    m.commit_block(x, kv, refresh=False)
    torch.cuda.synchronize()
    assert torch.equal(kv.k[:, :, :, L:L + 256], dbg["canvas_k"])
    assert torch.equal(kv.v[:, :, :, L:L + 256], dbg["canvas_v"])
    assert torch.equal(kv.k[:, :, :, :L].cpu(), np_bf16_dev(k[:, :, :, :L]).cpu())
    # the appended K/V are the oracle's canvas K/V of these tokens (parity bar)
    fw = omodel.denoise_forward(w, SHAPE, x.cpu().numpy(), [k[l, 0] for l in range(2)],
                                [v[l, 0] for l in range(2)], L, with_head=False)
    for l in range(2):
        close(bf16_to_np(kv.k[l, 0, :, L:L + 256]), fw["canvas_k"][l], what=f"appended K layer {l}", bf16_out=True)


def test_causal_commit_reencodes_the_canvas(env):
    """DG_COMMIT_CAUSAL appends the causal prefill K/V of the canvas tokens: bit-identical to
    dg_prefill_causal of the same tokens (whose parity with the oracle the prefill tests check
    layer by layer), different from the bidirectional K/V of the same canvas, and for the first
    layer within the parity bar of the oracle's causal commit.  Deeper layers are not compared
    end to end here: over 256 rows a router near-tie in layer 0 moves a row's layer-1 input by
    O(1), and causal attention carries it to the later rows."""
    dg, w, m = env
    x = torch.from_numpy(synth.tokens(256, SHAPE.vocab, SEED, 73)).cuda()
    kv, k, v = _kv(dg, cap=L + 256)
    m.denoise_step(x, kv, dg.sampler_cfg(), 0, dg.Stats(1, 256))
    m.commit_block(x, kv, dg.COMMIT_CAUSAL)
    kv2, _, _ = _kv(dg, cap=L + 256)
    m.prefill(x, [256], kv2)
    kv3, _, _ = _kv(dg, cap=L + 256)
    m.denoise_step(x, kv3, dg.sampler_cfg(), 0, dg.Stats(1, 256))
    m.commit_block(x, kv3, dg.COMMIT_LAST)
    torch.cuda.synchronize()
    assert kv.lengths == [L + 256] and kv2.lengths == [L + 256]
    assert torch.equal(kv.k, kv2.k) and torch.equal(kv.v, kv2.v)
    assert not torch.equal(kv.k[:, :, :, L:L + 256], kv3.k[:, :, :, L:L + 256])
    ck = [k[l, 0].astype(np.float64).copy() for l in range(2)]
    cv = [v[l, 0].astype(np.float64).copy() for l in range(2)]
    assert omodel.commit_block_causal(w, SHAPE, x.cpu().numpy(), ck, cv, L) == L + 256
    close(bf16_to_np(kv.k[0, 0, :, L:L + 256]), ck[0][:, L:L + 256], what="causal K layer 0", bf16_out=True)
    close(bf16_to_np(kv.v[0, 0, :, L:L + 256]), cv[0][:, L:L + 256], what="causal V layer 0", bf16_out=True)


def test_refresh_recomputes_kv_of_final_canvas(env):
    dg, w, m = env
    kv, k, v = _kv(dg, cap=L + 256)
    x0 = torch.from_numpy(synth.tokens(256, SHAPE.vocab, SEED, 71)).cuda()
    x1 = torch.from_numpy(synth.tokens(256, SHAPE.vocab, SEED, 72)).cuda()
    m.denoise_step(x0, kv, dg.sampler_cfg(), 0, dg.Stats(1, 256))
    m.commit_block(x1, kv, refresh=True)
    kv2, _, _ = _kv(dg, cap=L + 256)
    m.denoise_step(x1, kv2, dg.sampler_cfg(), 0, dg.Stats(1, 256))
    m.commit_block(x1, kv2, refresh=False)
    torch.cuda.synchronize()
    assert torch.equal(kv.k, kv2.k) and torch.equal(kv.v, kv2.v)


def test_deterministic_bitwise(env):
    dg, w, m = env
    kv, _, _ = _kv(dg)
    x = torch.from_numpy(synth.tokens(256, SHAPE.vocab, SEED, 80)).cuda()
    cfg = dg.sampler_cfg(seed=77)
    outs = []
    for _ in range(2):
        s = dg.Stats(1, 256)
        m.denoise_step(x, kv, cfg, 5, s)
        torch.cuda.synchronize()
        outs.append([getattr(s, k).clone() for k in ("cand", "t_cand", "t_cur", "lse", "entropy")])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_peaked_head_stops_after_three_steps(env):
    """End-to-end through head + sampler with the peaked fixture: f and W_out chosen so that the
    logit of target_i is 50 and every other logit is 0 → exactly three steps."""
    dg, w, m = env
    d, V = SHAPE.d_model, SHAPE.vocab
    target = synth.tokens(256, V, SEED, 90)
    # f_i = e_{j(i)} * 1, W_out[v] = 50 * e_{j} for v == target of rows using basis j: use d >= 256
    # distinct basis vectors, one per row, and give row i's target that vector.
    W = np.zeros((V, d), np.float32)
    f = np.zeros((256, d), np.float32)
    # rows sharing a target share its basis vector
    basis = {}
    for i, t in enumerate(target):
        j = basis.setdefault(int(t), len(basis))
        f[i, j] = 1.0
        W[t, j] = 50.0
    m2 = dg.Model(SHAPE, {**w, "lm_head": W}, max_batch=1)
    try:
        kv, _, _ = _kv(dg)
        cfg = dg.sampler_cfg(seed=3)
        st = dg.Canvas(1, 256)
        m2.canvas_init(st, kv, cfg)
        stats = dg.Stats(1, 256)
        status = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
        fdev = np_bf16_dev(f)
        steps = 0
        for s in range(48):
            m2.denoise_step(st.tokens, kv, cfg, s, stats, flags=dg.DG_STEP_HEAD_ONLY, hidden_in=fdev)
            m2.sample_commit(st, stats, cfg, s, kv, status)
            torch.cuda.synchronize()
            steps += 1
            if dg.status_dict(status)[0]["stop"]:
                break
        assert steps == 3
        assert np.array_equal(st.tokens[0].cpu().numpy(), target)
        assert int(st.committed.sum()) == 48
    finally:
        m2.close()


def _pool(dg, n_slots=4, cap=L + 600, seed=90):
    kv = dg.KV(SHAPE, n_slots, cap)
    k, v = random_cache(SHAPE, L + 300, cap, seed, n_slots)
    load_cache(kv, k, v, [L, L + 300, L + 100, L + 7][:n_slots])
    return kv


def _run_slots(dg, m, kv, slots, cfg, steps=3):
    """canvas init, a few denoise + sampler steps and a commit on `slots` of a 4-slot pool."""
    st = dg.Canvas(kv.n_slots, 256)
    stats = dg.Stats(kv.n_slots, 256)
    status = torch.zeros((kv.n_slots, 8), dtype=torch.int32, device="cuda")
    m.canvas_init(st, kv, cfg, slots=slots)
    for s in range(steps):
        m.denoise_step(st.tokens, kv, cfg, s, stats, slots=slots)
        m.sample_commit(st, stats, cfg, s, kv, status, slots=slots)
    m.commit_block(st.tokens, kv, dg.COMMIT_REFRESH, slots=slots)
    torch.cuda.synchronize()
    return st, stats, status


def test_slot_mapped_calls_do_not_depend_on_call_order(env):
    """Requests run on slots of a larger pool (continuous batching): every per-slot output -- canvas
    state, row statistics, step status, the appended cache -- is bit-identical whether the call
    lists the slots as [3, 1] or [1, 3], and slots outside the call are left untouched."""
    dg, w, m = env
    cfg = dg.sampler_cfg(seed=2718, renoise_committed=False)
    kv_a, kv_b = _pool(dg), _pool(dg)
    k0, v0 = kv_a.k.clone(), kv_a.v.clone()
    a = _run_slots(dg, m, kv_a, [3, 1], cfg)
    b = _run_slots(dg, m, kv_b, [1, 3], cfg)
    assert kv_a.lengths == kv_b.lengths == [L, L + 300 + 256, L + 100, L + 7 + 256]
    for x in (1, 3):
        assert torch.equal(a[0].tokens[x], b[0].tokens[x]) and torch.equal(a[0].committed[x], b[0].committed[x])
        for k in ("cand", "t_cand", "t_cur", "lse", "entropy"):
            assert torch.equal(getattr(a[1], k)[x], getattr(b[1], k)[x]), k
        assert torch.equal(a[2][x], b[2][x])
    assert torch.equal(kv_a.k, kv_b.k) and torch.equal(kv_a.v, kv_b.v)
    for x in (0, 2):  # not in the call
        assert torch.equal(kv_a.k[:, x], k0[:, x]) and torch.equal(kv_a.v[:, x], v0[:, x])
        assert not a[0].tokens[x].any()


def test_commit_last_finds_each_slot_in_the_last_forward(env):
    """COMMIT_LAST takes each slot's canvas K/V from wherever the last forward pass held it: after
    a pass over slots [3, 1], committing [1] and then [3] (separately, the other way round) writes
    the same cache as committing [3, 1] at once, and a slot the pass did not cover is refused
    without writing anything."""
    dg, w, m = env
    cfg = dg.sampler_cfg(seed=4242)
    kv_a, kv_b = _pool(dg), _pool(dg)
    st = dg.Canvas(4, 256)
    stats = dg.Stats(4, 256)
    m.canvas_init(st, kv_a, cfg, slots=[3, 1])
    for kv in (kv_a, kv_b):
        m.denoise_step(st.tokens, kv, cfg, 0, stats, slots=[3, 1])
        if kv is kv_a:
            m.commit_block(st.tokens, kv, dg.COMMIT_LAST, slots=[3, 1])
        else:
            k0, v0, n0 = kv.k.clone(), kv.v.clone(), kv.lengths
            with pytest.raises(dg.DGError):
                m.commit_block(st.tokens, kv, dg.COMMIT_LAST, slots=[0])
            torch.cuda.synchronize()
            assert kv.lengths == n0 and torch.equal(kv.k, k0) and torch.equal(kv.v, v0)
            m.commit_block(st.tokens, kv, dg.COMMIT_LAST, slots=[1])
            m.commit_block(st.tokens, kv, dg.COMMIT_LAST, slots=[3])
    torch.cuda.synchronize()
    assert kv_a.lengths == kv_b.lengths == [L, L + 300 + 256, L + 100, L + 7 + 256]
    assert torch.equal(kv_a.k, kv_b.k) and torch.equal(kv_a.v, kv_b.v)


def test_slot_mapped_streams_follow_the_slot(env):
    """A request's random streams are keyed by its slot: canvas init on slots [2, 0] equals the
    oracle's draws for requests 2 and 0, and the sampler on identical statistics is bit-exact
    against the oracle run with b = slot."""
    dg, w, m = env
    kv = _pool(dg)
    cfg = dg.sampler_cfg(seed=31415, max_steps=6)
    oc = oracle_cfg(cfg)
    st = dg.Canvas(4, 256)
    m.canvas_init(st, kv, cfg, slots=[2, 0])
    torch.cuda.synchronize()
    lens = kv.lengths
    o_state = {}
    for x in (2, 0):
        want = osampler.canvas_init(cfg.seed, x, lens[x] + np.arange(256), SHAPE.vocab)
        assert np.array_equal(st.tokens[x].cpu().numpy(), want)
        o_state[x] = [want, np.zeros(256, bool), 0]
    stats = dg.Stats(4, 256)
    status = torch.zeros((4, 8), dtype=torch.int32, device="cuda")
    for s in range(cfg.max_steps):
        rs = {"cand": synth.tokens(1024, SHAPE.vocab, s, 11).reshape(4, 256),
              "t_cand": synth.uniform((4, 256), -4.0, 0.5, s, 12), "t_cur": synth.uniform((4, 256), -4.0, 0.5, s, 13),
              "lse": synth.uniform((4, 256), 0.0, 0.5, s, 14), "entropy": synth.uniform((4, 256), 0.0, 3.0, s, 15)}
        for k, v in rs.items():
            getattr(stats, k).copy_(torch.from_numpy(np.ascontiguousarray(v)))
        m.sample_commit(st, stats, cfg, s, kv, status, slots=[2, 0])
        torch.cuda.synchronize()
        got = dg.status_dict(status)
        for x in (2, 0):
            x_o, com, sr, ost = osampler.sample_commit({k: rs[k][x] for k in rs}, *o_state[x], oc, s, x,
                                                       lens[x] + np.arange(256), SHAPE.vocab)
            o_state[x] = [x_o, com, sr]
            assert np.array_equal(st.tokens[x].cpu().numpy(), x_o), (s, x)
            assert np.array_equal(st.committed[x].cpu().numpy().astype(bool), com), (s, x)
            for k in ("changed", "n_committed", "n_new", "n_renoised", "stable_run", "stop"):
                assert got[x][k] == ost[k], (s, x, k)
