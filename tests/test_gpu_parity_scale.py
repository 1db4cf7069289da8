"""GPU vs oracle parity beyond the single small canvas: the full layer shape (d 2048, 16/8 heads,
head_dim 128, 64 experts top-4, F 768, with and without the shared FFN 4096) at its real prefix
lengths, the vocab-65536 fused head, batched requests with ragged prefixes, and block-by-block
generation with commits.  Every call goes through the C ABI."""
import dataclasses

import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import synth
from oracle import fp8 as ofp8
from oracle import model as omodel
from oracle import sampler as osampler
from tests.gpu_common import (MARGIN, bf16_to_np, check_layer, check_layers_teacher_forced, close,
                              layer_debug, load_cache, need_gpu, np_bf16_dev, oracle_cfg, random_cache)

pytestmark = pytest.mark.gpu

SEED = 20260610
FULL1 = dataclasses.replace(synth.FULL, n_layers=1)   # one layer of the 12-layer model + head


def _host(t):
    return t.detach().to("cpu", torch.float32).numpy()


@pytest.fixture(scope="module")
def full_env():
    dg = need_gpu()
    w = synth.torch_model_weights(FULL1, "cuda", SEED)
    m = dg.Model(FULL1, w, max_batch=1, max_prefill_rows=256)
    host = {"layers": [{k: _host(v) for k, v in w["layers"][0].items()}]}
    yield dg, w, m, host
    m.close()


@pytest.mark.parametrize("prefix", [2048, 4096, 777, 8192])
def test_full_shape_layer_with_shared_ffn(full_env, prefix):
    """One layer at the full shape with the shared FFN: attention over `prefix` cached keys plus
    the canvas, routed experts, shared FFN; all 256 rows against the oracle.  The prefixes take
    every canvas attention shape: 16-row tasks with 4 waves (777) or 8 waves (2048, 4096), and
    the long-range variant with 32-row tasks (8192)."""
    dg, w, m, host = full_env
    check_layer(dg, m, host, FULL1, prefix, SEED + prefix, prefix + 256)


def test_long_range_attention_moving_reference(full_env):
    """Scores that climb inside every key range, so that the pipelined kernel's exponent
    reference moves during a split: the 9000 cached keys are scaled by a sawtooth from 0.05 to 3
    over each 1024 keys.  Each split then starts low and its running maximum passes the
    reference by more than the lazy-rescale margin (8 in log2 units) about 1.5 times per query
    (emulated on the host: maxima up to ~19 log2 units); every such move rescales O and the row
    sum and shifts the already computed scores of the next half to the new offset.  All 256 rows
    against the oracle, as the other full-shape layers."""
    dg, w, m, host = full_env
    Lp, seed = 9000, SEED + 9000
    k, v = random_cache(FULL1, Lp, Lp + 256, seed)
    ramp = 0.05 + 2.95 * ((np.arange(Lp) % 1024) / 1023.0)
    k[:, :, :, :Lp] = synth.bf16_round(k[:, :, :, :Lp] * ramp[None, None, None, :, None].astype(np.float32))
    check_layer(dg, m, host, FULL1, Lp, seed, Lp + 256, cache=(k, v))


def test_full_shape_layer_without_shared_ffn(full_env):
    """The single-layer shape of the mid configuration: no shared FFN, prefix 4096."""
    dg, w, _, host = full_env
    shape = dataclasses.replace(synth.MID_LAYER, vocab=FULL1.vocab)
    lw = {k: v for k, v in w["layers"][0].items() if not k.startswith("ws_")}
    m = dg.Model(shape, {**w, "layers": [lw]}, max_batch=1, max_prefill_rows=256)
    try:
        hl = {"layers": [{k: v for k, v in host["layers"][0].items() if not k.startswith("ws_")}]}
        check_layer(dg, m, hl, shape, 4096, SEED + 1, 4096 + 256)
    finally:
        m.close()


def test_full_shape_layer_fp8_experts(full_env):
    """The full layer shape with the routed experts as E4M3 bytes (per-channel scales) and the
    shared FFN in bf16, prefix 2048, against the oracle layer whose experts are its own E4M3
    round trip of the same weights."""
    dg, w, _, host = full_env
    shape = dataclasses.replace(FULL1, expert_fp8=True)
    m = dg.Model(shape, w, max_batch=1, max_prefill_rows=256)
    try:
        hl = {"layers": [ofp8.dequantize_experts(host["layers"][0])]}
        check_layer(dg, m, hl, shape, 2048, SEED + 77, 2048 + 256)
    finally:
        m.close()


@pytest.mark.parametrize("step", [0, 30])
def test_full_vocab_head(full_env, step):
    """Fused head at vocab 65536 on identical bf16 final states: logits, row statistics and
    Gumbel-max candidates of all 256 rows against the oracle."""
    dg, w, m, _ = full_env
    d, V = FULL1.d_model, FULL1.vocab
    L = 2048
    kv = dg.KV(FULL1, 1, L + 256)
    kv.set_lengths([L])
    f = synth.bf16_normal((256, d), SEED, 200 + step)
    x = synth.tokens(256, V, SEED, 201 + step)
    cfg = dg.sampler_cfg(seed=31337 + step)
    stats = dg.Stats(1, 256)
    logits = torch.zeros((256, V), dtype=torch.float32, device="cuda")
    m.denoise_step(torch.from_numpy(x).cuda(), kv, cfg, step, stats, flags=dg.DG_STEP_HEAD_ONLY,
                   hidden_in=np_bf16_dev(f), debug={"logits": logits})
    torch.cuda.synchronize()
    rows = np.arange(256)  # every row of the canvas
    W = _host(w["lm_head"]).astype(np.float64)
    z = omodel.head_logits(f[rows], W)
    close(logits[torch.from_numpy(rows).cuda()].cpu().numpy(), z, what="logits V=65536")
    oc = oracle_cfg(cfg)
    want = osampler.row_stats(z, x[rows], osampler.temperature(oc, step), cfg.seed, 0, L + rows, step)
    ok = want["margin"] >= MARGIN
    assert ok.mean() > 0.9
    assert np.array_equal(stats.cand.cpu().numpy()[0][rows][ok], want["cand"][ok])
    for k in ("t_cand", "t_cur", "lse"):
        close(getattr(stats, k).cpu().numpy()[0][rows][ok], want[k][ok], max_abs=1e-3, rel_l2=1e-5, what=k)
    close(stats.entropy.cpu().numpy()[0][rows], want["entropy"], max_abs=1e-3, rel_l2=1e-4, what="entropy")


# ------------------------------------------------------------------------------- small shape
SHAPE = synth.TINY


@pytest.fixture(scope="module")
def tiny_env():
    dg = need_gpu()
    w = synth.model_weights(SHAPE, SEED)
    m = dg.Model(SHAPE, w, max_batch=4, max_prefill_rows=512)
    yield dg, w, m
    m.close()


def test_batched_ragged_step(tiny_env):
    """Four requests with ragged prefixes (64, 37, 1000 and 0 keys) in one denoise step.  Cache
    slots past each request's length hold huge values the kernels must never read.  Each
    request's layers are checked teacher-forced against the oracle; the head is checked on the
    GPU's own final state (logits within the bar, candidates wherever the oracle margin is
    clear)."""
    dg, w, m = tiny_env
    lens = [64, 37, 1000, 0]
    B, cap = len(lens), 1300
    kv = dg.KV(SHAPE, B, cap)
    k, v = random_cache(SHAPE, max(lens), cap, SEED + 9, B)
    for b, Lb in enumerate(lens):
        k[:, b, :, Lb:] = 1e4
        v[:, b, :, Lb:] = -1e4
    load_cache(kv, k, v, lens)
    x = synth.tokens(B * 256, SHAPE.vocab, SEED, 300).reshape(B, 256)
    cfg = dg.sampler_cfg(seed=8)
    stats = dg.Stats(B, 256)
    dbg = layer_debug(dg, m, SHAPE, B * 256, SHAPE.n_layers, batch=B)
    dbg["logits"] = torch.zeros((B * 256, SHAPE.vocab), dtype=torch.float32, device="cuda")
    m.denoise_step(torch.from_numpy(x).cuda(), kv, cfg, 2, stats, debug=dbg)
    torch.cuda.synchronize()
    oc = oracle_cfg(cfg)
    T = osampler.temperature(oc, 2)
    for b, Lb in enumerate(lens):
        check_layers_teacher_forced(w, SHAPE, dbg, b, x[b], [k[l, b] for l in range(SHAPE.n_layers)],
                                    [v[l, b] for l in range(SHAPE.n_layers)], Lb)
        sl = slice(b * 256, (b + 1) * 256)
        h = dbg["hidden_out"][sl].cpu().numpy()
        f = omodel.to_bf16(omodel.rmsnorm(h, w["final_norm"], SHAPE.rms_eps))
        z = omodel.head_logits(f, w["lm_head"])
        close(dbg["logits"][sl].cpu().numpy(), z, what=f"logits request {b}")
        want = osampler.row_stats(z, x[b], T, cfg.seed, b, Lb + np.arange(256), 2)
        close(stats.lse.cpu().numpy()[b], want["lse"], max_abs=2e-3, rel_l2=1e-4, what=f"lse request {b}")
        clear = want["margin"] >= 1e-2
        assert clear.mean() > 0.9
        assert np.array_equal(stats.cand.cpu().numpy()[b][clear], want["cand"][clear]), b


@pytest.mark.parametrize("renoise", [1, 0])
def test_block_autoregressive_generation(tiny_env, renoise):
    """Prefill two ragged prompts, then denoise and commit three canvases for each.
    * Commit semantics, bit-exact: every committed block equals the canvas K/V that a forward
      pass over the block's final tokens produces, with the cache as it stood when the block
      started (re-run here on the same batch).
    * Parity: that forward pass, layer by layer and teacher-forced, against the oracle over the
      GPU's cache (prompt + earlier committed blocks)."""
    dg, w, m = tiny_env
    lens = [64, 100]
    n_blocks = 3
    cap = max(lens) + n_blocks * 256
    kv = dg.KV(SHAPE, 2, cap)
    prefix = np.concatenate([synth.tokens(n, SHAPE.vocab, SEED, 400 + i) for i, n in enumerate(lens)])
    cfg = dg.sampler_cfg(seed=2024 + renoise, renoise_committed=renoise)
    blocks = m.generate(torch.from_numpy(prefix).cuda(), lens, n_blocks, cfg, kv)
    torch.cuda.synchronize()
    final = [n + n_blocks * 256 for n in lens]
    assert kv.lengths == final
    K = [[bf16_to_np(kv.k[l, b]) for b in range(2)] for l in range(SHAPE.n_layers)]
    V = [[bf16_to_np(kv.v[l, b]) for b in range(2)] for l in range(SHAPE.n_layers)]
    for j in range(n_blocks):
        starts = [n + 256 * j for n in lens]
        toks = blocks[j]
        assert int(toks.min()) >= 0 and int(toks.max()) < SHAPE.vocab
        kv.set_lengths(starts)
        dbg = layer_debug(dg, m, SHAPE, 512, SHAPE.n_layers, batch=2)
        m.denoise_step(toks, kv, None, 0, None, flags=dg.DG_STEP_NO_HEAD, debug=dbg)
        torch.cuda.synchronize()
        kv.set_lengths(final)
        for b, st in enumerate(starts):
            for l in range(SHAPE.n_layers):
                assert torch.equal(kv.k[l, b, :, st:st + 256], dbg["canvas_k"][l, b]), (j, b, l)
                assert torch.equal(kv.v[l, b, :, st:st + 256], dbg["canvas_v"][l, b]), (j, b, l)
            check_layers_teacher_forced(w, SHAPE, dbg, b, toks[b].cpu().numpy(),
                                        [K[l][b] for l in range(SHAPE.n_layers)],
                                        [V[l][b] for l in range(SHAPE.n_layers)], st)
    assert not torch.equal(blocks[0], blocks[1])


def test_layer_narrower_than_a_work_group_with_split_projection():
    """d = 1024 (fewer row elements than the 512-lane norm/router work-group covers) with a
    2048-wide attention output, so the O-projection is split into slices that the norm adds:
    lanes past the row width must stay out of the sum (regression: they once summed slices
    that were never loaded and turned every router logit into NaN)."""
    dg = need_gpu()
    shape = synth.ModelShape(n_layers=1, d_model=1024, n_q_heads=16, n_kv_heads=8, head_dim=128,
                             n_experts=8, top_k=2, d_ff_expert=256, d_ff_shared=0, vocab=1024)
    w = synth.model_weights(shape, SEED + 5)
    m = dg.Model(shape, w, max_batch=1)
    try:
        check_layer(dg, m, w, shape, 300, SEED + 6, 300 + 256)
    finally:
        m.close()


_LONG_PREFILL = {}


@pytest.mark.parametrize("chunk", [512, 2048])
def test_long_causal_prefill(chunk):
    """Causal prefill of 8300 tokens in chunks of 512 or 2048 rows: the later chunks attend to
    more than 8192 keys (the long-range attention variant, causal), and 2048-row chunks take the
    many-rows-per-group router and the large GEMM tiles; the cache equals the oracle's prefill.
    Every expert is active (top-k = E) so that no router near-tie can swap experts for a row
    and move the next layer's inputs: the comparison is end to end over both layers."""
    dg = need_gpu()
    shape = dataclasses.replace(SHAPE, n_experts=4, top_k=4)
    w = synth.model_weights(shape, SEED + 7)
    m = dg.Model(shape, w, max_batch=1, max_prefill_rows=chunk)
    try:
        n = 8300
        toks = synth.tokens(n, shape.vocab, SEED, 500)
        kv = dg.KV(shape, 1, n + 256)
        m.prefill(torch.from_numpy(toks).cuda(), [n], kv)
        torch.cuda.synchronize()
        assert kv.lengths == [n]
        if not _LONG_PREFILL:
            ck = [np.zeros((shape.n_kv_heads, n + 256, shape.head_dim)) for _ in range(shape.n_layers)]
            cv = [np.zeros((shape.n_kv_heads, n + 256, shape.head_dim)) for _ in range(shape.n_layers)]
            omodel.prefill(w, shape, toks, ck, cv, 0)
            _LONG_PREFILL["kv"] = (ck, cv)
        ck, cv = _LONG_PREFILL["kv"]
        for l in range(shape.n_layers):
            close(bf16_to_np(kv.k[l, 0, :, :n]), ck[l][:, :n], what=f"prefill K layer {l}", bf16_out=True)
            close(bf16_to_np(kv.v[l, 0, :, :n]), cv[l][:, :n], what=f"prefill V layer {l}", bf16_out=True)
    finally:
        m.close()


@pytest.mark.parametrize("sawtooth", [False, True])
def test_causal_prefill_chunk_over_a_long_cache(sawtooth):
    """A 2048-row causal prefill chunk over 8000 cached positions (N(0,1) bf16 K/V) at head dim
    128: its attention runs on the long-range pipelined kernel, causal, with per-request splits
    (a split past a work-group's last query is empty).  Two layers with every expert active
    (top-k = E, so no router tie can move a row); layer 1's K/V of the chunk depend on layer 0's
    attention and must equal the oracle's prefill of the chunk over the same cache.  With
    `sawtooth` the cached keys are scaled by 0.05 -> 3 over each 1024 positions, so that the
    exponent reference of the causal kernel moves inside its splits as well."""
    dg = need_gpu()
    shape = dataclasses.replace(synth.MID_LAYER, n_layers=2, n_experts=4, top_k=4, vocab=1024)
    w = synth.model_weights(shape, SEED + 9)
    L0, n = 8000, 2048
    m = dg.Model(shape, w, max_batch=1, max_prefill_rows=n)
    try:
        k, v = random_cache(shape, L0, L0 + n + 256, SEED + 10)
        if sawtooth:
            ramp = (0.05 + 2.95 * ((np.arange(L0) % 1024) / 1023.0)).astype(np.float32)
            k[:, :, :, :L0] = synth.bf16_round(k[:, :, :, :L0] * ramp[None, None, None, :, None])
        kv = dg.KV(shape, 1, L0 + n + 256, fill=None)
        load_cache(kv, k, v, [L0])
        toks = synth.tokens(n, shape.vocab, SEED, 501)
        m.prefill(torch.from_numpy(toks).cuda(), [n], kv)
        torch.cuda.synchronize()
        assert kv.lengths == [L0 + n]
        ck = [k[l, 0].astype(np.float64) for l in range(shape.n_layers)]
        cv = [v[l, 0].astype(np.float64) for l in range(shape.n_layers)]
        omodel.prefill(w, shape, toks, ck, cv, L0)
        for l in range(shape.n_layers):
            close(bf16_to_np(kv.k[l, 0, :, L0:L0 + n]), ck[l][:, L0:L0 + n], what=f"chunk K layer {l}", bf16_out=True)
            close(bf16_to_np(kv.v[l, 0, :, L0:L0 + n]), cv[l][:, L0:L0 + n], what=f"chunk V layer {l}", bf16_out=True)
        # the cached positions before the chunk are untouched
        assert torch.equal(kv.k[:, 0, :, :L0].float().cpu(), torch.from_numpy(k[:, 0, :, :L0]))
    finally:
        m.close()


def test_short_causal_chunk_over_a_long_cache():
    """A 70-row causal prefill chunk over 8200 cached positions at head dim 128: the long-range
    kernel, causal, with 3 row blocks of 32 (the last one 6 rows) per head, so two of the eight
    waves hold no query task, and the causal mask cuts the last key half block of every wave.
    Two layers with every expert active; the chunk's K/V of both layers against the oracle."""
    dg = need_gpu()
    shape = dataclasses.replace(synth.MID_LAYER, n_layers=2, n_experts=4, top_k=4, vocab=1024)
    w = synth.model_weights(shape, SEED + 13)
    L0, n = 8200, 70
    m = dg.Model(shape, w, max_batch=1, max_prefill_rows=256)
    try:
        k, v = random_cache(shape, L0, L0 + n + 256, SEED + 14)
        kv = dg.KV(shape, 1, L0 + n + 256, fill=None)
        load_cache(kv, k, v, [L0])
        toks = synth.tokens(n, shape.vocab, SEED, 502)
        m.prefill(torch.from_numpy(toks).cuda(), [n], kv)
        torch.cuda.synchronize()
        assert kv.lengths == [L0 + n]
        ck = [k[l, 0].astype(np.float64) for l in range(shape.n_layers)]
        cv = [v[l, 0].astype(np.float64) for l in range(shape.n_layers)]
        omodel.prefill(w, shape, toks, ck, cv, L0)
        for l in range(shape.n_layers):
            close(bf16_to_np(kv.k[l, 0, :, L0:L0 + n]), ck[l][:, L0:L0 + n], what=f"chunk K layer {l}", bf16_out=True)
            close(bf16_to_np(kv.v[l, 0, :, L0:L0 + n]), cv[l][:, L0:L0 + n], what=f"chunk V layer {l}", bf16_out=True)
    finally:
        m.close()


def test_prefill_2048_rows_on_the_large_tile_gemms():
    """A 2048-row causal prefill at width 2048 with the shared FFN 4096: the QKV projection (RoPE
    epilogue), the split O-projection, the shared gate/up pair and the split shared down
    projection all take the large-tile direct-to-LDS GEMMs (2048 rows give them a full chip of
    tiles).  Both layers' caches are compared with the oracle's prefill; all experts are active
    (top-k = E) so no router near-tie can move the second layer's inputs."""
    dg = need_gpu()
    shape = synth.ModelShape(n_layers=2, d_model=2048, n_q_heads=16, n_kv_heads=8, head_dim=128,
                             n_experts=4, top_k=4, d_ff_expert=256, d_ff_shared=4096, vocab=1024)
    w = synth.model_weights(shape, SEED + 9)
    m = dg.Model(shape, w, max_batch=1, max_prefill_rows=2048)
    try:
        n = 2048
        toks = synth.tokens(n, shape.vocab, SEED, 900)
        kv = dg.KV(shape, 1, n + 256)
        print("prefill 2048 rows, d 2048, shared FFN 4096", flush=True)
        m.prefill(torch.from_numpy(toks).cuda(), [n], kv)
        torch.cuda.synchronize()
        ck = [np.zeros((shape.n_kv_heads, n + 256, shape.head_dim)) for _ in range(shape.n_layers)]
        cv = [np.zeros((shape.n_kv_heads, n + 256, shape.head_dim)) for _ in range(shape.n_layers)]
        omodel.prefill(w, shape, toks, ck, cv, 0)
        for l in range(shape.n_layers):
            close(bf16_to_np(kv.k[l, 0, :, :n]), ck[l][:, :n], what=f"prefill K layer {l}", bf16_out=True)
            close(bf16_to_np(kv.v[l, 0, :, :n]), cv[l][:, :n], what=f"prefill V layer {l}", bf16_out=True)
    finally:
        m.close()
