"""GPU vs oracle parity at the low-to-medium batch shape: eight requests with ragged prefixes
denoised together at the full layer shape (d 2048, 16/8 heads, head_dim 128, 64 experts top-4,
F 768, shared FFN 4096), i.e. 2048 canvas rows and 8192 routes per step, the regime the pages
describe for one accelerator (DiffusionGemma docs, "Compensação com modelos tradicionais";
"Google's DiffusionGemma Atinge 1.000 Tokens por Segundo", fifth paragraph).

It takes the kernel variants that only this shape reaches: the long-range attention tasks
(32 query rows, 8 waves; one request over 8192 keys) next to short ragged prefixes, the
many-rows router, the separate route permutation (more than 2048 routes), the expert GEMMs with
160-row passes split over two work-groups, and the fused head at 2048 rows x vocab 65536.
Every request is checked layer by layer, teacher-forced; the route tables bit for bit against a
stable sort; skewed routings (an empty expert, an expert holding every row) on both the fused
(<= 2048 routes) and the separate permutation path."""
import dataclasses

import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import synth
from oracle import model as omodel
from oracle import sampler as osampler
from tests.gpu_common import (MARGIN, check_layers_teacher_forced, check_routes, close, layer_debug,
                              load_cache, need_gpu, np_bf16_dev, oracle_cfg, random_cache)

pytestmark = pytest.mark.gpu

SEED = 20260610
FULL1 = dataclasses.replace(synth.FULL, n_layers=1)
LENS = [9000, 0, 37, 300, 777, 1024, 64, 2000]   # one request past 8192 keys, the rest short


def _host(t):
    return t.detach().to("cpu", torch.float32).numpy()


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    w = synth.torch_model_weights(FULL1, "cuda", SEED + 40)
    host = {"layers": [{k: _host(v) for k, v in w["layers"][0].items()}]}
    m = dg.Model(FULL1, w, max_batch=8, max_prefill_rows=256)
    yield dg, w, host, m
    m.close()


def _step(dg, m, shape, lens, h, seed):
    """One denoise step (layers only) of len(lens) requests on hidden state h [B*256, d] over
    random bf16 prefix K/V; returns (debug dumps, host K, host V)."""
    B = len(lens)
    cap = max(lens) + 256
    kv = dg.KV(shape, B, cap)
    k, v = random_cache(shape, max(lens), cap, seed, B)
    load_cache(kv, k, v, lens)
    dbg = layer_debug(dg, m, shape, B * 256, shape.n_layers, batch=B)
    print(f"denoise step: {B} requests, prefixes {lens}", flush=True)
    m.denoise_step(None, kv, None, 0, None, flags=dg.DG_STEP_HIDDEN_IN | dg.DG_STEP_NO_HEAD,
                   hidden_in=torch.from_numpy(h).cuda(), debug=dbg)
    torch.cuda.synchronize()
    return dbg, k, v


def test_eight_ragged_requests_full_layer_shape(env):
    dg, w, host, m = env
    h = synth.hidden(8 * 256, FULL1.d_model, SEED, 41)
    dbg, k, v = _step(dg, m, FULL1, LENS, h, SEED + 42)
    check_routes(dbg, FULL1, 8 * 256, 0)
    for b, Lb in enumerate(LENS):
        check_layers_teacher_forced(host, FULL1, dbg, b, None, [k[0, b]], [v[0, b]], Lb,
                                    h0=h[b * 256:(b + 1) * 256])


def _skewed(dg, w, host, batch, seed):
    """A model whose router sends every row to expert 0, no row to expert 1 and about half the
    rows to expert 2: the hidden state carries a common direction u (and, on half the rows, a
    second direction u2) that the router rows of experts 0, 1 and 2 read with weight +c, -c and
    +c.  The other three picks of a row follow its random logits."""
    d = FULL1.d_model
    r = np.random.default_rng(seed)
    u = r.standard_normal(d)
    u /= np.linalg.norm(u)
    u2 = r.standard_normal(d)
    u2 -= (u2 @ u) * u
    u2 /= np.linalg.norm(u2)
    wr = host["layers"][0]["w_router"].copy()
    wr[0] = synth.bf16_round((0.5 * u).astype(np.float32))
    wr[1] = synth.bf16_round((-0.5 * u).astype(np.float32))
    wr[2] = synth.bf16_round((0.5 * u2).astype(np.float32))
    hl = {"layers": [dict(host["layers"][0], w_router=wr)]}
    wd = dict(w)
    wd["layers"] = [dict(w["layers"][0], w_router=np_bf16_dev(wr))]
    h = synth.hidden(batch * 256, d, seed, 43).astype(np.float64)
    h += 30.0 * u
    h[::2] += 30.0 * u2
    return wd, hl, h.astype(np.float32)


@pytest.mark.parametrize("batch", [2, 8])
def test_skewed_routing_route_tables_and_layer(env, batch):
    """2 requests (2048 routes: the gate/up GEMM ranks the routes itself) and 8 requests (8192
    routes: the separate permutation).  Expert 0 holds every row (several passes on both
    work-groups of each feature tile), expert 1 none; the route tables equal a stable sort and
    each request's layer matches the oracle teacher-forced."""
    dg, w, host, _ = env
    wd, hl, h = _skewed(dg, w, host, batch, SEED + 50 + batch)
    m = dg.Model(FULL1, wd, max_batch=batch, max_prefill_rows=256)
    try:
        lens = [40 + 13 * b for b in range(batch)]
        dbg, k, v = _step(dg, m, FULL1, lens, h, SEED + 60 + batch)
        check_routes(dbg, FULL1, batch * 256, 0)
        offs = dbg["route_offs"][0].cpu().numpy()
        counts = np.diff(offs)
        assert counts[0] == batch * 256 and counts[1] == 0, counts[:4]
        assert counts[2] > 0.4 * batch * 256, counts[:4]
        for b, Lb in enumerate(lens):
            check_layers_teacher_forced(hl, FULL1, dbg, b, None, [k[0, b]], [v[0, b]], Lb,
                                        h0=h[b * 256:(b + 1) * 256])
    finally:
        m.close()


@pytest.mark.parametrize("step", [5, 41])
def test_head_2048_rows_vocab_65536(env, step):
    """The fused head at 2048 rows (8 requests) on identical bf16 final states: row statistics
    and Gumbel-max candidates of 16 rows of every request, one in each residue class mod 16,
    against the oracle on the same rows."""
    dg, w, _, m = env
    d, V = FULL1.d_model, FULL1.vocab
    B = 8
    kv = dg.KV(FULL1, B, 256 + max(LENS))
    kv.set_lengths(LENS)
    f = synth.bf16_normal((B * 256, d), SEED, 70 + step)
    x = synth.tokens(B * 256, V, SEED, 71 + step).reshape(B, 256)
    cfg = dg.sampler_cfg(seed=777 + step)
    stats = dg.Stats(B, 256)
    m.denoise_step(torch.from_numpy(x).cuda(), kv, cfg, step, stats, flags=dg.DG_STEP_HEAD_ONLY,
                   hidden_in=np_bf16_dev(f))
    torch.cuda.synchronize()
    W = _host(w["lm_head"]).astype(np.float64)
    T = osampler.temperature(oracle_cfg(cfg), step)
    for b in range(B):
        rows = (np.arange(16) * 17 + 5 * b) % 256   # residues mod 16: all of 0..15
        assert sorted(rows % 16) == list(range(16))
        z = omodel.head_logits(f[b * 256 + rows], W)
        want = osampler.row_stats(z, x[b][rows], T, cfg.seed, b, LENS[b] + rows, step)
        ok = want["margin"] >= MARGIN
        assert np.array_equal(stats.cand.cpu().numpy()[b][rows][ok], want["cand"][ok]), b
        for k in ("t_cand", "t_cur", "lse"):
            close(getattr(stats, k).cpu().numpy()[b][rows][ok], want[k][ok], max_abs=1e-3, rel_l2=1e-5,
                  what=f"{k} request {b}")
        close(stats.entropy.cpu().numpy()[b][rows], want["entropy"], max_abs=1e-3, rel_l2=1e-4,
              what=f"entropy request {b}")
