"""The continuous batcher on the GPU (small configuration: 2 layers, d 256, 4/2 heads, D 64,
8 experts top-2, V 1024).  Five requests with ragged prompts (one empty) and one to three blocks
share a pool of three cache slots, at most two canvases per call; the first arrives two steps
before the others, so requests join and leave while others are mid-canvas and calls mix step
counters.

Checked:
* every sampler step of every canvas, bit-exact against the oracle's sampler run on the GPU's
  own row statistics with the request's slot, step and positions (teacher-forced), and every
  canvas start against the oracle's uniform draws;
* each request's prompt K/V, bit-identical to a prefill of that prompt alone on the same slot;
* each committed block's K/V against a forward pass of that block alone over the same cache
  prefix (layer 0 within the parity bar everywhere; all layers within it on almost every row --
  the batched and the lone pass add in different orders, which can flip a near-tied expert);
* with the causal commit, each request's whole cache bit-identical to a lone replay (prefill of
  the prompt, then of each block), which no other request can influence."""
import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import synth
from oracle import sampler as osampler
from tests.gpu_common import BF16_ULP, MAX_ABS, REL_L2, close, layer_debug, need_gpu, oracle_cfg

pytestmark = pytest.mark.gpu

SHAPE = synth.TINY
SEED = 20261203
C = 256
REQS = [(40, 2), (173, 1), (0, 2), (260, 1), (90, 1)]  # (prompt length, blocks)
CAP = 260 + 2 * C + 16
N_SLOTS = 3


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    from block_discrete_diffusion_amd import scheduler
    w = synth.model_weights(SHAPE, SEED)
    m = dg.Model(SHAPE, w, max_batch=3, max_prefill_rows=512)
    yield dg, scheduler, m
    m.close()


def _prompts():
    return [synth.tokens(n, SHAPE.vocab, SEED, 100 + i) if n else np.zeros(0, np.int32)
            for i, (n, _) in enumerate(REQS)]


class Checker:
    """Trace hook: oracle sampler checks per step, and a cache snapshot of each finished request."""

    def __init__(self, dg, cfg):
        self.dg, self.cfg, self.oc = dg, cfg, oracle_cfg(cfg)
        self.b = None
        self.prev = {}
        self.snap = {}
        self.n_steps = 0
        self.n_starts = 0
        self.mixed_steps = 0
        self.commit_modes = set()

    def __call__(self, ev, info):
        b = self.b
        if ev == "denoise":
            torch.cuda.synchronize()
            self.prev = {}
            if len(set(info["steps"])) > 1:
                self.mixed_steps += 1
            for s, step in zip(info["slots"], info["steps"]):
                tok = b.state.tokens[s].cpu().numpy()
                com = b.state.committed[s].cpu().numpy().astype(bool)
                sr = int(b.state.stable_run[s])
                Lc = b.kv.len[s]
                if step == 0:
                    want = osampler.canvas_init(self.cfg.seed, s, Lc + np.arange(C), SHAPE.vocab)
                    assert np.array_equal(tok, want) and not com.any() and sr == 0, (s, Lc)
                    self.n_starts += 1
                stats = {k: getattr(b.stats, k)[s].cpu().numpy()
                         for k in ("cand", "t_cand", "t_cur", "lse", "entropy")}
                self.prev[s] = (tok, com, sr, step, Lc, stats)
        elif ev == "sample":
            for s in info["slots"]:
                tok, com, sr, step, Lc, stats = self.prev[s]
                x, c, sr2, ost = osampler.sample_commit(stats, tok, com, sr, self.oc, step, s,
                                                        Lc + np.arange(C), SHAPE.vocab)
                assert np.array_equal(b.state.tokens[s].cpu().numpy(), x), (s, step)
                assert np.array_equal(b.state.committed[s].cpu().numpy().astype(bool), c), (s, step)
                got = info["status"][s]
                for k in ("changed", "n_committed", "n_new", "n_renoised", "stable_run", "stop"):
                    assert got[k] == ost[k], (s, step, k)
                self.n_steps += 1
        elif ev == "commit":
            self.commit_modes.add(info["mode"])
        elif ev == "finish":
            s = info["slot"]
            n = b.kv.len[s]
            torch.cuda.synchronize()
            self.snap[info["rid"]] = (s, n, b.kv.k[:, s, :, :n].clone(), b.kv.v[:, s, :, :n].clone())


def _serve(dg, scheduler, m, cfg, commit):
    kv = dg.KV(SHAPE, N_SLOTS, CAP)
    chk = Checker(dg, cfg)
    b = scheduler.ContinuousBatcher(m, kv, cfg, max_active=2, commit=commit, trace=chk)
    chk.b = b
    prompts = _prompts()
    print(f"serving {len(REQS)} requests, commit mode {commit}", flush=True)
    # the first request arrives alone; the others two steps later, so the live canvases of one
    # call sit at different steps from then on
    rids = [b.submit(prompts[0], REQS[0][1])]
    b.step()
    b.step()
    rids += [b.submit(p, n) for p, (_, n) in zip(prompts[1:], REQS[1:])]
    done = b.run(max_iterations=2000)
    torch.cuda.synchronize()
    assert sorted(done) == rids and b.idle()
    assert chk.n_starts == sum(n for _, n in REQS) and chk.mixed_steps > 0
    return b, done, chk, prompts, rids


def _lone_prefill(dg, m, slot, chunks):
    """A fresh pool; prefill `chunks` (token arrays) one after another on `slot` alone."""
    kv = dg.KV(SHAPE, N_SLOTS, CAP)
    for t in chunks:
        if len(t):
            m.prefill(torch.from_numpy(np.ascontiguousarray(t, np.int32)).cuda(), [len(t)], kv, slots=[slot])
    torch.cuda.synchronize()
    return kv


@pytest.mark.parametrize("schedule", ["stable_stop", "max_steps_stop"])
def test_continuous_batcher_matches_the_oracle_sampler_and_lone_passes(env, schedule):
    dg, scheduler, m = env
    if schedule == "stable_stop":  # canvases stop unchanged: COMMIT_LAST of the batched pass
        cfg = dg.sampler_cfg(seed=515, max_steps=12, commit_per_step=64, renoise_committed=False)
    else:  # canvases still change at the last step: re-run before the commit
        cfg = dg.sampler_cfg(seed=516, max_steps=5)
    b, done, chk, prompts, rids = _serve(dg, scheduler, m, cfg, dg.COMMIT_LAST)
    assert chk.n_steps == sum(sum(r.steps_per_block) for r in done.values())
    want_modes = {dg.COMMIT_LAST} if schedule == "stable_stop" else {dg.COMMIT_REFRESH}
    assert want_modes <= chk.commit_modes
    for rid, p, (n_p, n_b) in zip(rids, prompts, REQS):
        r = done[rid]
        s, n, k, v = chk.snap[rid]
        assert s == r.slot and n == n_p + n_b * C
        # the prompt: bit-identical to a lone prefill on the same slot
        kv1 = _lone_prefill(dg, m, s, [p])
        assert torch.equal(kv1.k[:, s, :, :n_p], k[:, :, :n_p]) and torch.equal(kv1.v[:, s, :, :n_p], v[:, :, :n_p])
        # each block: a lone bidirectional pass over the same prefix
        kv1.k[:, s, :, :n] = k
        kv1.v[:, s, :, :n] = v
        for j, blk in enumerate(r.blocks):
            Lj = n_p + j * C
            kv1.len[s] = Lj
            canvas = torch.zeros((N_SLOTS, C), dtype=torch.int32, device="cuda")
            canvas[s] = blk
            dbg = layer_debug(dg, m, SHAPE, C, SHAPE.n_layers)
            m.denoise_step(canvas, kv1, None, 0, None, flags=dg.DG_STEP_NO_HEAD,
                           debug={"canvas_k": dbg["canvas_k"], "canvas_v": dbg["canvas_v"]}, slots=[s])
            torch.cuda.synchronize()
            for name, got, ref in (("K", k, dbg["canvas_k"]), ("V", v, dbg["canvas_v"])):
                g = got[:, :, Lj:Lj + C].float().cpu().numpy()
                w = ref[:, 0].float().cpu().numpy()
                close(g[0], w[0], what=f"request {rid} block {j} layer-0 {name}", bf16_out=True)
                err = np.abs(g - w).max(axis=-1)  # per (layer, head, position)
                bound = MAX_ABS + BF16_ULP * np.abs(w).max(axis=-1)
                assert (err <= bound).mean() >= 0.97, (rid, j, name, float((err <= bound).mean()))
                rl = np.linalg.norm(g - w) / np.linalg.norm(w)
                assert rl <= REL_L2, (rid, j, name, rl)


def test_continuous_batcher_causal_commit_is_independent_of_the_batch(env):
    dg, scheduler, m = env
    cfg = dg.sampler_cfg(seed=517, max_steps=4)
    b, done, chk, prompts, rids = _serve(dg, scheduler, m, cfg, dg.COMMIT_CAUSAL)
    for rid, p, (n_p, n_b) in zip(rids, prompts, REQS):
        r = done[rid]
        s, n, k, v = chk.snap[rid]
        assert n == n_p + n_b * C
        kv1 = _lone_prefill(dg, m, s, [p] + [blk.cpu().numpy() for blk in r.blocks])
        assert kv1.len[s] == n
        assert torch.equal(kv1.k[:, s, :, :n], k) and torch.equal(kv1.v[:, s, :, :n], v), rid
