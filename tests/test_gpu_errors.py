"""Failure handling through the C ABI, forced from the host: capacity and step-range errors leave
the device untouched, a non-finite logit is reported in the step status, and token ids outside
the vocabulary are clamped by the kernels and reported by dg_device_errors instead of being read
out of bounds.  Every kernel involved exits normally; nothing here faults the GPU."""
import ctypes

import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import synth
from tests.gpu_common import load_cache, need_gpu, random_cache

pytestmark = pytest.mark.gpu

SHAPE = synth.TINY
SEED = 20260610
L = 64


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    w = synth.model_weights(SHAPE, SEED)
    m = dg.Model(SHAPE, w, max_batch=2, max_prefill_rows=256)
    yield dg, w, m
    m.close()


def _kv(dg, cap, lens):
    kv = dg.KV(SHAPE, len(lens), cap)
    k, v = random_cache(SHAPE, max(lens), cap, SEED + 1, len(lens))
    load_cache(kv, k, v, lens)
    return kv


def test_commit_and_prefill_beyond_capacity_are_refused(env):
    """len + 256 > cap: dg_commit_block returns DG_ERR_CAPACITY and writes nothing; a prefill
    that would pass cap is refused the same way; the lengths stay where they were."""
    dg, _, m = env
    kv = _kv(dg, L + 200, [L])
    before_k, before_v = kv.k.clone(), kv.v.clone()
    tok = torch.zeros((1, 256), dtype=torch.int32, device="cuda")
    with pytest.raises(dg.DGError) as e:
        m.commit_block(tok, kv, dg.COMMIT_LAST)
    assert e.value.code == dg.DG_ERR_CAPACITY
    with pytest.raises(dg.DGError) as e:
        m.prefill(torch.zeros(201, dtype=torch.int32, device="cuda"), [201], kv)
    assert e.value.code == dg.DG_ERR_CAPACITY
    torch.cuda.synchronize()
    assert kv.lengths == [L]
    assert torch.equal(kv.k, before_k) and torch.equal(kv.v, before_v)


def test_step_beyond_the_schedule_is_refused(env):
    """A step outside [0, max_steps) is refused by the denoise step and by the sampler."""
    dg, _, m = env
    kv = _kv(dg, L + 256, [L])
    cfg = dg.sampler_cfg(seed=3, max_steps=48)
    st = dg.Canvas(1, 256)
    stats = dg.Stats(1, 256)
    status = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    m.canvas_init(st, kv, cfg)
    for bad in (48, -1):
        with pytest.raises(dg.DGError) as e:
            m.denoise_step(st.tokens, kv, cfg, bad, stats)
        assert e.value.code == dg.DG_ERR_ARG
        with pytest.raises(dg.DGError) as e:
            m.sample_commit(st, stats, cfg, bad, kv, status)
        assert e.value.code == dg.DG_ERR_ARG
    # the last step of the schedule is accepted and ends the canvas
    m.denoise_step(st.tokens, kv, cfg, 47, stats)
    m.sample_commit(st, stats, cfg, 47, kv, status)
    torch.cuda.synchronize()
    assert dg.status_dict(status)[0]["stop"] == 1


def test_nonfinite_logit_is_reported_in_the_status():
    """One LM-head row set to NaN makes every row's log-sum-exp NaN: the sampler reports
    nonfinite = 1 (a device-side condition, not an error code).  With finite weights it is 0."""
    dg = need_gpu()
    for poison in (False, True):
        w = synth.model_weights(SHAPE, SEED + 2)
        if poison:
            w["lm_head"] = w["lm_head"].copy()
            w["lm_head"][5] = np.nan
        m = dg.Model(SHAPE, w, max_batch=1, max_prefill_rows=256)
        try:
            kv = _kv(dg, L + 256, [L])
            cfg = dg.sampler_cfg(seed=4)
            st = dg.Canvas(1, 256)
            stats = dg.Stats(1, 256)
            status = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
            m.canvas_init(st, kv, cfg)
            m.denoise_step(st.tokens, kv, cfg, 0, stats)
            m.sample_commit(st, stats, cfg, 0, kv, status)
            torch.cuda.synchronize()
            s = dg.status_dict(status)[0]
            assert s["nonfinite"] == int(poison), s
            if poison:
                assert torch.isnan(stats.lse).all()
            assert int(st.tokens.min()) >= 0 and int(st.tokens.max()) < SHAPE.vocab
        finally:
            m.close()


def test_out_of_range_tokens_are_clamped_and_reported(env):
    """Ids outside [0, vocab) reach the kernels only past the binding's check (here through the
    raw ABI).  The embedding and the head clamp them, the call succeeds, and dg_device_errors
    reports DG_DEVERR_TOKEN_RANGE once, then reads clear.  In-range calls leave it clear."""
    dg, _, m = env
    assert m.device_errors() == 0
    kv = _kv(dg, 8 + 256, [0])
    bad = torch.tensor([3, SHAPE.vocab + 5, -1, 7, 2 ** 31 - 1, 0, 1, 2], dtype=torch.int32, device="cuda")
    n = (ctypes.c_int32 * 1)(8)
    rc = dg._lib.dg_prefill_causal(m.ctx, dg._ptr(bad), n, 1, ctypes.byref(kv.c), dg._stream())
    assert rc == dg.DG_OK
    kv.len[0] = 8
    assert m.device_errors() == dg.DG_DEVERR_TOKEN_RANGE
    assert m.device_errors() == 0
    # the binding refuses the same ids before anything is enqueued
    with pytest.raises(ValueError):
        m.prefill(bad, [8], kv)
    # a canvas token out of range: clamped by the embedding and by the head's current-token read
    cfg = dg.sampler_cfg(seed=5)
    stats = dg.Stats(1, 256)
    canvas = torch.from_numpy(synth.tokens(256, SHAPE.vocab, SEED, 9).reshape(1, 256)).cuda()
    m.denoise_step(canvas, kv, cfg, 0, stats)
    assert m.device_errors() == 0
    canvas[0, 17] = SHAPE.vocab
    canvas[0, 200] = -3
    m.denoise_step(canvas, kv, cfg, 0, stats)
    assert m.device_errors() == dg.DG_DEVERR_TOKEN_RANGE
    assert torch.isfinite(stats.lse).all()
