"""The allocation-free head call (dg_denoise_head_static) against dg_denoise_step with
DG_STEP_HEAD_ONLY: same inputs, bit-identical row statistics, on two calls in a row (the second
with fewer rows, so stale scratch from the first must not leak into it), a slot-mapped call (its
canvas tokens are gathered into the static scratch), and the refusal of a call whose scratch
would exceed the fixed array.  Every call goes through the C ABI."""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import synth
from tests.gpu_common import need_gpu, np_bf16_dev

pytestmark = pytest.mark.gpu

SEED = 20260610
SHAPE = dataclasses.replace(synth.TINY, n_layers=1, vocab=16384)
STATS = ("cand", "t_cand", "t_cur", "lse", "entropy")


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    w = synth.model_weights(SHAPE, SEED)
    m = dg.Model(SHAPE, w, max_batch=8, max_prefill_rows=256)
    yield dg, m
    m.close()


def _params(dg, step, hidden):
    return dg.StepParams(int(step), dg.DG_STEP_HEAD_ONLY, dg._ptr(hidden), None, None)


def _call_static(dg, m, canvas, view, cfg, params, stats):
    return dg._lib.dg_denoise_head_static(m.ctx, dg._ptr(canvas), ctypes.byref(view.c), ctypes.byref(cfg),
                                          ctypes.byref(params), ctypes.byref(stats.c), dg._stream())


def _case(dg, m, n_slots, slots, step, tag):
    """Both entry points on the same bf16 final states and canvas; returns (static, reference)."""
    kv = dg.KV(SHAPE, n_slots, 600, fill=None)
    kv.set_lengths([37 * (i + 1) for i in range(n_slots)])
    rows = len(slots) * 256
    f = np_bf16_dev(synth.bf16_normal((rows, SHAPE.d_model), SEED, tag))
    canvas = torch.from_numpy(synth.tokens(n_slots * 256, SHAPE.vocab, SEED, tag + 1).reshape(n_slots, 256)).cuda()
    cfg = dg.sampler_cfg(seed=SEED + tag)
    view = kv.view(slots)
    got, ref = dg.Stats(n_slots, 256), dg.Stats(n_slots, 256)
    for s in (got, ref):
        for k in STATS:
            getattr(s, k).fill_(-7)
    params = _params(dg, step, f)
    rc = _call_static(dg, m, canvas, view, cfg, params, got)
    assert rc == dg.DG_OK, dg._lib.dg_last_error(m.ctx)
    m.denoise_step(canvas, kv, cfg, step, ref, flags=dg.DG_STEP_HEAD_ONLY, hidden_in=f, slots=slots)
    torch.cuda.synchronize()
    return got, ref


def _same(got, ref, what):
    for k in STATS:
        a, b = getattr(got, k), getattr(ref, k)
        assert torch.equal(a, b), f"{what}: {k} differs"


def test_static_head_matches_the_head_only_step_on_two_calls(env):
    dg, m = env
    # 1024 rows, slot-mapped in a pool of six (tokens gathered into the static scratch) ...
    got, ref = _case(dg, m, 6, [3, 1, 5, 0], 7, 10)
    _same(got, ref, "first call (4 requests, slots 3 1 5 0)")
    assert int((got.cand[torch.tensor([2, 4])] == -7).sum()) == 2 * 256  # slots outside the call untouched
    # ... then 256 rows, identity slots: must not see the first call's partials
    got, ref = _case(dg, m, 1, [0], 30, 20)
    _same(got, ref, "second call (1 request)")


def test_static_head_refuses_what_the_array_cannot_hold(env):
    dg, m = env
    kv = dg.KV(SHAPE, 8, 300, fill=None)
    kv.set_lengths([0] * 8)
    rows = 8 * 256  # 2048 rows x 256 slices x 32 bytes = 16 MiB, plus the tokens: too much
    f = torch.zeros((rows, SHAPE.d_model), dtype=torch.bfloat16, device="cuda")
    canvas = torch.zeros((8, 256), dtype=torch.int32, device="cuda")
    stats = dg.Stats(8, 256)
    stats.lse.fill_(-7)
    cfg = dg.sampler_cfg(seed=1)
    rc = _call_static(dg, m, canvas, kv.view(None), cfg, _params(dg, 0, f), stats)
    assert rc == dg.DG_ERR_CAPACITY
    assert b"static" in dg._lib.dg_last_error(m.ctx)
    bad = dg.StepParams(0, 0, dg._ptr(f), None, None)  # a full step is not this call's job
    assert _call_static(dg, m, canvas, kv.view([0]), cfg, bad, stats) == dg.DG_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((stats.lse == -7).all())
