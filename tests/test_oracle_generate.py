"""Invariants of the oracle's block-autoregressive loop (CPU, tiny shapes)."""
import dataclasses

import numpy as np

from oracle import generate, model, sampler
from block_discrete_diffusion_amd import synth

SHAPE = synth.ModelShape(n_layers=2, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8,
                         n_experts=4, top_k=2, d_ff_expert=24, d_ff_shared=0, vocab=64, canvas=16)


def _cfg(**kw):
    c = dict(max_steps=8, temp_start=0.8, temp_end=0.4, commit_per_step=4, renoise_conf=0.1,
             stable_steps=2, seed=77)
    c.update(kw)
    return sampler.SamplerConfig(**c)


def test_generate_grows_cache_and_blocks_condition_on_history():
    w = synth.model_weights(SHAPE, 3)
    prefix = synth.tokens(10, SHAPE.vocab, 3)
    out = generate.generate(w, SHAPE, prefix, 2, _cfg())
    assert out["length"] == 10 + 2 * 16
    ck, cv = out["cache_k"], out["cache_v"]
    # prefix part equals a standalone prefill
    pk, pv = generate.new_cache(SHAPE, 10)
    model.prefill(w, SHAPE, prefix, pk, pv, 0)
    for l in range(2):
        assert np.array_equal(ck[l][:, :10], pk[l][:, :10])
    # first block's K/V are the bidirectional canvas K/V of its final tokens
    toks0 = out["blocks"][0]["tokens"]
    fw = model.denoise_forward(w, SHAPE, toks0, ck, cv, 10, with_head=False)
    for l in range(2):
        assert np.allclose(ck[l][:, 10:26], model.to_bf16(fw["canvas_k"][l]), atol=2e-2)
    # a different prefix gives a different first block (the canvas conditions on the cache)
    out2 = generate.generate(w, SHAPE, (prefix + 1) % SHAPE.vocab, 1, _cfg())
    assert not np.array_equal(out2["blocks"][0]["trace"][0]["tokens"], out["blocks"][0]["trace"][0]["tokens"])


def test_resume_from_snapshot_equals_uninterrupted():
    w = synth.model_weights(SHAPE, 4)
    prefix = synth.tokens(8, SHAPE.vocab, 4)
    ck, cv = generate.new_cache(SHAPE, 8 + 16)
    model.prefill(w, SHAPE, prefix, ck, cv, 0)
    c = _cfg(max_steps=8, renoise_committed=True)
    full = generate.denoise_canvas(w, SHAPE, ck, cv, 8, c)
    part = generate.denoise_canvas(w, SHAPE, ck, cv, 8, c, max_step=3)
    rest = generate.denoise_canvas(w, SHAPE, ck, cv, 8, c, tokens=part["tokens"],
                                   committed=part["committed"], stable_run=part["stable_run"],
                                   start_step=part["next_step"])
    assert np.array_equal(rest["tokens"], full["tokens"])
    assert part["steps"] + rest["steps"] == full["steps"]


def test_commit_refreshes_kv_when_last_step_changed_canvas():
    w = synth.model_weights(SHAPE, 5)
    ck, cv = generate.new_cache(SHAPE, 4 + 16)
    model.prefill(w, SHAPE, synth.tokens(4, SHAPE.vocab, 5), ck, cv, 0)
    res = generate.denoise_canvas(w, SHAPE, ck, cv, 4, _cfg(max_steps=3))  # random weights: cap
    assert res["steps"] == 3 and res["last_changed"]
    L = generate.finish_block(w, SHAPE, ck, cv, 4, res)
    fw = model.denoise_forward(w, SHAPE, res["tokens"], ck, cv, 4, with_head=False)
    assert L == 20
    for l in range(2):
        assert np.array_equal(ck[l][:, 4:20], model.to_bf16(fw["canvas_k"][l]))
