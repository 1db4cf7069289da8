"""Pins for the oracle's sampler: schedule closed form, exact stop steps, invariants, statistics."""
import math

import numpy as np
import pytest
from scipy import special

from oracle import philox, sampler


def cfg(**kw):
    base = dict(max_steps=48, temp_start=0.8, temp_end=0.4, commit_per_step=16, renoise_conf=0.1,
                stable_steps=2, entropy_stop=-1.0, renoise_committed=True, seed=1234)
    base.update(kw)
    return sampler.SamplerConfig(**base)


def test_temperature_schedule_closed_form():
    c = cfg()
    T = [sampler.temperature(c, s) for s in range(48)]
    assert T[0] == np.float32(0.8) and T[47] == np.float32(0.4)
    assert all(a > b for a, b in zip(T, T[1:]))
    for s in (1, 10, 23, 46):
        assert T[s] == np.float32(0.8 - 0.4 * s / 47)
    assert all(t.dtype == np.float32 for t in T)


def test_row_stats_against_library_and_bruteforce():
    V, n = 37, 5
    r = np.random.default_rng(0)
    z = r.standard_normal((n, V)) * 3
    x = r.integers(0, V, n)
    T = np.float32(0.65)
    pos = np.arange(100, 100 + n)
    st = sampler.row_stats(z, x, T, 42, 1, pos, 3)
    t = z.astype(np.float32) / T
    lse = special.logsumexp(t.astype(np.float64), axis=1)
    p = special.softmax(t.astype(np.float64), axis=1)
    ent = -(p * np.log(p)).sum(1)
    assert np.allclose(st["lse"], lse, rtol=1e-6)
    assert np.allclose(st["entropy"], ent, atol=1e-5)
    for i in range(n):
        g = philox.gumbel_row(42, 1, int(pos[i]), 3, V)
        sc = [float(np.float32(t[i, v]) + np.float32(g[v])) for v in range(V)]
        best = max(range(V), key=lambda v: (sc[v], -v))
        assert st["cand"][i] == best
        assert st["t_cand"][i] == t[i, best] and st["t_cur"][i] == t[i, x[i]]
        s2 = sorted(sc)
        assert np.isclose(st["margin"][i], s2[-1] - s2[-2], atol=1e-6)


def _run(z_fn, c, C=256, V=1024, L=64, x0=None):
    pos = L + np.arange(C)
    x = sampler.canvas_init(c.seed, 0, pos, V) if x0 is None else x0.copy()
    com = np.zeros(C, bool)
    sr = 0
    hist = []
    for s in range(c.max_steps):
        st = sampler.row_stats(z_fn(s, x), x, sampler.temperature(c, s), c.seed, 0, pos, s)
        x_new, com_new, sr, status = sampler.sample_commit(st, x, com, sr, c, s, 0, pos, V)
        hist.append((x.copy(), com.copy(), x_new.copy(), com_new.copy(), status, st))
        x, com = x_new, com_new
        if status["stop"]:
            break
    return x, com, hist


def test_peaked_logits_stop_after_three_steps():
    """z = 50 * onehot(target): every draw is the target, confidence ~1, the canvas changes only
    at step 0, so the run stops after step 2 with 48 committed and canvas == targets."""
    V = 1024
    target = np.random.default_rng(1).integers(0, V, 256)
    z = np.zeros((256, V))
    z[np.arange(256), target] = 50.0
    x, com, hist = _run(lambda s, x: z, cfg(), V=V)
    assert len(hist) == 3
    assert np.array_equal(x, target)
    assert com.sum() == 48
    assert [h[4]["changed"] for h in hist] == [1, 0, 0]
    assert np.array_equal(np.nonzero(hist[0][3])[0], np.arange(16))  # ties → lowest index


def test_fixed_commit_schedule_without_renoise_of_committed():
    """Random logits, committed tokens never re-noised: 16 commits per step, all 256 committed
    after step 15, then two unchanged steps → 18 steps."""
    V = 1024
    r = np.random.default_rng(2)
    zs = r.standard_normal((48, 256, V))
    x, com, hist = _run(lambda s, x: zs[s], cfg(renoise_committed=False), V=V)
    assert len(hist) == 18
    assert [int(h[3].sum()) for h in hist[:16]] == [16 * (i + 1) for i in range(16)]
    assert com.all()
    assert [h[4]["changed"] for h in hist[-3:]] == [1, 0, 0]


def test_commit_count_and_fixed_committed_invariants():
    V = 1024
    r = np.random.default_rng(3)
    target = r.integers(0, V, 256)

    def z_fn(s, x):  # mixed: half the rows peaked, half random → some keep, some re-noise
        z = r.standard_normal((256, V))
        z[np.arange(0, 256, 2), target[::2]] = 12.0
        return z

    c = cfg()
    pos = 64 + np.arange(256)  # _run's positions
    _, _, hist = _run(z_fn, c, V=V)
    n_dropped = 0
    for step, (x0, c0, x1, c1, status, st) in enumerate(hist):
        U = int((~c0).sum())
        renoised_committed = int((c0 & ~c1).sum())
        assert c1.sum() == c0.sum() - renoised_committed + min(16, U)
        # a committed position keeps its token unless it was re-noised (then it is uncommitted)
        kept = c0 & c1
        assert np.array_equal(x0[kept], x1[kept])
        # re-noised committed positions got the step's fresh token
        drop = c0 & ~c1
        fresh = philox.token_draw(c.seed, 0, pos, step, philox.RENOISE, V)
        assert np.array_equal(x1[drop], fresh[drop])
        n_dropped += int(drop.sum())
        # newly committed positions hold their candidate
        new = ~c0 & c1
        assert np.array_equal(x1[new], st["cand"][new])
        assert new.sum() == min(16, U)
    assert n_dropped > 0  # the mixed logits do re-noise some committed positions


def test_selection_is_topm_by_confidence():
    V, C = 64, 40
    r = np.random.default_rng(4)
    st = {"cand": r.integers(0, V, C).astype(np.int32),
          "t_cand": np.round(r.standard_normal(C), 1).astype(np.float32),  # ties
          "t_cur": r.standard_normal(C).astype(np.float32),
          "lse": np.zeros(C, np.float32), "entropy": np.ones(C, np.float32),
          "margin": np.ones(C, np.float32)}
    com = np.zeros(C, bool)
    com[::3] = True
    x = r.integers(0, V, C).astype(np.int32)
    c = cfg(commit_per_step=5)
    _, _, _, status = sampler.sample_commit(st, x, com, 0, c, 0, 0, np.arange(C), V)
    U = [i for i in range(C) if not com[i]]
    want = sorted(U, key=lambda i: (-float(st["t_cand"][i]), i))[:5]
    assert list(status["selected"]) == want


def test_same_seed_same_trajectory_and_seed_matters():
    V = 1024
    zs = np.random.default_rng(5).standard_normal((48, 256, V))
    a = _run(lambda s, x: zs[s], cfg(max_steps=6), V=V)
    b = _run(lambda s, x: zs[s], cfg(max_steps=6), V=V)
    c = _run(lambda s, x: zs[s], cfg(max_steps=6, seed=99), V=V)
    assert np.array_equal(a[0], b[0]) and len(a[2]) == len(b[2]) == 6
    assert not np.array_equal(a[0], c[0])


def test_step_cap_stops():
    V = 1024
    zs = np.random.default_rng(6).standard_normal((5, 256, V))
    _, _, hist = _run(lambda s, x: zs[s], cfg(max_steps=5), V=V)
    assert len(hist) == 5 and hist[-1][4]["stop"] == 1


def test_entropy_stop_optional():
    V = 1024
    target = np.random.default_rng(7).integers(0, V, 256)
    z = np.zeros((256, V))
    z[np.arange(256), target] = 50.0
    # entropy ~0 and unchanged at step 1 → stops one step earlier than the stable-run rule
    _, _, hist = _run(lambda s, x: z, cfg(entropy_stop=0.005), V=V)
    assert len(hist) == 2
    _, _, hist = _run(lambda s, x: z, cfg(entropy_stop=0.005, stable_steps=5), V=V)
    assert len(hist) == 2


def test_canvas_init_is_uniform_and_positional():
    a = sampler.canvas_init(3, 0, np.arange(256), 1024)
    b = sampler.canvas_init(3, 0, np.arange(256, 512), 1024)
    assert a.min() >= 0 and a.max() < 1024 and (a != b).mean() > 0.9


# ----- entropy-bounded selection ([DOCS] table, token-selection row) -----

def _stats(ent, cand=None, V=64):
    C = len(ent)
    r = np.random.default_rng(11)
    return {"cand": (r.integers(0, V, C) if cand is None else np.asarray(cand)).astype(np.int32),
            "t_cand": np.zeros(C, np.float32), "t_cur": np.zeros(C, np.float32),
            "lse": np.zeros(C, np.float32), "entropy": np.asarray(ent, np.float32),
            "margin": np.ones(C, np.float32)}


def _select(ent, com=None, budget=0.1, **kw):
    C = len(ent)
    st = _stats(ent)
    com = np.zeros(C, bool) if com is None else np.asarray(com, bool)
    x = np.arange(C, dtype=np.int32) % 64
    c = cfg(select_mode=1, entropy_budget=budget, renoise_committed=False, **kw)
    x1, c1, _, status = sampler.sample_commit(st, x, com, 0, c, 0, 0, np.arange(C), 64)
    return st, x, x1, c1, status


def test_entropy_selection_hand_worked():
    # uncommitted 0..5 with H = .05 .02 .04 .5 .01(committed) .03: ascending over U is
    # 1 (.02), 5 (.03), 2 (.04), 0 (.05) ...; running sums .02 .05 .09 .14 -> {1, 5, 2}
    ent = [0.05, 0.02, 0.04, 0.5, 0.01, 0.03]
    com = [0, 0, 0, 0, 1, 0]
    st, x, x1, c1, status = _select(ent, com)
    assert list(status["selected"]) == [1, 5, 2] and status["n_new"] == 3
    assert list(c1) == [False, True, True, False, True, True]
    assert all(x1[i] == st["cand"][i] for i in (1, 5, 2))
    # every unselected uncommitted slot got the fresh uniform token of its position
    fresh = philox.token_draw(1234, 0, np.arange(6), 0, philox.RENOISE, 64)
    assert x1[0] == fresh[0] and x1[3] == fresh[3] and status["n_renoised"] == 2
    assert x1[4] == x[4]  # committed and not re-noised (flag off)


def test_entropy_selection_takes_at_least_one_and_lowest_index_on_ties():
    st, x, x1, c1, status = _select([3.0, 2.5, 2.5, 7.0])
    assert list(status["selected"]) == [1]
    # equal entropies: lower index first; .03 * 3 = .09 <= .1 < .12
    _, _, _, _, status = _select([0.03] * 8)
    assert list(status["selected"]) == [0, 1, 2]
    # the budget is inclusive: dyadic entropies summing to exactly the budget are all taken
    _, _, _, _, status = _select([0.25, 0.125, 0.125, 0.5], budget=0.5)
    assert list(status["selected"]) == [1, 2, 0]
    # nothing uncommitted: nothing selected
    _, _, x1, _, status = _select([0.0] * 4, com=[1] * 4)
    assert status["n_new"] == 0 and len(status["selected"]) == 0


def test_entropy_selection_matches_bruteforce_over_exact_sums():
    """Position i is selected iff the exact sum of the entropies of every uncommitted position
    ordered at or before it is within the budget, or it comes first.  Entropies are multiples
    of 1/256 below 1, so every float32 partial sum is exact and both rules must agree."""
    from fractions import Fraction
    r = np.random.default_rng(12)
    for trial in range(200):
        C = int(r.integers(1, 24))
        q = r.integers(0, 24, C)  # many ties
        ent = q / 256.0
        com = r.random(C) < 0.3
        budget = float(r.integers(0, 40)) / 256.0
        _, _, _, _, status = _select(ent, com, budget=budget)
        U = [i for i in range(C) if not com[i]]
        order = sorted(U, key=lambda i: (Fraction(int(q[i]), 256), i))
        want = [i for k, i in enumerate(order)
                if k == 0 or sum(Fraction(int(q[j]), 256) for j in order[:k + 1])
                <= Fraction(int(round(budget * 256)), 256)]
        assert list(status["selected"]) == want, (trial, ent, com, budget)


def test_entropy_selection_run_peaked_and_random():
    V = 1024
    target = np.random.default_rng(7).integers(0, V, 256)
    z = np.zeros((256, V))
    z[np.arange(256), target] = 50.0
    # near-zero entropy everywhere: all 256 are selected at step 0, the canvas is then still,
    # so the entropy stop ends the run at step 1 and the stable-run rule at step 2
    x, com, hist = _run(lambda s, x: z, cfg(select_mode=1, entropy_stop=0.005), V=V)
    assert len(hist) == 2 and hist[0][4]["n_new"] == 256 and com.all()
    assert np.array_equal(x, target)
    _, _, hist = _run(lambda s, x: z, cfg(select_mode=1), V=V)
    assert len(hist) == 3
    # random logits: entropies are far above the budget, so exactly one commit per step and
    # every other uncommitted slot is re-noised
    zs = np.random.default_rng(8).standard_normal((6, 256, V))
    _, com, hist = _run(lambda s, x: zs[s], cfg(select_mode=1, max_steps=6,
                                                 renoise_committed=False), V=V)
    assert [h[4]["n_committed"] for h in hist] == [1, 2, 3, 4, 5, 6]
    assert [h[4]["n_renoised"] for h in hist] == [255, 254, 253, 252, 251, 250]
