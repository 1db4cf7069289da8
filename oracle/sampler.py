"""Confidence sampler of one denoise step: temperature, Gumbel-max draw, commit, re-noise, stop.

Sources: [DOCS] table "Configuração de exibição recomendada" (at most 48 steps; temperature
linear from 0.8 down to 0.4 as a function of the step; adaptive early stop when the canvas has
settled; token selection); [NEWS] second paragraph (15-20 high-confidence tokens per pass are
kept as anchors and low-confidence positions may be re-noised later); [GUIDE] Sudoku demo (when
confidence drops, the sampler puts random tokens back); [RANK] "Pontos-chave" (correct tokens are
consolidated and used as anchors).

Readings (the pages leave these open; the configuration used for this path fixes them):

* T_s = T0 + (T1 - T0) * s / (S_max - 1), in float64, rounded once to float32.
* t = z / T_s per logit (float32).  The draw is Gumbel-max: y = argmax_v (t_v + g_v), lowest v on
  ties.  The confidence of a position is its tempered log-probability, log kappa = t - lse(t),
  of the drawn token (candidate) or of the current token (committed positions).
* Commit (select_mode 0): the min(m, |U|) uncommitted positions with the highest candidate
  confidence (lowest index on ties) take their candidate and become committed.
* Commit (select_mode 1, [DOCS] table, token-selection row): the uncommitted positions are
  taken in ascending order of entropy (lowest index on ties) and added while the running
  float32 sum of their entropies, added in that order, stays <= the budget (0.1); the first
  one is always taken.  Those take their candidate and become committed.
* Re-noise: a position committed before this step whose current-token confidence is below tau
  gets a fresh uniform token and is uncommitted (flag).  In select_mode 0 every other
  uncommitted position takes its candidate when its confidence is >= tau and a fresh uniform
  token otherwise; in select_mode 1 every unselected uncommitted position gets a fresh uniform
  token (the token-selection row re-noises what it did not select).
* Stop: stable_run counts consecutive steps that changed no token; stop once it reaches
  `stable_steps`, or at the last allowed step, or (optional, off by default) when the mean
  entropy is below `entropy_stop` and the step changed nothing.

Decisions (argmax, ranking, threshold) are taken in float32 like the kernels take them; lse and
entropy are accumulated in float64 and rounded to float32.

Parity: pinned by tests/test_oracle_sampler.py (closed-form schedule, peaked-logits fixture with
an exact stop step, the fixed-commit schedule, Gumbel-max statistics, invariants, determinism,
hand-worked entropy-bounded selections and a brute-force check of the selection rule).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Sequence

import numpy as np

from . import philox


@dataclasses.dataclass
class SamplerConfig:
    max_steps: int = 48
    temp_start: float = 0.8
    temp_end: float = 0.4
    commit_per_step: int = 16
    renoise_conf: float = 0.1
    stable_steps: int = 2
    entropy_stop: float = -1.0  # < 0: off
    renoise_committed: bool = True
    seed: int = 0
    select_mode: int = 0  # 0: top commit_per_step by confidence; 1: entropy-bounded
    entropy_budget: float = 0.1


def entropy_bounded_count(h_sorted: np.ndarray, budget: float) -> int:
    """How many of the entropies (already in selection order) are selected: the longest
    prefix whose float32 running sum, added left to right, stays <= budget; at least one
    when there is any ([DOCS] table, token-selection row)."""
    n = h_sorted.shape[0]
    if n == 0:
        return 0
    b = np.float32(budget)
    run = np.float32(0.0)
    k = 0
    for j in range(n):
        run = np.float32(run + np.float32(h_sorted[j]))
        if j > 0 and run > b:
            break
        k = j + 1
    return k


def temperature(cfg: SamplerConfig, step: int) -> np.float32:
    if cfg.max_steps <= 1:
        return np.float32(cfg.temp_start)
    t = cfg.temp_start + (cfg.temp_end - cfg.temp_start) * step / (cfg.max_steps - 1)
    return np.float32(t)


def row_stats(z: np.ndarray, x: Sequence[int], T: np.float32, seed: int, b: int,
              positions: Sequence[int], step: int) -> Dict[str, np.ndarray]:
    """Per-position statistics of the tempered distribution and the Gumbel-max draw.

    z: logits [n, V] (any float precision); x: current tokens [n].
    Returns float32 arrays t_cand, t_cur, lse, entropy, margin and int32 cand."""
    z32 = np.asarray(z, dtype=np.float64).astype(np.float32)
    n, V = z32.shape
    t = z32 / np.float32(T)  # float32 division
    g = philox.gumbel_rows(seed, b, positions, step, V)
    score = t + g  # float32
    cand = np.argmax(score, axis=1)  # first maximum = lowest index on ties
    srt = np.sort(score, axis=1)
    margin = (srt[:, -1] - srt[:, -2]).astype(np.float32)
    t64 = t.astype(np.float64)
    m = t64.max(axis=1, keepdims=True)
    e = np.exp(t64 - m)
    s = e.sum(axis=1)
    lse = m[:, 0] + np.log(s)
    ent = lse - (e * t64).sum(axis=1) / s
    rows = np.arange(n)
    xi = np.asarray(x, dtype=np.int64)
    return {
        "cand": cand.astype(np.int32),
        "t_cand": t[rows, cand].astype(np.float32),
        "t_cur": t[rows, xi].astype(np.float32),
        "lse": lse.astype(np.float32),
        "entropy": ent.astype(np.float32),
        "margin": margin,
    }


def sample_commit(stats: Dict[str, np.ndarray], tokens: np.ndarray, committed: np.ndarray,
                  stable_run: int, cfg: SamplerConfig, step: int, b: int,
                  positions: Sequence[int], vocab: int):
    """One sampler step for one canvas.  Returns (tokens, committed, stable_run, status)."""
    x_prev = np.asarray(tokens, dtype=np.int32)
    com_prev = np.asarray(committed, dtype=bool)
    n = x_prev.shape[0]
    x = x_prev.copy()
    com = com_prev.copy()
    conf_cand = (stats["t_cand"].astype(np.float32) - stats["lse"].astype(np.float32))
    conf_cur = (stats["t_cur"].astype(np.float32) - stats["lse"].astype(np.float32))
    log_tau = np.float32(math.log(cfg.renoise_conf)) if cfg.renoise_conf > 0 else np.float32(-np.inf)
    fresh = philox.token_draw(cfg.seed, b, positions, step, philox.RENOISE, vocab)

    U = np.nonzero(~com_prev)[0]
    if cfg.select_mode == 1:
        # rank U by entropy ascending, index ascending
        ent = stats["entropy"].astype(np.float32)
        order = U[np.lexsort((U, ent[U].astype(np.float64)))]
        m = entropy_bounded_count(ent[order], cfg.entropy_budget)
    else:
        # rank U by confidence descending, index ascending
        order = U[np.lexsort((U, -conf_cand[U].astype(np.float64)))]
        m = min(cfg.commit_per_step, U.size)
    S = order[:m]
    rest = order[m:]
    x[S] = stats["cand"][S]
    com[S] = True
    n_renoised = 0
    if cfg.renoise_committed:
        C_prev = np.nonzero(com_prev)[0]
        drop = C_prev[conf_cur[C_prev] < log_tau]
        x[drop] = fresh[drop]
        com[drop] = False
        n_renoised += drop.size
    if cfg.select_mode == 1:
        low = rest
        keep = rest[:0]
    else:
        low = rest[conf_cand[rest] < log_tau]
        keep = rest[~(conf_cand[rest] < log_tau)]
    x[low] = fresh[low]
    x[keep] = stats["cand"][keep]
    n_renoised += low.size

    changed = bool(np.any(x != x_prev))
    stable_run = 0 if changed else stable_run + 1
    mean_ent = float(np.mean(stats["entropy"].astype(np.float64)))
    stop = stable_run >= cfg.stable_steps or step >= cfg.max_steps - 1
    if cfg.entropy_stop >= 0 and (not changed) and mean_ent < cfg.entropy_stop:
        stop = True
    status = {
        "changed": int(changed), "n_committed": int(com.sum()), "n_new": int(m),
        "n_renoised": int(n_renoised), "stable_run": int(stable_run), "stop": int(stop),
        "nonfinite": int(not np.all(np.isfinite(stats["lse"]))), "mean_entropy": mean_ent,
        "selected": S.astype(np.int32),
    }
    return x, com, stable_run, status


def canvas_init(seed: int, b: int, positions: Sequence[int], vocab: int) -> np.ndarray:
    """Uniform-state start: every canvas slot gets a uniform random token ([GUIDE]
    "Arquitetura em Detalhes", uniform-state diffusion)."""
    return philox.token_draw(seed, b, positions, 0, philox.INIT, vocab)
