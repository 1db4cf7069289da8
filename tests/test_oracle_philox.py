"""Pins for the oracle's counter-based RNG and the draws built on it (CPU only)."""
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("->")
        a = [int(v, 16) for v in lhs.split()]
        b = [int(v, 16) for v in rhs.split()]
        out.append((a[:4], a[4:], b))
    return out


@pytest.mark.parametrize("ctr,key,want", _kat())
def test_known_answers_scalar(ctr, key, want):
    assert list(philox.philox_scalar(ctr, key)) == want


@pytest.mark.parametrize("ctr,key,want", _kat())
def test_known_answers_vector(ctr, key, want):
    got = philox.philox_np(*ctr, *key)
    assert [int(g) for g in got] == want


def test_two_implementations_agree():
    rng = np.random.default_rng(7)
    c = rng.integers(0, 2**32, size=(500, 4), dtype=np.uint64)
    k = rng.integers(0, 2**32, size=2, dtype=np.uint64)
    vec = np.stack(philox.philox_np(c[:, 0], c[:, 1], c[:, 2], c[:, 3], int(k[0]), int(k[1])), 1)
    for i in range(c.shape[0]):
        assert tuple(int(v) for v in vec[i]) == philox.philox_scalar(c[i], k)


def test_uniform_mapping_is_exact_and_open():
    w = np.array([0, 1, 511, 512, 2**32 - 1, 2**31, 12345678], dtype=np.uint32)
    u = philox.uniform_from_word(w)
    assert u.dtype == np.float32
    assert np.all(u > 0) and np.all(u < 1)
    # u * 2^23 - 0.5 must be exactly the integer w >> 9
    back = u.astype(np.float64) * 2.0**23 - 0.5
    assert np.array_equal(back, (w >> 9).astype(np.float64))
    assert u[0] == np.float32(2.0**-24) and u[4] == np.float32(1 - 2.0**-24)


def test_uniform_chi2():
    k0, k1 = philox.seed_key(99)
    w = np.concatenate(philox.philox_np(np.arange(50000), 3, 4, 5, k0, k1))
    u = philox.uniform_from_word(w)
    counts, _ = np.histogram(u, bins=64, range=(0, 1))
    p = stats.chisquare(counts).pvalue
    assert p > 1e-4


def test_gumbel_moments():
    g = np.concatenate([philox.gumbel_row(5, 0, p, 2, 65536) for p in range(16)]).astype(np.float64)
    n = g.size
    assert abs(g.mean() - 0.5772156649) < 5 * math.sqrt(math.pi**2 / 6 / n)
    assert abs(g.var() - math.pi**2 / 6) < 0.02


def test_gumbel_max_matches_softmax():
    """argmax(t + G) is a draw from softmax(t)."""
    t = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4, 0.7, 1.6], np.float32)
    p = np.exp(t - t.max())
    p /= p.sum()
    n = 40000
    g = np.stack([philox.gumbel_row(11, 0, pos, 0, 8) for pos in range(n)])
    draws = np.argmax(t[None, :] + g, axis=1)
    counts = np.bincount(draws, minlength=8)
    assert stats.chisquare(counts, n * p).pvalue > 1e-4


def test_gumbel_row_word_layout():
    """Entry v uses word v & 3 of counter chunk v >> 2 (checked against the scalar generator)."""
    seed, b, pos, step = (1 << 40) + 17, 3, 777, 9
    g = philox.gumbel_row(seed, b, pos, step, 13)
    k = philox.seed_key(seed)
    for v in range(13):
        w = philox.philox_scalar((v >> 2, pos, step, (b << 8) | philox.GUMBEL), k)[v & 3]
        u = ((w >> 9) + 0.5) / 2.0**23
        assert abs(float(g[v]) - (-math.log(-math.log(u)))) < 1e-5


def test_token_draw_range_and_uniformity():
    V = 1000
    tok = philox.token_draw(3, 0, np.arange(200000), 5, philox.RENOISE, V)
    assert tok.min() >= 0 and tok.max() < V
    counts = np.bincount(tok, minlength=V)
    assert stats.chisquare(counts).pvalue > 1e-4
    # multiply-shift against exact integer arithmetic
    k = philox.seed_key(3)
    for p in (0, 1, 199999):
        w = philox.philox_scalar((0, p, 5, philox.RENOISE), k)[0]
        assert tok[p] == (w * V) >> 32


def test_streams_and_steps_differ():
    a = philox.token_draw(1, 0, np.arange(64), 0, philox.INIT, 1 << 16)
    b = philox.token_draw(1, 0, np.arange(64), 0, philox.RENOISE, 1 << 16)
    c = philox.token_draw(1, 0, np.arange(64), 1, philox.RENOISE, 1 << 16)
    d = philox.token_draw(1, 1, np.arange(64), 1, philox.RENOISE, 1 << 16)
    assert (a != b).mean() > 0.9 and (b != c).mean() > 0.9 and (c != d).mean() > 0.9
