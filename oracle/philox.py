"""Philox4x32-10 counter-based RNG and the draws the sampler takes from it.

Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11): a 4×32-bit counter is mixed with a 2×32-bit key by ten
rounds, each round multiplying two counter words by fixed constants, swapping and xoring the
high halves with the key words, and bumping the key by two Weyl constants between rounds.
Both implementations below are written from that definition and share no code; the tests check
them against each other and against the published known-answer vectors.

How the method uses it (the pages only say the canvas starts from random tokens and that
low-confidence positions get random tokens; the counter layout below is a reading of them):

* key     = (seed & 0xffffffff, seed >> 32)
* counter = (c0, p, s, (b << 8) | stream) with p the absolute sequence position, s the denoise
            step, b the request index, and c0 = v >> 2 for the Gumbel draw of vocab entry v
            (word v & 3 of the output), 0 otherwise.
* streams: GUMBEL 0, RENOISE 1, INIT 2.
* uniform in (0, 1):   u = ((w >> 9) + 0.5) * 2^-23   (exact in float32; never 0 or 1)
* Gumbel(0, 1):        g = -log(-log(u)) in float32
* token in [0, V):     (w * V) >> 32   (multiply-shift; exact integer arithmetic)

Parity: pinned (known-answer vectors; two independent implementations; distribution tests).
"""
from __future__ import annotations

import numpy as np

GUMBEL, RENOISE, INIT = 0, 1, 2

# Round multipliers and key increments of Philox4x32 (Salmon et al., SC'11).
_M0 = 0xD2511F53
_M1 = 0xCD9E8D57
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK = 0xFFFFFFFF


# --------------------------------------------------------------------------------------------
# Implementation A: scalar Python integers.
# --------------------------------------------------------------------------------------------

def philox_scalar(ctr, key, rounds: int = 10):
    """One Philox4x32 block: ctr = 4 ints, key = 2 ints → 4 ints (each < 2^32)."""
    c0, c1, c2, c3 = (int(v) & _MASK for v in ctr)
    k0, k1 = (int(v) & _MASK for v in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> 32, p0 & _MASK
        hi1, lo1 = p1 >> 32, p1 & _MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return (c0, c1, c2, c3)


# --------------------------------------------------------------------------------------------
# Implementation B: vectorised NumPy over many counters.
# --------------------------------------------------------------------------------------------

def philox_np(c0, c1, c2, c3, k0, k1, rounds: int = 10):
    """Vectorised Philox4x32: counter words are broadcastable integer arrays; returns 4 uint32
    arrays.  Products are formed in uint64, which holds a 32×32-bit product exactly."""
    x = [np.asarray(c, dtype=np.uint64) & np.uint64(_MASK) for c in (c0, c1, c2, c3)]
    x = np.broadcast_arrays(*x)
    x = [a.copy() for a in x]
    key0 = np.uint64(int(k0) & _MASK)
    key1 = np.uint64(int(k1) & _MASK)
    m0, m1 = np.uint64(_M0), np.uint64(_M1)
    mask, sh = np.uint64(_MASK), np.uint64(32)
    for r in range(rounds):
        if r:
            key0 = np.uint64((int(key0) + _W0) & _MASK)
            key1 = np.uint64((int(key1) + _W1) & _MASK)
        prod0 = x[0] * m0
        prod1 = x[2] * m1
        y0 = (prod1 >> sh) ^ x[1] ^ key0
        y1 = prod1 & mask
        y2 = (prod0 >> sh) ^ x[3] ^ key1
        y3 = prod0 & mask
        x = [y0, y1, y2, y3]
    return tuple(a.astype(np.uint32) for a in x)


def seed_key(seed: int):
    seed = int(seed) & ((1 << 64) - 1)
    return seed & _MASK, seed >> 32


def stream_word(b: int, stream: int) -> int:
    return ((int(b) << 8) | int(stream)) & _MASK


def uniform_from_word(w) -> np.ndarray:
    """u = ((w >> 9) + 0.5) * 2^-23 in float32 (every step exact)."""
    w = np.asarray(w, dtype=np.uint32)
    return ((w >> np.uint32(9)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)


def gumbel_row(seed: int, b: int, pos: int, step: int, vocab: int) -> np.ndarray:
    """Gumbel(0,1) noise for every vocab entry of one canvas position, float32 [vocab]."""
    k0, k1 = seed_key(seed)
    chunks = np.arange((vocab + 3) // 4, dtype=np.uint64)
    w = philox_np(chunks, pos, step, stream_word(b, GUMBEL), k0, k1)
    words = np.stack(w, axis=1).reshape(-1)[:vocab]  # entry v is word v & 3 of chunk v >> 2
    u = uniform_from_word(words)
    return -np.log(-np.log(u))


def gumbel_rows(seed: int, b: int, positions, step: int, vocab: int) -> np.ndarray:
    """Gumbel noise for several positions: float32 [len(positions), vocab]."""
    return np.stack([gumbel_row(seed, b, int(p), step, vocab) for p in positions])


def token_draw(seed: int, b: int, positions, step: int, stream: int, vocab: int) -> np.ndarray:
    """Uniform token ids, one per position: (word0 * vocab) >> 32."""
    k0, k1 = seed_key(seed)
    pos = np.asarray(positions, dtype=np.uint64)
    w0 = philox_np(0, pos, step, stream_word(b, stream), k0, k1)[0]
    return ((w0.astype(np.uint64) * np.uint64(vocab)) >> np.uint64(32)).astype(np.int32)
