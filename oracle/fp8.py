"""FP8 (OCP E4M3) expert weights with one float32 scale per output channel.

Test infrastructure: the plain reference the GPU path is checked against.  Nothing in the
product imports it.

Sources: [NEWS] third paragraph (FP8 and NVFP4 checkpoints are published; a quantized build
fits in 18 GB) and fourth paragraph (the H200 throughput figure is measured with FP8 weights);
[DOCS] feature list (the quantized model fits consumer GPUs).  The pages name the format only;
the encoding below is the OCP 8-bit floating point E4M3 format, written from its definition:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 1..15: (-1)^s * 2^(e - 7) * (1 + m / 8);  field 0: (-1)^s * 2^-6 * (m / 8);
* S.1111.111 is NaN; there are no infinities; the largest finite value is 448 (S.1111.110).

Readings (the pages give none of this):

* per output channel (one row of an [out][in] matrix): scale = amax / 448 in float32, where
  amax is the largest |w| of the row (exact: the weights are bfloat16); an all-zero row gets
  scale 1;
* q = encode(float32(w) / scale), the division in float32, the encoding rounding to nearest
  with ties to even and saturating at +-448 (values beyond it, finite, become +-448);
* the dequantized weight is scale * decode(q), exactly; the product over the row is scaled after
  the sum, which is the same value.

Parity: pinned by tests/test_oracle_fp8.py (the format's own table: every byte decodes to the
value the definition gives and encodes back to itself; ties between neighbours go to the even
mantissa; saturation; the subnormal range; per-row scaling maps the row maximum to 448).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode(q: np.ndarray) -> np.ndarray:
    """Bytes (uint8) to their float64 values; NaN for the two NaN encodings."""
    q = np.asarray(q, dtype=np.uint8).astype(np.int64)
    s = np.where((q >> 7) & 1, -1.0, 1.0)
    e = (q >> 3) & 15
    m = (q & 7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    val = np.where((e == 15) & ((q & 7) == 7), np.nan, val)
    return s * val


def encode(x: np.ndarray) -> np.ndarray:
    """Finite float32 values to E4M3 bytes: round to nearest, ties to even, saturating."""
    x = np.asarray(x, dtype=np.float32)
    sign = (np.signbit(x)).astype(np.int64) << 7
    a = np.abs(x.astype(np.float64))  # exact
    out = np.zeros(a.shape, dtype=np.int64)
    sat = a >= E4M3_MAX
    sub = (a < 2.0 ** -6) & ~sat
    nor = ~sat & ~sub
    # subnormal grid: multiples of 2^-9 (m / 8 * 2^-6); m = 8 is the smallest normal, 0x08
    out = np.where(sub, np.rint(np.where(sub, a, 0.0) * 512.0).astype(np.int64), out)
    # normal: a = 2^e * f with f in [1, 2)
    fr, ex = np.frexp(np.where(nor, a, 1.0))  # a = fr * 2^ex, fr in [0.5, 1)
    e = ex - 1
    m = np.rint((fr * 2.0 - 1.0) * 8.0).astype(np.int64)  # (f - 1) * 8, ties to even
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    out = np.where(nor, ((e + 7) << 3) | m, out)
    out = np.where(sat, 0x7E, out)
    return (out | sign).astype(np.uint8)


def quantize_rows(w: np.ndarray):
    """Per-row E4M3 quantization of w [rows, cols] (bfloat16 values).

    Returns (q uint8 [rows, cols], scale float32 [rows])."""
    w32 = np.asarray(w, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(w32), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    x = (w32 / scale[..., None]).astype(np.float32)  # float32 division
    return encode(x), scale


def dequantize_rows(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """scale * decode(q), float64 [rows, cols]."""
    return np.asarray(scale, np.float64)[..., None] * decode(q)


def dequantize_experts(lw: dict) -> dict:
    """A layer's weights with the routed experts replaced by their E4M3 round trip (the shared
    FFN, attention and router stay as they are)."""
    out = dict(lw)
    for name in ("w_gate", "w_up", "w_down"):
        w = np.asarray(lw[name], np.float64)
        q, s = quantize_rows(w.reshape(-1, w.shape[-1]))
        out[name] = dequantize_rows(q, s).reshape(w.shape)
    return out
