"""Pins for the oracle's E4M3 encoding and per-channel quantization: the format's own values,
a brute-force nearest-value search, ties, saturation, the subnormal range and row scaling."""
import numpy as np

from oracle import fp8


def test_known_encodings_of_the_format():
    # values that the OCP E4M3 definition fixes
    table = {0x00: 0.0, 0x38: 1.0, 0x30: 0.5, 0x40: 2.0, 0xC0: -2.0, 0x3C: 1.5, 0x77: 240.0,
             0x78: 256.0, 0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x07: 0.875 * 2.0 ** -6,
             0x01: 2.0 ** -9, 0x81: -(2.0 ** -9)}
    for b, v in table.items():
        assert fp8.decode(np.uint8(b)) == v, hex(b)
        assert fp8.encode(np.float32(v)) == b, hex(b)
    assert np.isnan(fp8.decode(np.uint8(0x7F))) and np.isnan(fp8.decode(np.uint8(0xFF)))
    assert fp8.encode(np.float32(-0.0)) == 0x80


def test_every_finite_byte_round_trips_and_values_increase():
    b = np.arange(0x7F, dtype=np.uint8)  # positive finite codes
    v = fp8.decode(b)
    assert np.all(np.diff(v) > 0)
    for sign in (0, 0x80):
        bb = (b | sign).astype(np.uint8)
        assert np.array_equal(fp8.encode(fp8.decode(bb).astype(np.float32)), bb)


def _nearest_bruteforce(x: float) -> int:
    """The finite code nearest to x; on a tie the one with the even mantissa; beyond the
    largest finite value the largest (saturation)."""
    codes = [c for c in range(256) if not np.isnan(fp8.decode(np.uint8(c)))]
    if abs(x) >= 448.0:
        return 0x7E | (0x80 if x < 0 else 0)
    best = None
    for c in codes:
        if (c >> 7) != (1 if np.signbit(x) else 0):
            continue
        d = abs(float(fp8.decode(np.uint8(c))) - x)
        key = (d, c & 1)  # ties: the even mantissa (lowest bit 0) wins
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_encode_matches_bruteforce_nearest_with_ties_to_even():
    r = np.random.default_rng(3)
    xs = list(r.standard_normal(300) * 30) + list(r.uniform(-0.03, 0.03, 200))
    # every midpoint between neighbouring values, both signs
    v = fp8.decode(np.arange(0x7F, dtype=np.uint8))
    mids = (v[:-1] + v[1:]) / 2
    xs += list(mids) + list(-mids) + [447.9, 449.0, 463.9, 464.0, 1e6, -1e6]
    for x in xs:
        x32 = np.float32(x)
        assert int(fp8.encode(x32)) == _nearest_bruteforce(float(x32)), x


def test_ties_and_saturation_cases():
    assert fp8.encode(np.float32(1.0625)) == 0x38      # between 1.0 (m 0) and 1.125 (m 1)
    assert fp8.encode(np.float32(1.1875)) == 0x3A      # between 1.125 (m 1) and 1.25 (m 2)
    assert fp8.encode(np.float32(2.0 ** -10)) == 0x00  # half the smallest subnormal
    assert fp8.encode(np.float32(3 * 2.0 ** -10)) == 0x02
    assert fp8.encode(np.float32(15.5 * 2.0 ** -10)) == 0x08  # rounds up into the normals
    assert fp8.encode(np.float32(460.0)) == 0x7E and fp8.encode(np.float32(-1e30)) == 0xFE


def test_quantize_rows_scales_each_row_to_448():
    r = np.random.default_rng(4)
    w = r.standard_normal((16, 256)) * np.logspace(-3, 1, 16)[:, None]
    w[3] = 0.0
    w = w.astype(np.float32).astype(np.float64)
    q, s = fp8.quantize_rows(w)
    assert q.dtype == np.uint8 and s.dtype == np.float32
    assert s[3] == 1.0 and np.all(q[3] == 0)
    for i in range(16):
        if i == 3:
            continue
        j = np.argmax(np.abs(w[i]))
        assert q[i, j] in (0x7E, 0xFE)
        assert s[i] == np.float32(np.max(np.abs(w[i]))) / np.float32(448.0)
    # relative error of normal codes at most half a mantissa step (2^-4), absolute error of
    # subnormal codes at most half the subnormal spacing
    d = fp8.dequantize_rows(q, s)
    x = np.abs(w) / s[:, None]
    nor = x >= 2.0 ** -6
    assert np.all(np.abs(d - w)[nor] <= (2.0 ** -4 * np.abs(w) + 1e-30)[nor] * (1 + 1e-6))
    assert np.all((np.abs(d - w) / s[:, None])[~nor] <= 2.0 ** -10 * (1 + 1e-6))


def test_dequantize_experts_touches_only_the_routed_experts():
    r = np.random.default_rng(5)
    lw = {"w_gate": r.standard_normal((2, 8, 32)), "w_up": r.standard_normal((2, 8, 32)),
          "w_down": r.standard_normal((2, 32, 8)), "ws_gate": r.standard_normal((16, 32)),
          "w_router": r.standard_normal((2, 32))}
    out = fp8.dequantize_experts(lw)
    assert out["ws_gate"] is lw["ws_gate"] and out["w_router"] is lw["w_router"]
    for k in ("w_gate", "w_up", "w_down"):
        assert out[k].shape == lw[k].shape and not np.array_equal(out[k], lw[k])
        q, s = fp8.quantize_rows(lw[k].reshape(-1, lw[k].shape[-1]))
        assert np.array_equal(out[k].reshape(-1, lw[k].shape[-1]), fp8.dequantize_rows(q, s))
