"""Pins for the oracle's FP8 formats and quantizers (CPU only).

Each pin ties the oracle to something other than itself: torch's float8 dtypes,
values fixed by the format definitions (tests/golden), brute-force search, exact
rational arithmetic, or properties of correct rounding."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8


def _golden(path):
    rows = []
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            rows.append(line.split())
    return rows


def test_e4m3_table_matches_torch_float8_e4m3fn():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(t), np.isnan(fp8.E4M3_TABLE))
    fin = ~np.isnan(t)
    assert np.array_equal(t[fin], fp8.E4M3_TABLE[fin])
    assert np.array_equal(np.signbit(t[fin]), np.signbit(fp8.E4M3_TABLE[fin]))
    assert fin.sum() == 254


def test_e4m3_golden_values(golden_dir):
    for code, value in _golden(os.path.join(golden_dir, "e4m3_values.txt")):
        c = int(code, 16)
        got = fp8.E4M3_TABLE[c]
        if value == "nan":
            assert math.isnan(got)
        else:
            assert got == float(value) and math.copysign(1, got) == math.copysign(1, float(value)), code


def test_e4m3_order_and_symmetry():
    pos = fp8.E4M3_TABLE[:127]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(fp8.E4M3_TABLE[128:255], -pos)


def test_e8m0_table_matches_torch_and_golden(golden_dir):
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(np.isnan(t), np.isnan(fp8.E8M0_TABLE))
    fin = ~np.isnan(t)
    assert np.array_equal(t[fin], fp8.E8M0_TABLE[fin])
    for code, lg in _golden(os.path.join(golden_dir, "e8m0_values.txt")):
        v = fp8.E8M0_TABLE[int(code)]
        assert math.isnan(v) if lg == "nan" else v == 2.0 ** int(lg)


def _brute_encode(y):
    """Nearest finite code by exhaustive search; ties to the even code; saturating."""
    y = float(y)
    neg = math.copysign(1.0, y) < 0
    a = min(abs(y), 448.0)
    best = None
    for c in range(127):
        d = abs(fp8.e4m3_value(c) - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if neg else 0)


def _encode_samples():
    pos = fp8.E4M3_TABLE[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    rng = np.random.default_rng(7)
    rnd = (rng.standard_normal(3000) * rng.choice([1e-4, 1e-2, 1, 30, 300, 600], 3000)).astype(np.float32)
    extra = np.array([0, 448, 449, 463.99, 464, 465, 1e4, 3e38, 2.0 ** -10, 2.0 ** -11, 1e-42], np.float32)
    x = np.concatenate([pos.astype(np.float32), mids, up, dn, rnd, extra])
    return np.concatenate([x, -x]).astype(np.float64)


def test_encode_matches_brute_force():
    x = _encode_samples()
    got = fp8.encode_e4m3(x)
    want = np.array([_brute_encode(v) for v in x], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_encode_matches_torch_cast_in_range():
    x = _encode_samples()
    x = x[np.abs(x) <= 448].astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode_e4m3(x.astype(np.float64)), t)


def test_encode_golden(golden_dir):
    for value, code in _golden(os.path.join(golden_dir, "e4m3_encode.txt")):
        v = float(np.float32(float(value)))
        assert fp8.encode_e4m3(np.array([v]))[0] == int(code, 16), value


def test_encode_round_trip_all_codes():
    codes = np.array([c for c in range(256) if c not in fp8.E4M3_NAN_CODES], dtype=np.uint8)
    for s in [1.0, 2.0 ** -7, 0.0123, 3.7, 1e-3, 250.0]:
        s32 = float(np.float32(s))
        y = fp8.to_fp32(fp8.dequant_fp32(codes, s32) / s32)
        assert np.array_equal(fp8.encode_e4m3(y), codes), s


def test_encode_rejects_nan():
    with pytest.raises(ValueError):
        fp8.encode_e4m3(np.array([np.nan]))


def test_fp32_scale_is_correctly_rounded_quotient():
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(400).astype(np.float32)) * np.float32(10.0)
    s = fp8.fp32_scale_from_amax(amax.astype(np.float64))
    for a, si in zip(amax, s):
        exact = Fraction(float(a)) / 448
        got = Fraction(float(si))
        assert float(np.float32(si)) == si
        for nb in (np.nextafter(np.float32(si), np.float32(np.inf)), np.nextafter(np.float32(si), np.float32(0))):
            assert abs(got - exact) <= abs(Fraction(float(nb)) - exact)
    assert fp8.fp32_scale_from_amax(0.0) == 1.0
    assert fp8.fp32_scale_from_amax(448.0) == 1.0


def _brute_e8m0(amax):
    if amax == 0:
        return 127
    k = -200
    while not (amax <= 448.0 * 2.0 ** k):
        k += 1
    return min(max(k + 127, 0), 254)


def test_e8m0_code_matches_search():
    rng = np.random.default_rng(5)
    a = np.concatenate([np.abs(rng.standard_normal(300)) * 10.0 ** rng.integers(-30, 30, 300),
                        448.0 * 2.0 ** np.arange(-20, 20), 448.0 * 2.0 ** np.arange(-20, 20) * (1 + 2 ** -20),
                        [0.0, 1e-300, 1e300, 448.0, 449.0, 224.0, 224.0001]])
    got = fp8.e8m0_code_from_amax(a)
    want = np.array([_brute_e8m0(float(v)) for v in a])
    assert np.array_equal(got, want)


def test_quantize_fp32_block_maps_amax_to_448_and_bounds_error():
    rng = np.random.default_rng(11)
    for trial in range(20):
        x = fp8.to_fp32(rng.standard_normal((16, 64)) * 10.0 ** rng.uniform(-3, 3))
        codes, s = fp8.quantize_fp32_block(x)
        i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert codes[i] in (0x7E, 0xFE)
        xh = fp8.dequant(codes, s)
        # RNE error <= half the E4M3 spacing at |x|/s (2^-4 relative for normals,
        # 2^-10 absolute below 2^-6), plus the fp32 rounding of x/s.
        y = np.abs(x) / s
        half_step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 4), 2.0 ** -10)
        assert np.all(np.abs(xh - x) <= (half_step * (1 + 2 ** -20) + y * 2 ** -23) * s)


def test_quantize_e8m0_groups_use_smallest_power_of_two():
    rng = np.random.default_rng(12)
    x = fp8.to_fp32(rng.standard_normal((8, 128)) * 10.0 ** rng.uniform(-3, 3, (8, 1)))
    codes, u = fp8.quantize_e8m0_g32(x)
    assert codes.shape == x.shape and u.shape == (8, 4)
    g = np.abs(x).reshape(8, 4, 32).max(axis=-1)
    sc = fp8.E8M0_TABLE[u]
    assert np.all(g <= 448 * sc) and np.all(g > 224 * sc)
    xh = fp8.dequant(codes, np.repeat(sc, 32, axis=-1))
    assert np.all(np.abs(xh - x) <= np.abs(x) * 2 ** -4 + np.repeat(sc, 32, axis=-1) * 2 ** -10)
