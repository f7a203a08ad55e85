"""Pins of the oracle's codecs and quantisers against the format definitions, the pages'
numbers and exact rational brute force (no GPU)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import csa2_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------- codecs ----------------

def test_e2m1_grid():
    # OCP MX E2M1: {0, 0.5, 1, 1.5, 2, 3, 4, 6} and their negatives (code 8 = -0)
    assert list(O.E2M1[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(O.E2M1[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert math.copysign(1.0, O.E2M1[8]) == -1.0


def test_e4m3_table():
    v = O.E4M3
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2                      # no infinities, two NaNs
    finite_pos = v[:0x7F]
    assert np.all(np.diff(finite_pos) > 0)             # monotone codes
    assert finite_pos[0] == 0 and finite_pos[1] == 2.0 ** -9   # smallest subnormal
    assert finite_pos[8] == 2.0 ** -6                   # smallest normal
    assert finite_pos[-1] == 448.0                      # largest finite
    assert v[0x38] == 1.0
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])


def test_e8m0_table():
    assert O.E8M0[127] == 1.0 and O.E8M0[0] == 2.0 ** -127 and O.E8M0[254] == 2.0 ** 127
    assert np.isnan(O.E8M0[255])


def test_pages_range_2688():
    g = _load("pages_constants.json")["fp4_range"]
    a, b = g["factors"]
    assert a == np.nanmax(O.E4M3) and b == O.E2M1.max()
    # every E2M1 x E4M3 product, maximum magnitude
    prods = np.abs(O.E2M1[:, None] * O.E4M3[None, :0x7F])
    assert prods.max() == g["value"] == a * b


def _bf16_exact(x):
    f = np.asarray(x, np.float32)
    return np.all(f.astype(np.float64) == x) and np.all((f.view(np.uint32) & 0xFFFF) == 0)


def test_dequant_exact_in_bf16_fp16_fp32():
    # every main-KV dequantised value (E2M1 x E4M3) and every SWA value (E4M3) is exactly
    # representable in bf16, fp16 and fp32
    prods = (O.E2M1[:, None] * O.E4M3[None, :0x7F]).reshape(-1)
    for vals in (prods, O.E4M3[:0x7F]):
        assert _bf16_exact(vals)
        assert np.all(vals.astype(np.float16).astype(np.float64) == vals)


# ---------------- exact brute force for rounding ----------------

def _nearest_exact(x: Fraction, grid):
    """grid: list of (Fraction value, code) non-negative ascending; ties to even code."""
    best = None
    for val, code in grid:
        d = abs(x - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


E2M1_GRID = [(Fraction(O.E2M1[c]), c) for c in range(8)]
E4M3_GRID = [(Fraction(O.E4M3[c]), c) for c in range(0x7F)]


def _nvfp4_exact(group):
    xs = [Fraction(float(v)) for v in group]
    amax = max(abs(v) for v in xs)
    sc = _nearest_exact(amax / 6, E4M3_GRID)
    s = Fraction(O.E4M3[sc])
    codes = []
    for v, fv in zip(xs, group):
        mag = 0 if s == 0 else _nearest_exact(abs(v) / s, E2M1_GRID)
        codes.append(mag | (8 if math.copysign(1.0, fv) < 0 else 0))
    return sc, codes


def _adversarial_groups(rng, n):
    """Groups whose amax/6 and whose element ratios sit on or 1 ulp beside the midpoints."""
    groups = []
    mids_e4m3 = [(O.E4M3[c] + O.E4M3[c + 1]) / 2 for c in range(0x7E)]
    t = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for _ in range(n):
        m = mids_e4m3[rng.integers(len(mids_e4m3))]
        amax = np.float32(6 * m)
        amax = [amax, np.nextafter(amax, np.float32(0)), np.nextafter(amax, np.float32(1e9))][rng.integers(3)]
        g = np.zeros(16, np.float32)
        g[0] = amax
        # resulting scale, elements near s*t
        sc = _nearest_exact(Fraction(float(amax)) / 6, E4M3_GRID)
        s = O.E4M3[sc]
        for i in range(1, 16):
            v = np.float32(s * t[rng.integers(len(t))]) if s > 0 else np.float32(rng.normal())
            v = [v, np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(1e9))][rng.integers(3)]
            g[i] = v if rng.random() < 0.5 else -v
        rng.shuffle(g)
        groups.append(g)
    return groups


def test_nvfp4_quantizer_matches_exact_rational_bruteforce():
    rng = np.random.default_rng(7)
    groups = _adversarial_groups(rng, 300)
    groups += [rng.normal(size=16).astype(np.float32) * np.float32(10 ** rng.uniform(-4, 3))
               for _ in range(200)]
    x = np.stack(groups)
    codes, scales = O.quantize_nvfp4(x)
    unpacked = O.unpack_nibbles(codes)
    for i, g in enumerate(groups):
        sc, cs = _nvfp4_exact(g)
        assert scales[i, 0] == sc, (i, g)
        assert list(unpacked[i]) == cs, (i, g)


def test_nvfp4_hand_examples():
    for case in _load("hand_quant.json")["nvfp4"]:
        x = np.zeros((1, 16), np.float32)
        x[0, : len(case["x"])] = case["x"]
        codes, scales = O.quantize_nvfp4(x)
        assert scales[0, 0] == case["scale"], case["why"]
        assert list(O.unpack_nibbles(codes)[0, : len(case["codes"])]) == case["codes"], case["why"]


def test_nvfp4_packing_order():
    # channel 2i in the low nibble of byte i
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1] = 6.0, -3.0
    codes, _ = O.quantize_nvfp4(x)
    assert codes[0, 0] == (7 | (13 << 4))


def test_mxfp4_hand_examples():
    for case in _load("hand_quant.json")["mxfp4"]:
        x = np.zeros((1, 32), np.float32)
        x[0, : len(case["x"])] = case["x"]
        codes, scales = O.quantize_mxfp4(x)
        assert scales[0, 0] == case["scale"], case["why"]
        assert list(O.unpack_nibbles(codes)[0, : len(case["codes"])]) == case["codes"], case["why"]


def _mxfp4_exact(group):
    xs = [Fraction(float(v)) for v in group]
    amax = max(abs(v) for v in xs)
    if amax == 0:
        e = -127
        code = 0
    else:
        e = 0
        while Fraction(2) ** (e + 1) <= amax:
            e += 1
        while Fraction(2) ** e > amax:
            e -= 1
        e = max(-127, min(127, e - 2))
        code = e + 127
    out = []
    for v, fv in zip(xs, group):
        mag = _nearest_exact(abs(v) / Fraction(2) ** e, E2M1_GRID)
        out.append(mag | (8 if math.copysign(1.0, fv) < 0 else 0))
    return code, out


def test_mxfp4_matches_ocp_rule_bruteforce():
    rng = np.random.default_rng(11)
    groups = []
    for _ in range(150):
        g = rng.normal(size=32).astype(np.float32) * np.float32(2.0 ** rng.integers(-20, 20))
        groups.append(g)
    for _ in range(150):   # powers of two and the (6, 8) * 2^E clip band
        E = int(rng.integers(-30, 30))
        g = (rng.choice([4.0, 6.0, 6.5, 7.0, 7.99, 2.0, 0.25, 0.75, 5.0, 3.5], size=32)
             * 2.0 ** E * rng.choice([-1, 1], size=32)).astype(np.float32)
        groups.append(g)
    x = np.stack(groups)
    codes, scales = O.quantize_mxfp4(x)
    un = O.unpack_nibbles(codes)
    for i, g in enumerate(groups):
        c, cs = _mxfp4_exact(g)
        assert scales[i, 0] == c
        assert list(un[i]) == cs


def test_fp8_hand_examples_and_bruteforce():
    case = _load("hand_quant.json")["fp8"][0]
    got = O.quantize_fp8(np.array(case["x"], np.float32))
    assert list(got) == case["codes"], case["why"]
    rng = np.random.default_rng(3)
    x = (rng.normal(size=400) * 10.0 ** rng.uniform(-4, 2.8, size=400)).astype(np.float32)
    got = O.quantize_fp8(x)
    for v, c in zip(x, got):
        mag = _nearest_exact(abs(Fraction(float(v))), E4M3_GRID)
        assert c == (mag | (0x80 if v < 0 else 0))


def test_quantize_dequant_roundtrip_on_grid():
    # values already on the grid are reproduced exactly (quantiser inverts the decoder)
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(64, 256), dtype=np.uint8)
    scales = rng.integers(0x20, 0x60, size=(64, 32), dtype=np.uint8)
    # force each group's max element to magnitude 6 so amax/6 is exactly the scale
    un = O.unpack_nibbles(codes)
    un[:, ::16] = 7
    codes = (un[:, 0::2] | (un[:, 1::2] << 4)).astype(np.uint8)
    x = O.dequant_nvfp4(codes, scales).astype(np.float32)
    c2, s2 = O.quantize_nvfp4(x)
    assert np.array_equal(s2, scales)
    # -0 and +0 dequantise alike; compare through the decoder
    assert np.array_equal(O.dequant_nvfp4(c2, s2), O.dequant_nvfp4(codes, scales))


def test_fp8_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    x = O.dequant_fp8(codes).astype(np.float32)
    assert np.array_equal(O.quantize_fp8(x), codes)
