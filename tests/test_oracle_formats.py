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


def _rows_in_both_indexer_formats(rng, rows, d=128):
    """Rows that MXFP4 and the NVFP4-style format both hold exactly, with the same values:
    each 32-channel block is E2M1 grid values times one power of two 2^e (e within both
    scale ranges), and each 16-channel half holds a +-6 * 2^e element, so the per-32 E8M0
    rule and the per-16 amax/6 E4M3 rule both pick the scale 2^e."""
    grid = np.array([O.e2m1_value(c) for c in range(16)])
    x = rng.choice(grid, size=(rows, d))
    x[:, ::16] = rng.choice([-6.0, 6.0], size=(rows, d // 16))
    e = rng.integers(-6, 5, size=(rows, d // 32))
    return x * np.ldexp(1.0, np.repeat(e, 32, axis=1))


def test_indexer_formats_lossless_on_shared_grid():
    """[W] "FP4 与 SWA Bounded Replay": the indexer in FP4, either scale format.  On rows both
    formats represent, each round trip is exact and the two layouts differ only in their
    scale arrays (4 E8M0 bytes per 128 channels against 8 E4M3 bytes)."""
    rng = np.random.default_rng(41)
    x = _rows_in_both_indexer_formats(rng, 50)
    for fmt, n_sc in (("mxfp4", 4), ("nvfp4", 8)):
        codes, scales = O.quantize_indexer(x, fmt)
        assert codes.shape == (50, 64) and scales.shape == (50, n_sc)
        assert np.array_equal(O.dequant_indexer(codes, scales, fmt), x)
    mx, nv = O.quantize_indexer(x, "mxfp4"), O.quantize_indexer(x, "nvfp4")
    assert np.array_equal(mx[0], nv[0])        # same E2M1 codes, different scales
    with pytest.raises(ValueError):
        O.quantize_indexer(x, "fp8")


def test_indexer_scores_nvfp4_closed_form():
    """Scores over an NVFP4 indexer cache: on shared-grid rows they equal the MXFP4 scores
    and the definition sum_h w_h * max(0, q_h . k_j) evaluated term by term in exact
    rationals; on general rows they follow the NVFP4 dequantised values (which differ from
    the MXFP4 ones there)."""
    rng = np.random.default_rng(42)
    H, n = 4, 30
    qx = _rows_in_both_indexer_formats(rng, H)
    kx = _rows_in_both_indexer_formats(rng, n)
    w = rng.uniform(size=H)
    res = {}
    for fmt in ("mxfp4", "nvfp4"):
        kc, ks = O.quantize_indexer(kx, fmt)
        qc, qs = O.quantize_indexer(qx, fmt)
        caches = O.PackedCaches(None, None, kc, ks, index_fmt=fmt)
        res[fmt] = O.full_scores(qc, qs, w, caches, n)[1]
    for j in range(n):
        exact = sum(Fraction(float(w[h])) * max(Fraction(0), sum(Fraction(float(a)) * Fraction(float(b))
                                                                 for a, b in zip(qx[h], kx[j])))
                    for h in range(H))
        assert res["nvfp4"][j] == res["mxfp4"][j]
        assert abs(Fraction(float(res["nvfp4"][j])) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
    # general rows: per-16 E4M3 scales hold values the per-32 power-of-two scales cannot
    g = rng.normal(size=(8, 128))
    mx = O.dequant_indexer(*O.quantize_indexer(g, "mxfp4"), "mxfp4")
    nv = O.dequant_indexer(*O.quantize_indexer(g, "nvfp4"), "nvfp4")
    assert not np.array_equal(mx, nv)
    assert np.abs(nv - g).mean() < np.abs(mx - g).mean()
    kc, ks = O.quantize_indexer(g, "nvfp4")
    caches = O.PackedCaches(None, None, kc, ks, index_fmt="nvfp4")
    qc, qs = O.quantize_indexer(g[:2], "nvfp4")
    qd = O.dequant_nvfp4(qc, qs)
    got = O.full_scores(qc, qs, np.array([0.5, 2.0]), caches, 8)[1]
    want = [0.5 * max(0.0, math.fsum(qd[0] * nv[j])) + 2.0 * max(0.0, math.fsum(qd[1] * nv[j])) for j in range(8)]
    assert np.allclose(got, want, rtol=1e-13, atol=1e-12)
