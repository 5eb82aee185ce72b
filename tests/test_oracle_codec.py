"""Pins of the oracle's NVFP4 codec against things other than itself.

* the E2M1 codebook and E4M3 points printed in tests/golden (OCP definitions of
  the element and scale types named by "Replay the Curvature", Abstract);
* torch's float8_e4m3fn decode and its round-to-nearest-even cast;
* brute-force nearest search in exact rational arithmetic for E2M1 and for
  E4M3 quotients, including constructed exact ties.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_e2m1_codebook_matches_golden():
    for code, val in _read_golden("e2m1_codebook.txt"):
        got = float(codec.e2m1_value(code))
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e4m3_points_match_golden():
    for code, val in _read_golden("e4m3_points.txt"):
        got = float(codec.e4m3_decode(code))
        if np.isnan(val):
            assert np.isnan(got)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codec.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def _torch_e4m3_code(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().astype(np.int64)


def test_e4m3_rne_vs_torch_cast():
    r = np.random.default_rng(1)
    x = np.exp2(r.uniform(-12, 9, size=200000)).astype(np.float32)
    x = np.minimum(x, np.float32(448.0))
    # exact midpoints between consecutive codes and their fp32 neighbours
    pos = codec.E4M3_POS
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1e9)), pos.astype(np.float32),
                        np.array([0.0, 2.0 ** -10, 2.0 ** -11], dtype=np.float32)])
    got = codec.e4m3_rne(x.astype(np.float64))
    ref = _torch_e4m3_code(x)
    assert np.array_equal(got, ref)


def test_e4m3_saturates_instead_of_nan():
    assert int(codec.e4m3_rne(480.0)) == 0x7E
    assert int(codec.e4m3_rne(1e30)) == 0x7E


def _nearest_even_fraction(q, grid):
    """Brute force: index of the grid value nearest to rational q; ties -> even index."""
    best, bestd = None, None
    for i, gv in enumerate(grid):
        dist = abs(q - Fraction(gv))
        if bestd is None or dist < bestd or (dist == bestd and i % 2 == 0):
            best, bestd = i, dist
    return best


def test_e4m3_ratio_bruteforce_exact():
    r = np.random.default_rng(2)
    gs = r.uniform(0.5, 2.0, size=40).astype(np.float32) * np.float32(2.0 ** -8)
    grid = [float(v) for v in codec.E4M3_POS]
    for g in gs:
        den = 6.0 * float(g)
        # random numerators plus exact midpoint ties and their neighbours
        nums = list(r.uniform(0, 460 * den, size=30).astype(np.float32).astype(np.float64))
        for i in r.integers(0, 126, size=10):
            t = (grid[i] + grid[i + 1]) / 2 * den     # exact in fp64
            nums += [t, np.nextafter(t, 0), np.nextafter(t, 1e9)]
        for a in nums:
            want = _nearest_even_fraction(Fraction(a) / Fraction(den), grid)
            got = int(codec.e4m3_rne_ratio(a, den))
            assert got == want, (a, den, got, want)


def test_e2m1_encode_bruteforce_exact():
    r = np.random.default_rng(3)
    grid = [float(v) for v in codec.E2M1_MAG]
    for _ in range(300):
        g = np.float32(r.uniform(1e-4, 1e-2))
        sc = int(r.integers(1, 127))
        sval = float(codec.e4m3_decode(sc))
        S = Fraction(sval) * Fraction(float(g))
        vals = list(r.normal(0, 3 * float(S), size=8).astype(np.float32))
        for i in range(7):
            mid = (grid[i] + grid[i + 1]) / 2 * sval * float(g)   # exact in fp64
            vals += [mid, -mid, np.nextafter(mid, 0.0), np.nextafter(mid, 1.0)]
        vals += [10 * float(S), -7 * float(S), 0.0, -0.0]
        for v in vals:
            got = int(codec.e2m1_encode(v, sval, g))
            idx = _nearest_even_fraction(abs(Fraction(float(v))) / S, grid)
            sign = 1 if (v < 0 and idx > 0) else 0
            assert got == (sign << 3 | idx), (v, sval, g, got, idx)


def test_grid_points_encode_to_themselves():
    g = np.float32(0.00123)
    for sc in (1, 7, 8, 56, 100, 126):
        sval = float(codec.e4m3_decode(sc))
        for i, m in enumerate(codec.E2M1_MAG):
            v = m * sval * float(g)
            assert int(codec.e2m1_encode(v, sval, g)) == i
            if i:
                assert int(codec.e2m1_encode(-v, sval, g)) == (8 | i)


def test_pack_unpack_roundtrip_and_nibble_order():
    r = np.random.default_rng(4)
    c = r.integers(0, 16, size=(5, 32)).astype(np.uint8)
    p = codec.pack_codes(c)
    assert p.shape == (5, 16)
    assert np.array_equal(p & 0xF, c[:, 0::2])
    assert np.array_equal(p >> 4, c[:, 1::2])
    assert np.array_equal(codec.unpack_codes(p), c)


def test_dequant_is_single_rounding_of_exact_product():
    r = np.random.default_rng(5)
    codes = r.integers(0, 16, size=(4, 64)).astype(np.uint8)
    scales = r.integers(1, 127, size=(4, 4)).astype(np.uint8)
    g = np.float32(r.uniform(1e-5, 1e-3))
    out = codec.dequantize(codec.pack_codes(codes), scales, g)
    for i in range(4):
        for j in range(64):
            exact = Fraction(float(codec.e2m1_value(codes[i, j]))) * \
                Fraction(float(codec.e4m3_decode(scales[i, j // 16]))) * Fraction(float(g))
            assert out[i, j] == np.float32(float(exact))   # float(Fraction) rounds once


def test_global_scale():
    r = np.random.default_rng(6)
    W = r.normal(0, 0.02, size=(64, 64)).astype(np.float32)
    g = codec.global_scale(W)
    amax = float(np.max(np.abs(W)))
    assert g == np.float32(Fraction(amax) / 2688)
    # the block holding amax gets an in-range scale code
    assert int(codec.e4m3_rne_ratio(amax, 6.0 * float(g))) <= 0x7E
    assert codec.global_scale(np.zeros((4, 16), np.float32)) == np.float32(1.0)
