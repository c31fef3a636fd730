"""Pins of the oracle's E4M3 codec against the format definition and torch.

The codec must agree with (a) hand-written landmark values of the OCP E4M3
format, (b) torch's independent ``float8_e4m3fn`` decode of all 256 codes and
(c) torch's round-to-nearest-even conversion after clamping to +-448, on every
rounding boundary (midpoints and their fp32 neighbours) of every binade, plus
random fp32 values.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _landmarks():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_landmarks.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, val = line.split()
            rows.append((int(code, 16), val))
    return rows


def test_landmark_values():
    table = oracle.decode_table()
    rows = _landmarks()
    assert len(rows) >= 20
    for code, val in rows:
        got = table[code]
        if val == "nan":
            assert np.isnan(got), hex(code)
        elif val == "-0":
            assert got == 0 and np.signbit(got), hex(code)
        else:
            assert Fraction(got) == Fraction(val), (hex(code), got, val)


def test_decode_matches_torch_all_codes():
    ours = oracle.decode_table()
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(theirs))
    assert list(np.nonzero(nan_ours)[0]) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan_ours], theirs[~nan_ours])
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(theirs[~nan_ours]))


def test_decode_structure():
    t = oracle.decode_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "non-negative codes must be strictly increasing"
    assert len(set(pos.tolist())) == 127
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])
    assert pos.max() == 448.0 == oracle.E4M3_MAX
    # top binade 256..448 in steps of 32
    assert list(pos[0x78:0x7F]) == [256, 288, 320, 352, 384, 416, 448]


def _torch_encode(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    t = torch.clamp(t, -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_roundtrip_all_finite_codes():
    t = oracle.decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert np.array_equal(oracle.encode(t[codes].astype(np.float32)), codes)


def test_encode_midpoints_ties_to_even_and_neighbours():
    t = oracle.decode_table()[:0x7F]
    lo, hi = t[:-1], t[1:]
    mids = ((lo + hi) / 2).astype(np.float32)  # midpoints are exact in fp32
    assert np.array_equal(mids.astype(np.float64), (lo + hi) / 2)
    codes_lo = np.arange(0, 0x7E)
    got = oracle.encode(mids)
    want = np.where(codes_lo % 2 == 0, codes_lo, codes_lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    assert np.array_equal(oracle.encode(up), (codes_lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.encode(dn), codes_lo.astype(np.uint8))
    for arr in (mids, up, dn, -mids, -up, -dn):
        assert np.array_equal(oracle.encode(arr), _torch_encode(arr))


def test_encode_specific_cases():
    # (value, code) pairs; a list because 0.0 and -0.0 are equal dict keys
    cases = [
        (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
        (432.0, 0x7E), (449.0, 0x7E), (1e30, 0x7E), (-1e30, 0xFE), (-1e-6, 0x80),
        (-0.0, 0x80), (0.0, 0x00), (464.0, 0x7E), (464.5, 0x7E), (480.0, 0x7E),
    ]
    v = np.array([c[0] for c in cases], dtype=np.float32)
    assert [int(c) for c in oracle.encode(v)] == [c[1] for c in cases]


def test_encode_matches_torch_bit_patterns():
    # every sign/exponent/top-3-mantissa combination crossed with low-bit
    # patterns that sit on and around every possible rounding position
    hi = np.arange(1 << 12, dtype=np.uint32) << 20  # sign, 8 exp bits, 3 mantissa bits
    lows = {0, (1 << 20) - 1}
    for b in range(20):
        lows |= {1 << b, (1 << b) - 1, (1 << b) + 1, (1 << 20) - (1 << b)}
    low = np.array(sorted(lows), dtype=np.uint32)
    bits = (hi[:, None] | low[None, :]).ravel()
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(oracle.encode(v), _torch_encode(v))


def test_encode_matches_torch_random():
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(oracle.encode(v), _torch_encode(v))
    w = rng.uniform(-500, 500, size=2_000_000).astype(np.float32)
    assert np.array_equal(oracle.encode(w), _torch_encode(w))


@pytest.mark.skipif(os.environ.get("FP8_ORACLE_EXHAUSTIVE") != "1",
                    reason="exhaustive sweep of all 2^32 fp32 patterns; set FP8_ORACLE_EXHAUSTIVE=1")
def test_encode_exhaustive_fp32():
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        bits = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        v = bits.view(np.float32)
        v = v[np.isfinite(v)]
        assert np.array_equal(oracle.encode(v), _torch_encode(v)), hex(start)
