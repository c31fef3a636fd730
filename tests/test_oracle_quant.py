"""Pins of the oracle's per-token / per-token-group quantizer.

Pinned by: hand-worked examples (tests/golden/quant_worked_examples.txt),
properties the definition implies (absmax maps to +-448, power-of-two scale
invariance, reconstruction bound, per-token == one group per row, row padding
leaves the first M rows unchanged), and brute force with exact rationals on
small rows.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS32 = np.float32(1e-10)


def _bf16(a):
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).float().numpy()


def _worked_examples():
    rows = []
    with open(os.path.join(GOLDEN, "quant_worked_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            g, vals, sbits, codes = [p.strip() for p in line.split("|")]
            rows.append((int(g), [float(v) for v in vals.split()], sbits,
                         [int(c, 16) for c in codes.split()]))
    return rows


def test_worked_examples():
    ex = _worked_examples()
    assert len(ex) == 4
    for g, vals, sbits, codes in ex:
        x = np.array([vals], dtype=np.float32)
        assert np.array_equal(_bf16(x), x), "fixture values must be bf16-exact"
        q, s = oracle.quant_per_token_group(x, g)
        assert [int(c) for c in q[0]] == codes
        if sbits == "EPS":
            want = np.float32(EPS32 / np.float32(448))
        else:
            want = np.array([int(sbits, 16)], dtype=np.uint32).view(np.float32)[0]
        assert s[0, 0].view(np.uint32) == np.float32(want).view(np.uint32)


def test_eps_value():
    # eps = 1e-10 as an fp32 constant (PR 27896 digest, "Key source excerpts")
    assert float(EPS32) == 1.0000000133514320e-10


def _brute_group(vals):
    """Exact-rational reference of one group: scale and codes.

    The fp32 steps are modelled as exact rationals rounded once to fp32 with
    round-half-even, and the E4M3 step as nearest-even over the finite values
    listed by torch's decode, so nothing here reuses the oracle's code.
    """
    def rn_f32(fr: Fraction) -> Fraction:
        # round a positive-or-zero rational to fp32, ties to even
        if fr == 0:
            return fr
        sign = -1 if fr < 0 else 1
        a = abs(fr)
        e = a.numerator.bit_length() - a.denominator.bit_length()
        while Fraction(2) ** e > a:
            e -= 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        e = max(e, -126)
        ulp = Fraction(2) ** (e - 23)
        q = a / ulp
        fl = q.numerator // q.denominator
        rem = q - fl
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
            fl += 1
        return sign * fl * ulp

    finite = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist()
    finite = [Fraction(v) for v in finite]

    def e4m3(fr: Fraction) -> int:
        neg = fr < 0 or (fr == 0 and False)
        a = min(abs(fr), Fraction(448))
        best = None
        for code, v in enumerate(finite):
            d = abs(v - a)
            if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
                best = (d, code)
        return best[1] | (0x80 if neg else 0)

    fx = [Fraction(float(v)) for v in vals]
    amax = max(abs(v) for v in fx)
    amax = max(amax, Fraction(float(EPS32)))
    s = rn_f32(amax / 448)
    codes = [e4m3(rn_f32(v / s)) for v in fx]
    return s, codes


def test_brute_force_small_rows():
    x = synth.activations("pin-brute", 6, 32).float().numpy()
    x[1] *= 1e-3
    x[2, :] = 0.0
    x[3, 5] = 300.0
    q, s = oracle.quant_per_token_group(x, 16)
    for r in range(x.shape[0]):
        for g in range(2):
            seg = x[r, g * 16:(g + 1) * 16]
            bs, bcodes = _brute_group(seg)
            assert Fraction(float(s[r, g])) == bs
            # brute force does not model -0: compare sign only where non-zero
            got = [int(c) for c in q[r, g * 16:(g + 1) * 16]]
            want = [c if not (c == 0 and v < 0) else 0x80 for c, v in zip(bcodes, seg)]
            assert got == want, (r, g)


def test_absmax_maps_to_448():
    x = synth.activations("pin-absmax", 64, 512).float().numpy()
    for G in (16, 32, 64, 128, 512):
        q, s = oracle.quant_per_token_group(x, G)
        xg = x.reshape(64, -1, G)
        qg = q.reshape(64, -1, G)
        idx = np.argmax(np.abs(xg), axis=2)
        top = np.take_along_axis(qg, idx[..., None], axis=2)[..., 0]
        assert np.all((top & 0x7F) == 0x7E)
        sign = np.take_along_axis(xg, idx[..., None], axis=2)[..., 0] < 0
        assert np.array_equal((top >> 7).astype(bool), sign)


def test_power_of_two_scaling_invariance():
    x = synth.activations("pin-pow2", 16, 256).float().numpy()
    q0, s0 = oracle.quant_per_token_group(x, 128)
    for j in (-20, -3, 1, 7, 30):
        q1, s1 = oracle.quant_per_token_group(x * np.float32(2.0 ** j), 128)
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, s0 * np.float32(2.0 ** j))


def test_reconstruction_bound():
    x = synth.activations("pin-recon", 32, 1024).float().numpy()
    q, s = oracle.quant_per_token_group(x, 128)
    dec = oracle.decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(dec - x)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    normal = np.abs(x) / srep >= 2.0 ** -6
    # 3 mantissa bits: half an ulp is 2^-4 relative; plus the fp32 division's rounding
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -20) * np.abs(x[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * srep[~normal] * (1 + 2.0 ** -20))


def test_per_token_is_one_group_per_row():
    x = synth.activations("pin-pt", 8, 384).float().numpy()
    q1, s1 = oracle.quant_per_token(x)
    q2, s2 = oracle.quant_per_token_group(x, 384)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2[:, 0])


def test_rows_are_independent():
    # row padding (PR 27896 digest, "Implementation"/"Risks and impact"):
    # quantizing the first M rows alone equals the first M rows of a larger batch
    x = synth.activations("pin-rows", 256, 256).float().numpy()
    qa, sa = oracle.quant_per_token_group(x, 128)
    for m in (1, 2, 3, 4, 5, 7, 13, 16, 31, 64, 256):
        qm, sm = oracle.quant_per_token_group(x[:m], 128)
        assert np.array_equal(qm, qa[:m]) and np.array_equal(sm, sa[:m])


@pytest.mark.parametrize("m,ra,want", [(0, 4, 0), (1, 4, 4), (3, 4, 4), (4, 4, 4), (5, 4, 8),
                                       (13, 4, 16), (31, 4, 32), (7, 1, 7), (7, 8, 8)])
def test_padded_rows(m, ra, want):
    assert oracle.padded_rows(m, ra) == want


def test_scales_col_major_layout():
    s = np.arange(6, dtype=np.float32).reshape(3, 2)  # M=3, 2 groups
    flat = oracle.scales_col_major(s, 4)
    assert flat.shape == (8,)
    assert list(flat[[0, 1, 2, 4, 5, 6]]) == [0, 2, 4, 1, 3, 5]
    assert np.isnan(flat[3]) and np.isnan(flat[7])


def test_weight_blockwise_matches_group_quant_for_single_row_blocks():
    # with block_n = 1 the 2-D block quant is the per-token-group quant
    w = synth.weights("pin-wblk", 8, 256).numpy()
    q1, s1 = oracle.quant_weight_blockwise(w, block_n=1, block_k=128)
    q2, s2 = oracle.quant_per_token_group(w, 128)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_weight_blockwise_block_absmax():
    w = synth.weights("pin-wblk2", 256, 384).numpy()
    q, s = oracle.quant_weight_blockwise(w)
    assert s.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            t = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert s[i, j] == np.float32(np.float32(np.abs(t).max()) / np.float32(448))
            assert np.sum((q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] & 0x7F) == 0x7E) >= 1
