"""Pins of the oracle's quantizer variants: SiLU-and-mul fused in front of the
quantizer, UE8M0 (power-of-two) scales, and static per-tensor quantization.

The pages name these without a body (PR 27896 digest, "Key source excerpts":
the quantizer's kernel call carries fuse_silu_and_mul and scale_ue8m0 flags;
PR 31340 digest, "Implementation": a static FP8 quantization kernel). Pinned by
hand-worked examples (tests/golden/quant_variants_worked_examples.txt), by
library routines for the special functions (scipy's expit, torch's bf16 and
float8 conversions), by exact rational arithmetic, and by invariants that tie
each variant to the plain quantizer.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from fp8_w8a8_quantized_token_amd import synth

from test_oracle_quant import _brute_group

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(v):
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def _examples():
    rows = []
    with open(os.path.join(GOLDEN, "quant_variants_worked_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            kind, g, vals, sbits, codes = [p.strip() for p in line.split("|")]
            rows.append((kind, None if g == "-" else int(g), [float(v) for v in vals.split()],
                         int(sbits, 16), [int(c, 16) for c in codes.split()]))
    return rows


def _torch_bf16(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16).float().numpy()


# ---------------------------------------------------------------- worked examples
def test_worked_examples():
    ex = _examples()
    assert [e[0] for e in ex].count("silu") == 2
    assert [e[0] for e in ex].count("ue8m0") == 2
    assert [e[0] for e in ex].count("static") == 2
    for kind, g, vals, sbits, codes in ex:
        x = np.array([vals], dtype=np.float32)
        assert np.array_equal(_torch_bf16(x), x), "fixture values must be bf16-exact"
        if kind == "silu":
            q, s = oracle.silu_mul_quant_per_token_group(x, g)
            assert _bits(s[0, 0]) == sbits
        elif kind == "ue8m0":
            q, s = oracle.quant_per_token_group(x, g, scale_ue8m0=True)
            assert _bits(s[0, 0]) == sbits
        else:
            sc = np.array([sbits], np.uint32).view(np.float32)[0]
            q = oracle.quant_static(x, sc)
        assert [int(c) for c in q[0]] == codes, (kind, vals)


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_round_exact_matches_torch_on_fp32_values():
    # torch rounds fp32 -> bf16 to nearest even, subnormals included (values
    # that stay below the bf16 overflow threshold)
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 0x7F7F8000, size=200000, dtype=np.uint32)
    v = bits.view(np.float32)
    v = np.where(rng.random(v.shape) < 0.5, -v, v).astype(np.float32)
    mid = (np.arange(0, 0x7F7F, dtype=np.uint32) << 16) + 0x8000  # every bf16 midpoint
    v = np.concatenate([v, mid.view(np.float32), -mid.view(np.float32)])
    got = oracle.bf16_round_exact(v.astype(np.float64))
    want = _torch_bf16(v).astype(np.float64)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_bf16_round_exact_between_fp32_values():
    # fp64 values that fp32 cannot hold: just above / below a bf16 midpoint must
    # go up / down (rounding through fp32 first would land on the midpoint)
    base = np.array([1.0, 3.0, 2.0 ** -120, 2.0 ** -130, 1.5 * 2.0 ** 100], dtype=np.float64)
    _, e = np.frexp(base)
    step = np.ldexp(1.0, np.maximum(e, -125) - 8)
    mid = base + step / 2
    assert np.array_equal(oracle.bf16_round_exact(mid + step * 2.0 ** -40), base + step)
    assert np.array_equal(oracle.bf16_round_exact(mid - step * 2.0 ** -40), base)


# ---------------------------------------------------------------- SiLU-and-mul
def _bf16_grid():
    # every finite positive bf16 value from 2^-20 to 2^7 and their negatives
    b = np.arange(0x3580, 0x4300, dtype=np.uint32) << 16
    v = b.view(np.float32)
    return np.concatenate([v, -v, [0.0]]).astype(np.float32)


def test_silu_against_expit():
    # with up = 1 the oracle's y is bf16(silu(g)); scipy's expit is an
    # independent evaluation of the logistic function
    g = _bf16_grid()
    x = np.stack([g, np.ones_like(g)], axis=1)
    y = oracle.silu_mul_bf16(x)[:, 0].astype(np.float64)
    ref = g.astype(np.float64) * scipy.special.expit(g.astype(np.float64))
    want = oracle.bf16_round_exact(ref)
    assert np.array_equal(y, want)
    # and silu(g) - silu(-g) = g (sigma(g) + sigma(-g) = 1), before rounding
    assert np.allclose(ref - (-g) * scipy.special.expit(-g.astype(np.float64)), g, rtol=1e-15, atol=0)


def test_silu_special_values():
    k = 8
    up = synth.activations("pin-silu-up", 1, k).float().numpy()[0]
    gate = np.array([0.0, 64.0, -64.0, 1000.0, -1000.0, 0.0, 64.0, -0.0], np.float32)
    y = oracle.silu_mul_bf16(np.concatenate([gate, up])[None, :])[0]
    assert y[0] == 0 and y[5] == 0 and y[7] == 0
    assert y[1] == np.float32(64.0) * up[1] and y[6] == np.float32(64.0) * up[6]  # sigma(64) = 1 in bf16
    assert y[3] == np.float32(1000.0) * up[3] or y[3] == _torch_bf16(1000.0 * up[3])
    assert abs(y[2]) < 1e-25 and y[4] == 0  # silu(-64) ~ -1e-26; exp(1000) overflows to silu = -0


def test_silu_gate_is_first_half():
    m, k = 4, 64
    x = synth.activations("pin-silu-half", m, 2 * k).float().numpy()
    zg = x.copy()
    zg[:, :k] = 0.0
    assert np.all(oracle.silu_mul_bf16(zg) == 0)  # zero gate kills every output
    big = x.copy()
    big[:, :k] = 64.0
    assert np.array_equal(oracle.silu_mul_bf16(big), np.float32(64.0) * x[:, k:])


def test_silu_quant_brute_force():
    # silu by math.exp, bf16 by exact rational rounding, then the exact-rational
    # quantizer of one group: no oracle code involved
    import math

    def rn8(v):
        fr = Fraction(v)
        if fr == 0:
            return 0.0
        a = abs(fr)
        e = a.numerator.bit_length() - a.denominator.bit_length()
        while Fraction(2) ** e > a:
            e -= 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        ulp = Fraction(2) ** (max(e, -126) - 7)
        q = a / ulp
        fl = q.numerator // q.denominator
        rem = q - fl
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
            fl += 1
        return float((1 if fr > 0 else -1) * fl * ulp)

    m, k, G = 3, 32, 16
    x = synth.activations("pin-silu-brute", m, 2 * k).float().numpy()
    x[1] *= 4.0
    q, s = oracle.silu_mul_quant_per_token_group(x, G)
    for r in range(m):
        y = [rn8((g / (1.0 + math.exp(-g))) * u) for g, u in zip(x[r, :k].tolist(), x[r, k:].tolist())]
        for gi in range(k // G):
            seg = np.array(y[gi * G:(gi + 1) * G], np.float32)
            bs, bcodes = _brute_group(seg)
            assert Fraction(float(s[r, gi])) == bs
            got = [int(c) for c in q[r, gi * G:(gi + 1) * G]]
            want = [c if not (c == 0 and v < 0) else 0x80 for c, v in zip(bcodes, seg)]
            assert got == want, (r, gi)


def test_silu_per_token_is_one_group():
    x = synth.activations("pin-silu-pt", 5, 2 * 384).float().numpy()
    q1, s1 = oracle.silu_mul_quant_per_token(x)
    q2, s2 = oracle.silu_mul_quant_per_token_group(x, 384)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2[:, 0])


# ---------------------------------------------------------------- UE8M0 scales
def test_pow2_ceil_definition():
    rng = np.random.default_rng(3)
    bits = rng.integers(0x00800000, 0x7F000000, size=5000, dtype=np.uint32)
    vals = list(bits.view(np.float32)) + [np.float32(2.0 ** j) for j in range(-126, 127, 5)]
    for s in vals:
        p = oracle.pow2_ceil(s)
        assert int(np.array([p], np.float32).view(np.uint32)[0]) & 0x7FFFFF == 0  # no mantissa
        fs, fp = Fraction(float(s)), Fraction(float(p))
        assert fp / 2 < fs <= fp


def test_ue8m0_scales_and_codes():
    x = synth.activations("pin-ue8m0", 32, 512).float().numpy()
    x[3] *= 1e-3
    x[4] = 0.0
    for G in (16, 128):
        q0, s0 = oracle.quant_per_token_group(x, G)
        q1, s1 = oracle.quant_per_token_group(x, G, scale_ue8m0=True)
        assert np.array_equal(s1, np.vectorize(oracle.pow2_ceil, otypes=[np.float32])(s0))
        # division by a power of two is exact, so the codes are torch's float8
        # conversion of the clamped exact quotient
        srep = np.repeat(s1, G, axis=1)
        ratio = np.clip(x / srep, -448, 448).astype(np.float32)
        want = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q1, want)
        # the group's absmax lands in [224, 448]
        top = np.max(np.abs(oracle.decode(q1)).reshape(32, -1, G), axis=2)
        live = np.max(np.abs(x).reshape(32, -1, G), axis=2) > 1e-10
        assert np.all((top[live] >= 224) & (top[live] <= 448))


def test_ue8m0_weight_blocks():
    w = synth.weights("pin-ue8m0-w", 256, 384).numpy()
    q0, s0 = oracle.quant_weight_blockwise(w)
    q1, s1 = oracle.quant_weight_blockwise(w, scale_ue8m0=True)
    assert np.array_equal(s1, np.vectorize(oracle.pow2_ceil, otypes=[np.float32])(s0))
    # one-row blocks are the per-token-group quantizer with the same flag
    qa, sa = oracle.quant_weight_blockwise(w[:8], block_n=1, block_k=128, scale_ue8m0=True)
    qb, sb = oracle.quant_per_token_group(w[:8], 128, scale_ue8m0=True)
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)
    # codes: torch's float8 conversion of the exact quotient by the block scale
    srep = np.repeat(np.repeat(s1, 128, axis=0), 128, axis=1)
    want = torch.from_numpy(np.clip(w / srep, -448, 448).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q1, want)


# ---------------------------------------------------------------- static
def test_static_equals_dynamic_with_its_scale():
    x = synth.activations("pin-static", 16, 256).float().numpy()
    q, s = oracle.quant_per_token(x)
    for r in range(16):
        assert np.array_equal(oracle.quant_static(x[r:r + 1], s[r])[0], q[r])


def test_static_brute_force_and_saturation():
    x = synth.activations("pin-static-brute", 2, 64).float().numpy()
    for sv in (0.03, 0.0071, 1.7, 2.0 ** -9):
        s = np.float32(sv)
        q = oracle.quant_static(x, s)
        fs = Fraction(float(s))
        for r in range(2):
            got = [int(c) for c in q[r]]
            want = [_code_of_exact(Fraction(v) / fs) for v in x[r].tolist()]
            want = [c if not (c == 0 and v < 0) else 0x80 for c, v in zip(want, x[r])]
            assert got == want, (sv, r)
    big = np.array([[1e4, -1e4, 448 * 0.5, -449 * 0.5]], np.float32)
    assert [int(c) for c in oracle.quant_static(big, np.float32(0.5))[0]] == [0x7E, 0xFE, 0x7E, 0xFE]
    with pytest.raises(ValueError):
        oracle.quant_static(big, np.float32(0))


def _code_of_exact(fr):
    """E4M3 code of fp32(fr), both roundings to nearest even, by exact arithmetic."""
    if fr == 0:
        return 0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    qq = a / ulp
    fl = qq.numerator // qq.denominator
    rem = qq - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = min(fl * ulp, Fraction(448))
    finite = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist()
    best = None
    for code, fv in enumerate(finite):
        d = abs(Fraction(fv) - v)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1] | (0x80 if sign < 0 else 0)
