"""Pins of the oracle's masked per-expert quantizer and grouped blockwise GEMM.

The pages only name ``masked_m`` (PR 27896 digest, "Key source excerpts": an
argument of the group quantizer's kernel call). Pinned by what the reading
fixes: every expert's valid rows equal the plain (pinned) quantizer and
blockwise GEMM on those rows; rows at or beyond masked_m[e] are untouched;
experts are independent; a full mask equals an unmasked batch; an empty
mask does nothing; a hand-sized two-expert example computed with exact
rationals.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import synth


def _batch(e, m, k, key):
    return np.stack([synth.activations(f"{key}/{i}", m, k).float().numpy() for i in range(e)])


def test_masked_quant_rows():
    x = _batch(3, 10, 256, "pin-moe-q")
    masked = [10, 0, 7]
    q, s = oracle.masked_quant_per_token_group(x, masked, 128)
    for e, rows in enumerate(masked):
        if rows:
            qe, se = oracle.quant_per_token_group(x[e, :rows], 128)
            assert np.array_equal(q[e, :rows], qe) and np.array_equal(s[e, :rows], se)
        assert np.all(q[e, rows:] == 0) and np.all(np.isnan(s[e, rows:]))


def test_masked_quant_experts_independent_and_full_mask():
    x = _batch(2, 6, 128, "pin-moe-ind")
    q0, s0 = oracle.masked_quant_per_token_group(x, [6, 6], 128)
    y = x.copy()
    y[1] *= 3.0
    q1, s1 = oracle.masked_quant_per_token_group(y, [6, 6], 128)
    assert np.array_equal(q0[0], q1[0]) and np.array_equal(s0[0], s1[0])
    qf, sf = oracle.quant_per_token_group(x.reshape(12, 128), 128)
    assert np.array_equal(q0.reshape(12, 128), qf) and np.array_equal(s0.reshape(12, 1), sf)
    qz, sz = oracle.masked_quant_per_token_group(x, [0, 0], 128)
    assert np.all(qz == 0) and np.all(np.isnan(sz))
    with pytest.raises(ValueError):
        oracle.masked_quant_per_token_group(x, [7, 0], 128)


def test_grouped_gemm_exact_rational():
    # two experts, tiny shapes, computed from torch's float8 decode with fractions
    e_n, m_max, n, k = 2, 3, 128, 256
    x = _batch(e_n, m_max, k, "pin-moe-mm")
    masked = [2, 3]
    a, sa = oracle.masked_quant_per_token_group(x, masked, 128)
    ws = [oracle.quant_weight_blockwise(synth.weights(f"pin-moe-w/{i}", n, k).numpy()) for i in range(e_n)]
    b = np.stack([w[0] for w in ws])
    sb = np.stack([w[1] for w in ws])
    out = oracle.scaled_mm_blockwise_masked(a, b, sa, sb, masked)
    dec = lambda c: torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()
    for e in range(e_n):
        A, B = dec(a[e]), dec(b[e])
        for m in range(m_max):
            if m >= masked[e]:
                assert np.all(np.isnan(out[e, m]))
                continue
            for nn in (0, 5, 77, 127):
                tot = Fraction(0)
                for kb in range(k // 128):
                    part = sum(Fraction(float(A[m, kk])) * Fraction(float(B[nn, kk]))
                               for kk in range(kb * 128, (kb + 1) * 128))
                    tot += part * Fraction(float(sa[e, m, kb])) * Fraction(float(sb[e, nn // 128, kb]))
                assert abs(out[e, m, nn] - float(tot)) <= 1e-12 * max(1.0, abs(float(tot)))
