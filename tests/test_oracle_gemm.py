"""Pins of the oracle's fp64 channelwise and blockwise GEMM references.

Pinned by: a hand-worked example (tests/golden/gemm_worked_example.txt), exact
rational brute force on tiny shapes (decode by torch, arithmetic in
``fractions``), closed-form identities, and the relations between the two GEMM
kinds (uniform block scales and single-K-block cases reduce to channelwise).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).double().numpy()


def _parse_matrix(txt):
    return [[int(c, 16) for c in row.split()] for row in txt.split(";")]


def _golden_example():
    d = {}
    with open(os.path.join(GOLDEN, "gemm_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = v.strip()
    return d


def test_worked_example():
    d = _golden_example()
    a = np.array(_parse_matrix(d["a"]), dtype=np.uint8)
    b = np.array(_parse_matrix(d["b"]), dtype=np.uint8)
    sa = np.array(d["a_scale"].split(), dtype=np.float32)
    sb = np.array(d["b_scale"].split(), dtype=np.float32)
    bias = np.array(d["bias"].split(), dtype=np.float64)
    want = np.array([[float(v) for v in r.split()] for r in d["out"].split(";")])
    got = oracle.scaled_mm_channelwise(a, b, sa, sb, bias)
    assert np.array_equal(got, want)


def _brute_channelwise(a, b, sa, sb, bias):
    A = _torch_decode(a)
    B = _torch_decode(b)
    M, K = A.shape
    N = B.shape[0]
    out = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = sum(Fraction(float(A[m, k])) * Fraction(float(B[n, k])) for k in range(K))
            v = acc * Fraction(float(sa[m])) * Fraction(float(sb[n]))
            if bias is not None:
                v += Fraction(float(bias[n]))
            out[m][n] = v
    return out


def _brute_blockwise(a, b, sa, sb, bias, bn, bk):
    A = _torch_decode(a)
    B = _torch_decode(b)
    M, K = A.shape
    N = B.shape[0]
    out = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            v = Fraction(0)
            for kb in range(-(-K // bk)):
                part = sum(Fraction(float(A[m, k])) * Fraction(float(B[n, k]))
                           for k in range(kb * bk, min(K, (kb + 1) * bk)))
                v += part * Fraction(float(sa[m, kb])) * Fraction(float(sb[n // bn, kb]))
            if bias is not None:
                v += Fraction(float(bias[n]))
            out[m][n] = v
    return out


def _close_to_exact(ref64, exact, rel=2.0 ** -40):
    for m, row in enumerate(exact):
        for n, v in enumerate(row):
            assert abs(Fraction(float(ref64[m, n])) - v) <= rel * (abs(v) + Fraction(1, 2 ** 60)), (m, n)


@pytest.mark.parametrize("M,N,K", [(3, 5, 128), (8, 4, 256), (1, 7, 128)])
def test_channelwise_exact_rational(M, N, K):
    a = synth.random_codes(f"pin-cw-a/{M}/{K}", (M, K)).numpy()
    b = synth.random_codes(f"pin-cw-b/{N}/{K}", (N, K)).numpy()
    sa = synth.positive_scales(f"pin-cw-sa/{M}", (M,)).numpy()
    sb = synth.positive_scales(f"pin-cw-sb/{N}", (N,)).numpy()
    bias = synth.bias("pin-cw", N).float().numpy()
    ref = oracle.scaled_mm_channelwise(a, b, sa, sb, bias)
    assert ref.shape == (M, N)
    _close_to_exact(ref, _brute_channelwise(a, b, sa, sb, bias))


@pytest.mark.parametrize("M,N,K,bn,bk", [(3, 5, 256, 2, 128), (4, 6, 384, 4, 128), (2, 3, 200, 2, 128)])
def test_blockwise_exact_rational(M, N, K, bn, bk):
    kb = -(-K // bk)
    a = synth.random_codes(f"pin-bw-a/{M}/{K}", (M, K)).numpy()
    b = synth.random_codes(f"pin-bw-b/{N}/{K}", (N, K)).numpy()
    sa = synth.positive_scales(f"pin-bw-sa/{M}/{K}", (M, kb)).numpy()
    sb = synth.positive_scales(f"pin-bw-sb/{N}/{K}", (-(-N // bn), kb)).numpy()
    bias = synth.bias("pin-bw", N).float().numpy()
    ref = oracle.scaled_mm_blockwise(a, b, sa, sb, bias, block_n=bn, block_k=bk)
    _close_to_exact(ref, _brute_blockwise(a, b, sa, sb, bias, bn, bk))


def test_identity_all_ones():
    K = 512
    a = np.full((4, K), 0x38, np.uint8)
    b = np.full((8, K), 0x38, np.uint8)
    sa = np.full(4, 2.0 ** -3, np.float32)
    sb = np.full(8, 2.0 ** -5, np.float32)
    out = oracle.scaled_mm_channelwise(a, b, sa, sb)
    assert np.all(out == K * 2.0 ** -8)


def test_identity_pattern_b():
    K = 128
    a = synth.random_codes("pin-id-a", (5, K)).numpy()
    b = np.zeros((K, K), np.uint8)
    b[np.arange(K), np.arange(K)] = 0x38
    sa = np.array([2.0 ** -j for j in range(5)], np.float32)
    sb = np.full(K, 4.0, np.float32)
    out = oracle.scaled_mm_channelwise(a, b, sa, sb)
    want = _torch_decode(a) * sa.astype(np.float64)[:, None] * 4.0
    assert np.array_equal(out, want)


def test_zero_a_gives_bias():
    a = np.zeros((3, 256), np.uint8)
    b = synth.random_codes("pin-zero-b", (16, 256)).numpy()
    bias = synth.bias("pin-zero", 16).float().numpy()
    out = oracle.scaled_mm_channelwise(a, b, np.ones(3, np.float32), np.ones(16, np.float32), bias)
    assert np.array_equal(out, np.broadcast_to(bias.astype(np.float64), (3, 16)))
    sa = np.ones((3, 2), np.float32)
    sb = np.ones((1, 2), np.float32)
    out2 = oracle.scaled_mm_blockwise(a, b, sa, sb, bias)
    assert np.array_equal(out2, out)


def test_operand_order_not_transposed():
    # non-square, non-symmetric: swapping A and B or K/N indexing changes the result
    a = np.array([[0x38, 0x40, 0x00]], np.uint8)  # [1, 2, 0]
    b = np.array([[0x38, 0x00, 0x00], [0x00, 0x38, 0x00]], np.uint8)
    out = oracle.scaled_mm_channelwise(a, b, np.ones(1, np.float32), np.array([1, 3], np.float32))
    assert out.tolist() == [[1.0, 6.0]]


def test_blockwise_uniform_scales_equals_channelwise():
    M, N, K = 6, 256, 384
    a = synth.random_codes("pin-u-a", (M, K)).numpy()
    b = synth.random_codes("pin-u-b", (N, K)).numpy()
    sa_row = synth.positive_scales("pin-u-sa", (M,)).numpy()
    sb_blk = synth.positive_scales("pin-u-sb", (N // 128,)).numpy()
    sa = np.repeat(sa_row[:, None], K // 128, axis=1)
    sb = np.repeat(sb_blk[:, None], K // 128, axis=1)
    out_b = oracle.scaled_mm_blockwise(a, b, sa, sb)
    out_c = oracle.scaled_mm_channelwise(a, b, sa_row, np.repeat(sb_blk, 128))
    np.testing.assert_allclose(out_b, out_c, rtol=1e-12, atol=0)


def test_blockwise_single_k_block_equals_channelwise():
    M, N, K = 4, 256, 128
    a = synth.random_codes("pin-k1-a", (M, K)).numpy()
    b = synth.random_codes("pin-k1-b", (N, K)).numpy()
    sa = synth.positive_scales("pin-k1-sa", (M, 1)).numpy()
    sb = synth.positive_scales("pin-k1-sb", (2, 1)).numpy()
    out_b = oracle.scaled_mm_blockwise(a, b, sa, sb)
    out_c = oracle.scaled_mm_channelwise(a, b, sa[:, 0], np.repeat(sb[:, 0], 128))
    np.testing.assert_allclose(out_b, out_c, rtol=1e-13, atol=0)


def test_power_of_two_weight_scale_scales_output():
    a = synth.random_codes("pin-p2-a", (3, 256)).numpy()
    b = synth.random_codes("pin-p2-b", (8, 256)).numpy()
    sa = synth.positive_scales("pin-p2-sa", (3,)).numpy()
    sb = synth.positive_scales("pin-p2-sb", (8,)).numpy()
    o1 = oracle.scaled_mm_channelwise(a, b, sa, sb)
    o2 = oracle.scaled_mm_channelwise(a, b, sa, sb * np.float32(8))
    assert np.array_equal(o2, o1 * 8)


def test_summation_bound_covers_fp32_accumulation():
    # an fp32 sequential accumulation of the exact products stays within tau
    M, N, K = 4, 8, 4096
    a = synth.random_codes("pin-tau-a", (M, K)).numpy()
    b = synth.random_codes("pin-tau-b", (N, K)).numpy()
    sa = np.ones(M, np.float32)
    sb = np.ones(N, np.float32)
    ref = oracle.scaled_mm_channelwise(a, b, sa, sb)
    tau = oracle.summation_bound_channelwise(a, b, sa, sb)
    prod = _torch_decode(a)[:, None, :] * _torch_decode(b)[None, :, :]
    acc = np.zeros((M, N), np.float32)
    for k in range(K):
        acc = (acc + prod[:, :, k].astype(np.float32)).astype(np.float32)
    assert np.all(np.abs(acc - ref) <= tau)
    assert np.any(tau > 0)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(7)
    # fp32 inputs: torch's double->bf16 goes through fp32 (a double rounding),
    # so the comparison uses values that are already exact in fp32
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, 448.0]]).astype(np.float32)
    v = v.astype(np.float64)
    want = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    assert oracle.bf16_round(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8])).tolist() == [1.0, 1.015625]
    assert np.array_equal(oracle.bf16_round(v), want)


def test_check_gemm_accepts_and_rejects():
    ref = np.array([[1.0, -2.0], [100.0, 0.5]])
    tau = np.zeros_like(ref)
    assert oracle.check_gemm(ref * (1 + 2.0 ** -8), ref, tau)["ok"]
    bad = ref.copy()
    bad[1, 1] *= 1.1
    assert not oracle.check_gemm(bad, ref, tau)["ok"]
    assert not oracle.check_gemm(ref + 2.0, ref, tau + 1.0)["ok"]  # above 1e-2 * max|ref|
    nan = ref.copy()
    nan[0, 0] = np.nan
    assert not oracle.check_gemm(nan, ref, tau)["ok"]


def test_blockwise_summation_bound_closed_form():
    # All codes 0x38 (1.0), K = 256 (two K blocks), N = 256 (two N blocks):
    # every product is 1, so sum_k |dec(A) dec(B)| over block kb is 128 and
    # tau[m, n] = K 2^-23 sum_kb 128 sa[m, kb] sb[n // 128, kb] exactly.
    M, N, K = 2, 256, 256
    a = np.full((M, K), 0x38, np.uint8)
    b = np.full((N, K), 0x38, np.uint8)
    sa = np.array([[1.0, 2.0], [0.5, 4.0]], np.float32)
    sb = np.array([[1.0, 4.0], [8.0, 16.0]], np.float32)
    tau = oracle.summation_bound_blockwise(a, b, sa, sb)
    per_block = np.array([[128 * (1 * 1 + 2 * 4), 128 * (1 * 8 + 2 * 16)],
                          [128 * (0.5 * 1 + 4 * 4), 128 * (0.5 * 8 + 4 * 16)]], np.float64)
    want = K * 2.0 ** -23 * np.repeat(per_block, 128, axis=1)
    assert np.array_equal(tau, want)


def test_blockwise_summation_bound_uniform_scales_equals_channelwise():
    # with one scale per row and one per 128-row weight block, the block-scaled
    # bound is the channelwise bound with the block scale spread over its rows
    M, N, K = 5, 384, 512
    a = synth.random_codes("pin-tb-a", (M, K)).numpy()
    b = synth.random_codes("pin-tb-b", (N, K)).numpy()
    sa_row = synth.positive_scales("pin-tb-sa", (M,)).numpy()
    sb_blk = synth.positive_scales("pin-tb-sb", (N // 128,)).numpy()
    tau_b = oracle.summation_bound_blockwise(a, b, np.repeat(sa_row[:, None], K // 128, axis=1),
                                             np.repeat(sb_blk[:, None], K // 128, axis=1))
    tau_c = oracle.summation_bound_channelwise(a, b, sa_row, np.repeat(sb_blk, 128))
    np.testing.assert_allclose(tau_b, tau_c, rtol=1e-12, atol=0)
    assert np.all(tau_b > 0)


def test_blockwise_summation_bound_covers_promoted_fp32_accumulation():
    # The blockwise kernels' arithmetic done in fp32 on the CPU: each 128-deep
    # block summed sequentially in fp32, scaled by fp32(sa * sb), added to an
    # fp32 accumulator. Scales differ per row, per K block and per N block.
    M, N, K = 3, 256, 1024
    a = synth.random_codes("pin-tp-a", (M, K)).numpy()
    b = synth.random_codes("pin-tp-b", (N, K)).numpy()
    sa = synth.positive_scales("pin-tp-sa", (M, K // 128)).numpy()
    sb = synth.positive_scales("pin-tp-sb", (N // 128, K // 128)).numpy()
    ref = oracle.scaled_mm_blockwise(a, b, sa, sb)
    tau = oracle.summation_bound_blockwise(a, b, sa, sb)
    prod = (_torch_decode(a)[:, None, :] * _torch_decode(b)[None, :, :]).astype(np.float32)
    acc = np.zeros((M, N), np.float32)
    nb = np.arange(N) // 128
    for kb in range(K // 128):
        part = np.zeros((M, N), np.float32)
        for k in range(kb * 128, (kb + 1) * 128):
            part = (part + prod[:, :, k]).astype(np.float32)
        sc = (sa[:, kb][:, None] * sb[nb, kb][None, :]).astype(np.float32)
        acc = (acc + (part * sc).astype(np.float32)).astype(np.float32)
    err = np.abs(acc.astype(np.float64) - ref)
    assert np.all(err <= tau)
    # the bound is a bound, not noise: it is within a few hundred times the
    # error actually made (K 2^-23 against ~sqrt(K) 2^-24 for random signs)
    assert np.max(err) > 0 and np.max(err / tau) > 1e-3


def test_check_gemm_probabilistic_floor_and_pure_relative_cap():
    # an fp32 sequential (round-to-nearest) accumulation passes the tighter
    # probabilistic floor and the pure-relative cap
    M, N, K = 4, 64, 4096
    a = synth.random_codes("pin-pf-a", (M, K)).numpy()
    b = synth.random_codes("pin-pf-b", (N, K)).numpy()
    sa = np.ones(M, np.float32)
    sb = np.ones(N, np.float32)
    ref = oracle.scaled_mm_channelwise(a, b, sa, sb)
    tau = oracle.summation_bound_channelwise(a, b, sa, sb)
    prod = (_torch_decode(a)[:, None, :] * _torch_decode(b)[None, :, :]).astype(np.float32)
    acc = np.zeros((M, N), np.float32)
    for k in range(K):
        acc = (acc + prod[:, :, k]).astype(np.float32)
    res = oracle.check_gemm(acc, ref, tau, k=K)
    assert res["ok"] and res["n_prob_floor_fail"] == 0 and res["prob_floor_used"] < 1.0, res
    floor = tau * 8.0 / (2.0 * np.sqrt(K))
    # one element off by twice the floor beyond 2^-6 |ref|: inside the
    # worst-case bound (floor << tau), outside the probabilistic one
    bad = ref.copy()
    bad[1, 3] += 2.0 ** -6 * abs(ref[1, 3]) + 2.0 * floor[1, 3]
    assert oracle.check_gemm(bad, ref, tau)["ok"]
    res = oracle.check_gemm(bad, ref, tau, k=K)
    assert not res["ok"] and res["n_prob_floor_fail"] == 1
    # 2% of the elements off by 1.5 * 2^-6 relative but inside the floor:
    # each passes the per-element test, the pure-relative cap fails
    idx = np.unravel_index(np.arange(0, M * N, 50), (M, N))
    off = ref.copy()
    off[idx] += np.minimum(1.5 * 2.0 ** -6 * np.abs(ref[idx]), 2.0 ** -6 * np.abs(ref[idx]) + 0.5 * floor[idx])
    res = oracle.check_gemm(off, ref, tau, k=K)
    assert res["n_prob_floor_fail"] == 0 and res["frac_pure_rel_fail"] > 0.01 and not res["ok"], res
