"""The matrix core's rounding of an FP8 dot product, measured through the
library's MFMA probe (fp8_probe_mfma_dot: one V_MFMA_F32_16X16X128_F8F6F4 or
V_MFMA_F32_32X32X64_F8F6F4 on given operands), against the error model the
GEMM tolerance assumes (oracle.gemm_tolerance_*): the products of every run of
8 consecutive K positions are aligned to the largest of them and truncated
toward zero below 2^-13 of its leading bit; run sums and the accumulator input
are added with fp32-like precision. A change in that behaviour fails here
before it can hide behind (or be blamed on) the GEMM tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import _lib
from gpu_common import device, say

pytestmark = pytest.mark.gpu

TAB = oracle.decode_table()
FORMS = {0: (16, 128), 1: (32, 64)}   # form -> (rows, K) of one MFMA


def _code(v):
    return int(oracle.encode(np.array([v], np.float64))[0])


def _mfma(w, x, c, form):
    """w, x uint8 [B, R, KD]; c [B, R, R] -> D [B, R, R] (float64)."""
    dev = device()
    tw = torch.from_numpy(np.ascontiguousarray(w, np.uint8)).to(dev)
    tx = torch.from_numpy(np.ascontiguousarray(x, np.uint8)).to(dev)
    tc = torch.from_numpy(np.ascontiguousarray(c, np.float32)).to(dev)
    d = torch.empty(tc.shape, dtype=torch.float32, device=dev)
    lib = _lib.load()
    _lib.check(lib.fp8_probe_mfma_dot(ctypes.c_void_p(tw.data_ptr()), ctypes.c_void_p(tx.data_ptr()),
                                      ctypes.c_void_p(tc.data_ptr()), ctypes.c_void_p(d.data_ptr()),
                                      w.shape[0], form, None))
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


def _exact(w, x, c):
    return np.einsum("bnk,bmk->bnm", TAB[w], TAB[x]) + c


def _pair(form, small_p, k_small, sign=1, big_w=256.0, big_x=256.0):
    """One problem: W[0, 0] * X[0, 0] = big_w * big_x and, at K position
    k_small, the product sign * 2^small_p (both factors powers of two)."""
    r, kd = FORMS[form]
    w = np.zeros((1, r, kd), np.uint8)
    x = np.zeros((1, r, kd), np.uint8)
    w[0, 0, 0], x[0, 0, 0] = _code(big_w), _code(big_x)
    a = max(-9, min(8, small_p // 2))
    w[0, 0, k_small] = _code(sign * 2.0 ** a)
    x[0, 0, k_small] = _code(2.0 ** (small_p - a))
    return w, x


def _d00(form, *args, **kw):
    r = FORMS[form][0]
    return _mfma(*_pair(form, *args, **kw), np.zeros((1, r, r)), form)[0, 0, 0]


@pytest.mark.parametrize("form", [0, 1])
def test_small_product_in_the_largest_products_run_is_truncated(form):
    for sign in (1, -1):
        for k_small in (1, 7):
            kept = _d00(form, 3, k_small, sign) - 65536.0   # 2^-13 of 2^16
            lost = _d00(form, 2, k_small, sign) - 65536.0   # 2^-14: truncated toward zero
            say("run", form, sign, k_small, kept, lost)
            assert kept == sign * 8.0 and lost == 0.0
    # the grid follows the leading bit of the largest product: 240 * 256 =
    # 1.875 * 2^15 keeps 2^2 and drops 2^1
    assert _d00(form, 2, 1, big_w=240.0) - 61440.0 == 4.0
    assert _d00(form, 1, 1, big_w=240.0) - 61440.0 == 0.0


@pytest.mark.parametrize("form", [0, 1])
def test_product_in_another_run_is_kept(form):
    for k_small in (8, 15, 32, FORMS[form][1] - 1):
        got = _d00(form, -4, k_small) - 65536.0
        assert got == 2.0 ** -4, (form, k_small, got)


@pytest.mark.parametrize("form", [0, 1])
def test_accumulator_input_added_at_fp32_precision(form):
    r, kd = FORMS[form]
    w = np.zeros((1, r, kd), np.uint8)
    x = np.zeros((1, r, kd), np.uint8)
    w[0, 0, 0], x[0, 0, 0] = _code(1.0), _code(1.0)
    for q in (0, 10, 20, 22):
        c = np.zeros((1, r, r))
        c[0, 0, 0] = 2.0 ** q
        assert _mfma(w, x, c, form)[0, 0, 0] == 2.0 ** q + 1.0, (form, q)


@pytest.mark.parametrize("form", [0, 1])
def test_random_blocks_within_the_tolerance_model(form):
    """Realistic operands (per-row scaled N(0, 0.02) weights, N(0, 1)
    activations with 1% outliers x50), accumulator 0 or a partial sum of the
    same size: every output of one MFMA within the oracle's worst-case and
    probabilistic allowances (unit scales), plus the accumulator's own fp32
    rounding."""
    rng = np.random.default_rng(7 + form)
    r, kd = FORMS[form]
    nb = 256

    def qrows(v):
        s = np.abs(v).max(axis=-1, keepdims=True) / 448.0
        return oracle.encode(v / s).astype(np.uint8)

    wv = rng.normal(0, 0.02, (nb, r, kd))
    xv = rng.normal(0, 1, (nb, r, kd))
    xv[rng.random((nb, r, kd)) < 0.01] *= 50
    w, x = qrows(wv), qrows(xv)
    ones = np.ones(r)
    for mode in ("zero", "partial"):
        c = np.zeros((nb, r, r))
        if mode == "partial":
            c = (_exact(w, x, c) * rng.uniform(-3, 3, (nb, r, r))).astype(np.float32).astype(np.float64)
        d = _mfma(w, x, c, form)
        ex = _exact(w, x, c)
        worst = used = 0.0
        for i in range(nb):
            # D is [n][m]: n a row of W (the oracle's b), m a row of X (its a)
            tol = oracle.gemm_tolerance_channelwise(x[i], w[i], ones, ones)
            err = np.abs(d[i].T - ex[i].T)
            cpart = np.abs(c[i].T) * 2.0 ** -23
            assert np.all(err <= tol.tau + cpart), (mode, i)
            worst = max(worst, float(np.max(err / (tol.tau + cpart))))
            used = max(used, float(np.max(err / (tol.floor + cpart))))
        say("mfma random", form, mode, "worst/tau", worst, "worst/floor", used)
        assert used <= 1.0
