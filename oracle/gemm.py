"""fp64 references for the channelwise and blockwise FP8 scaled GEMMs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Channelwise (PR 34331 digest, "Tune FP8 GEMM Triton tiles on L40S and enable
them by default", section "Key source excerpts", ``apply_fp8_linear``): the
quantized activation [M, K], the FP8 weight, a per-token activation scale and a
per-output-channel weight scale go into one scaled matmul with an optional
fused bias and an output dtype:

    out[m, n] = a_scale[m] * b_scale[n] * sum_k dec(A[m, k]) * dec(B[n, k]) + bias[n]

Blockwise (PR 27896 digest, "Remove the per-call padding overhead of the FP8
blockwise GEMM", section "Key source excerpts", the blockwise linear): the
activation carries one scale per 1 x 128 group and the weight one scale per
128 x 128 block (``block_size = [128, 128]``, the second entry being the
activation group along K); the weight is [N, K]; bias is added after the GEMM:

    out[m, n] = sum_kb a_scale[m, kb] * b_scale[n // 128, kb]
                       * sum_{k in block kb} dec(A[m, k]) * dec(B[n, k]) + bias[n]

Both are computed in fp64 over the decoded E4M3 values: every E4M3 x E4M3
product is exact in fp64, and the fp64 sum's relative error (<= K * 2^-53) is
far below any tolerance used against an fp32-accumulating kernel.
"""

import numpy as np

from .e4m3 import decode


def scaled_mm_channelwise(a_codes, b_codes, a_scale, b_scale, bias=None) -> np.ndarray:
    """a_codes uint8 [M, K], b_codes uint8 [N, K], a_scale [M], b_scale [N],
    bias [N] or None -> float64 [M, N]."""
    a = decode(a_codes)
    b = decode(b_codes)
    acc = a @ b.T
    out = acc * np.asarray(a_scale, np.float64)[:, None] * np.asarray(b_scale, np.float64)[None, :]
    if bias is not None:
        out = out + np.asarray(bias, np.float64)[None, :]
    return out


def scaled_mm_blockwise(a_codes, b_codes, a_scale, b_scale, bias=None,
                        block_n: int = 128, block_k: int = 128) -> np.ndarray:
    """a_codes uint8 [M, K]; b_codes uint8 [N, K]; a_scale [M, ceil(K/bk)]
    (logical layout, one scale per row and K-block); b_scale
    [ceil(N/bn), ceil(K/bk)]; bias [N] or None -> float64 [M, N]."""
    a = decode(a_codes)
    b = decode(b_codes)
    a_scale = np.asarray(a_scale, np.float64)
    b_scale = np.asarray(b_scale, np.float64)
    m, k = a.shape
    n = b.shape[0]
    n_block_of = np.arange(n) // block_n
    out = np.zeros((m, n), dtype=np.float64)
    for kb in range(-(-k // block_k)):
        ks = slice(kb * block_k, min(k, (kb + 1) * block_k))
        part = a[:, ks] @ b[:, ks].T
        out += part * a_scale[:, kb][:, None] * b_scale[n_block_of, kb][None, :]
    if bias is not None:
        out = out + np.asarray(bias, np.float64)[None, :]
    return out


def summation_bound_channelwise(a_codes, b_codes, a_scale, b_scale) -> np.ndarray:
    """Worst-case error of an fp32 K-term accumulation, per output element.

    tau[m, n] = K * 2^-23 * a_scale[m] * b_scale[n] * sum_k |dec(A) dec(B)|.
    Recursive fp32 summation of K exact products errs by at most
    gamma_K * sum |terms| with gamma_K ~ K * 2^-24 (Higham); 2^-23 also covers a
    truncating (round-toward-zero) internal accumulator.
    """
    a = np.abs(decode(a_codes))
    b = np.abs(decode(b_codes))
    k = a.shape[1]
    mag = a @ b.T
    return k * 2.0 ** -23 * mag * np.abs(np.asarray(a_scale, np.float64))[:, None] \
        * np.abs(np.asarray(b_scale, np.float64))[None, :]


def summation_bound_blockwise(a_codes, b_codes, a_scale, b_scale,
                              block_n: int = 128, block_k: int = 128) -> np.ndarray:
    """As summation_bound_channelwise, with the per-block scales applied."""
    a = np.abs(decode(a_codes))
    b = np.abs(decode(b_codes))
    a_scale = np.abs(np.asarray(a_scale, np.float64))
    b_scale = np.abs(np.asarray(b_scale, np.float64))
    m, k = a.shape
    n = b.shape[0]
    n_block_of = np.arange(n) // block_n
    mag = np.zeros((m, n))
    for kb in range(-(-k // block_k)):
        ks = slice(kb * block_k, min(k, (kb + 1) * block_k))
        mag += (a[:, ks] @ b[:, ks].T) * a_scale[:, kb][:, None] * b_scale[n_block_of, kb][None, :]
    return k * 2.0 ** -23 * mag


def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64. bfloat16 keeps 8 significant bits; finite normal range only."""
    v = np.asarray(v, dtype=np.float64)
    mant, expo = np.frexp(v)  # v = mant * 2**expo, 0.5 <= |mant| < 1
    return np.ldexp(np.rint(mant * 256.0) / 256.0, expo)
