"""Masked per-expert quantization and grouped blockwise GEMM (MoE experts).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The PR 27896 digest ("Remove the per-call padding overhead of the FP8
blockwise GEMM", "Key source excerpts") shows the group quantizer's kernel
call with a ``masked_m`` argument (None there); the digest prints no body for
it. Reading taken: a batch of E experts, each with its own slab of M_max rows
([E, M_max, K]), and ``masked_m[e]`` the number of valid rows of expert e; only
rows m < masked_m[e] are quantized (and, in the grouped GEMM, multiplied and
written), every other row is left as it was. Each expert has its own weight
[N, K] and 128x128 block scales; the per-expert computation is exactly the
plain group quantizer and blockwise GEMM of this package on the first
masked_m[e] rows.
"""

import numpy as np

from .gemm import scaled_mm_blockwise
from .quant import quant_per_token_group


def masked_quant_per_token_group(x, masked_m, group_size: int, eps: float = 1e-10,
                                 scale_ue8m0: bool = False):
    """x [E, M_max, K] bf16 values, masked_m [E] ints in [0, M_max].

    Returns (codes uint8 [E, M_max, K], scales float32 [E, M_max, K // G]);
    rows at or beyond masked_m[e] hold 0 codes and NaN scales here, only to
    mark them: the method leaves them untouched.
    """
    xf = np.asarray(x, dtype=np.float32)
    if xf.ndim != 3:
        raise ValueError("expects [E, M_max, K]")
    e_n, m_max, k = xf.shape
    masked_m = [int(v) for v in masked_m]
    if len(masked_m) != e_n or any(v < 0 or v > m_max for v in masked_m):
        raise ValueError("masked_m must hold E counts in [0, M_max]")
    codes = np.zeros((e_n, m_max, k), dtype=np.uint8)
    scales = np.full((e_n, m_max, k // group_size), np.nan, dtype=np.float32)
    for e in range(e_n):
        rows = masked_m[e]
        if rows:
            codes[e, :rows], scales[e, :rows] = quant_per_token_group(xf[e, :rows], group_size, eps,
                                                                      scale_ue8m0)
    return codes, scales


def scaled_mm_blockwise_masked(a, b, sa, sb, masked_m, block_n: int = 128, block_k: int = 128):
    """Grouped blockwise GEMM: a [E, M_max, K] codes, b [E, N, K] codes,
    sa [E, M_max, K/128], sb [E, N/128, K/128]; out[e, m] for m < masked_m[e]
    is the blockwise reference of expert e (float64), other rows NaN (unwritten)."""
    a = np.asarray(a)
    e_n, m_max, _ = a.shape
    n = np.asarray(b).shape[1]
    out = np.full((e_n, m_max, n), np.nan)
    for e in range(e_n):
        rows = int(masked_m[e])
        if rows:
            out[e, :rows] = scaled_mm_blockwise(a[e, :rows], b[e], sa[e, :rows], sb[e],
                                                block_n=block_n, block_k=block_k)
    return out
