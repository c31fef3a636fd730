"""Per-token and per-token-group FP8 quantization, row-padded, as a plain loop.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Method (PR 27896 digest, "Remove the per-call padding overhead of the FP8
blockwise GEMM", sections "Implementation" and "Key source excerpts"):

* the input is a 2-D activation [M, K] whose K is a multiple of the group size;
* each row is cut into groups of ``group_size`` consecutive columns and every
  group gets one fp32 scale; eps defaults to 1e-10;
* the code buffer has M_pad = ceil(M / row_alignment) * row_alignment rows
  (alignment 4 by default); the scale buffer is column-major: logical
  (M_pad, K / G) with unit stride along rows, i.e. the scale of (row m,
  group g) sits at flat index g * M_pad + m;
* only the first M rows are quantized; rows M..M_pad-1 of both buffers are left
  as they were ("Risks and impact": the tail rows are never read for output).

The scale formula is not printed on the pages; the reading taken is
``scale = fp32(max(absmax, fp32(eps)) / 448)`` and ``code = E4M3(x / scale)``
with both divisions in IEEE fp32 (round to nearest even), and x/scale clamped
to +-448 before conversion. Per-token quantization, which feeds the channelwise
GEMM of the PR 34331 digest but is produced off-page there, is the same
operation with a single group spanning the whole row.
"""

import math

import numpy as np

from .activation import silu_mul_bf16
from .e4m3 import E4M3_MAX, encode

F32 = np.float32


def padded_rows(m: int, row_alignment: int) -> int:
    """M_pad: M rounded up to a multiple of row_alignment (ceil-align)."""
    if row_alignment <= 0:
        raise ValueError("row_alignment must be positive")
    return -(-m // row_alignment) * row_alignment


def pow2_ceil(s) -> np.float32:
    """The smallest power of two >= s (s a positive finite fp32 value).

    UE8M0 scales (the ``scale_ue8m0`` flag of the group quantizer's kernel call,
    PR 27896 digest, "Key source excerpts"; the digest prints no body for it).
    Reading taken: the fp32 scale of the plain method is rounded UP to a power
    of two, so x / scale still lies within +-448 and the scale is an 8-bit
    exponent with no mantissa.
    """
    mant, expo = math.frexp(float(s))  # s = mant * 2^expo, 0.5 <= mant < 1
    return F32(s) if mant == 0.5 else F32(math.ldexp(1.0, expo))


def quant_per_token_group(x, group_size: int, eps: float = 1e-10, scale_ue8m0: bool = False):
    """Quantize rows of x group by group.

    x: array-like [M, K] of bf16 values (any dtype that holds them exactly;
    converted to fp32, which is exact for bf16).
    scale_ue8m0: round every scale up to a power of two (see pow2_ceil) before
    the codes are formed.
    Returns (codes uint8 [M, K], scales float32 [M, K // group_size]).
    """
    xf = np.asarray(x, dtype=F32)
    if xf.ndim != 2:
        raise ValueError("expects a 2-D input")
    m, k = xf.shape
    if k % group_size != 0:
        raise ValueError("K must be a multiple of group_size")
    n_groups = k // group_size
    codes = np.zeros((m, k), dtype=np.uint8)
    scales = np.zeros((m, n_groups), dtype=F32)
    eps32 = F32(eps)
    fmax = F32(E4M3_MAX)
    for row in range(m):
        for g in range(n_groups):
            seg = xf[row, g * group_size:(g + 1) * group_size]
            amax = np.max(np.abs(seg)) if group_size > 0 else F32(0)
            amax = max(F32(amax), eps32)
            s = F32(F32(amax) / fmax)
            if scale_ue8m0:
                s = pow2_ceil(s)
            scales[row, g] = s
            ratio = (seg / s).astype(F32)  # IEEE fp32 division per element
            codes[row, g * group_size:(g + 1) * group_size] = encode(ratio)
    return codes, scales


def quant_per_token(x, eps: float = 1e-10):
    """One group per row: returns (codes uint8 [M, K], scales float32 [M])."""
    xf = np.asarray(x, dtype=F32)
    codes, scales = quant_per_token_group(xf, xf.shape[1], eps)
    return codes, scales[:, 0].copy()


def silu_mul_quant_per_token_group(x, group_size: int, eps: float = 1e-10,
                                   scale_ue8m0: bool = False):
    """The group quantizer with SiLU-and-mul fused in front (``fuse_silu_and_mul``
    in the quantizer's kernel call, PR 27896 digest, "Key source excerpts"):
    x is [M, 2K] = [gate | up]; the quantized row is bf16(silu(gate) * up).
    Returns (codes uint8 [M, K], scales float32 [M, K // group_size])."""
    return quant_per_token_group(silu_mul_bf16(x), group_size, eps, scale_ue8m0)


def silu_mul_quant_per_token(x, eps: float = 1e-10):
    """Per-token form of the above: (codes uint8 [M, K], scales float32 [M])."""
    y = silu_mul_bf16(x)
    codes, scales = quant_per_token_group(y, y.shape[1], eps)
    return codes, scales[:, 0].copy()


def quant_static(x, scale):
    """Static per-tensor quantization with a given fp32 scale.

    The PR 31340 digest ("Fix FP8 Triton dtype selection on A100",
    "Implementation" and "Key files") names a static FP8 quantization kernel and
    the ModelOpt FP8 linear's precomputed ``input_scale``, without a body.
    Reading taken: the same element step as the dynamic quantizer with the scale
    supplied instead of derived, code = E4M3_RNE(clamp(fp32(x / scale), +-448)),
    IEEE fp32 division; no scale is produced.
    x: [M, K] bf16 values; scale: one positive finite fp32 value.
    Returns codes uint8 [M, K].
    """
    xf = np.asarray(x, dtype=F32)
    s = F32(scale)
    if not (np.isfinite(s) and s > 0):
        raise ValueError("scale must be a positive finite fp32 value")
    return encode((xf / s).astype(F32))


def scales_col_major(scales, m_pad: int) -> np.ndarray:
    """Flat column-major storage of [M, G] scales in an M_pad-row buffer.

    Entry (m, g) goes to index g * m_pad + m. Pad positions (m >= M) hold NaN
    here only to mark them; the method leaves them unwritten.
    """
    scales = np.asarray(scales, dtype=F32)
    m, g = scales.shape
    out = np.full(g * m_pad, np.nan, dtype=F32)
    for gi in range(g):
        out[gi * m_pad:gi * m_pad + m] = scales[:, gi]
    return out


def quant_weight_per_channel(w, eps: float = 1e-10):
    """Per-output-channel weight quantization of W[N, K] (one scale per row n)."""
    return quant_per_token(w, eps)


def quant_weight_blockwise(w, block_n: int = 128, block_k: int = 128, eps: float = 1e-10,
                           scale_ue8m0: bool = False):
    """128x128-block weight quantization of W[N, K].

    Each (block_n x block_k) tile gets scale = max(absmax, eps) / 448 and its
    entries are encoded as E4M3(w / scale), in fp32 like the activations.
    scale_ue8m0 rounds each block scale up to a power of two first, as for the
    activations (see pow2_ceil).
    Returns (codes uint8 [N, K], scales float32 [ceil(N/bn), ceil(K/bk)]).
    """
    wf = np.asarray(w, dtype=F32)
    n, k = wf.shape
    nb = -(-n // block_n)
    kb = -(-k // block_k)
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((nb, kb), dtype=F32)
    eps32 = F32(eps)
    fmax = F32(E4M3_MAX)
    for i in range(nb):
        for j in range(kb):
            tile = wf[i * block_n:(i + 1) * block_n, j * block_k:(j + 1) * block_k]
            amax = max(F32(np.max(np.abs(tile))), eps32)
            s = F32(amax / fmax)
            if scale_ue8m0:
                s = pow2_ceil(s)
            scales[i, j] = s
            codes[i * block_n:(i + 1) * block_n, j * block_k:(j + 1) * block_k] = encode(
                (tile / s).astype(F32))
    return codes, scales
