"""SiLU-and-mul of a [gate | up] activation, rounded once to bf16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The PR 27896 digest ("Remove the per-call padding overhead of the FP8
blockwise GEMM", section "Key source excerpts") shows the group quantizer's
kernel call with a ``fuse_silu_and_mul`` flag (passed as False there); the
digest prints no body for it. The reading taken, the plainest one that keeps
the fused call equal to the two calls it replaces:

* the input row holds 2K values, the gate in columns [0, K) and the up
  projection in columns [K, 2K) (the gate/up projection's output, whose N is
  twice the down projection's K);
* y = silu(gate) * up with silu(g) = g / (1 + exp(-g)), evaluated exactly
  (here in float64, whose error is far below the bf16 rounding that follows);
* y is rounded once to bf16 (round to nearest, ties to even) -- the activation
  dtype an unfused SiLU-and-mul would write -- and that bf16 row is what the
  quantizer sees. Fusing therefore changes no bits of the codes or scales.
"""

import numpy as np


def bf16_round_exact(v) -> np.ndarray:
    """float64 values -> nearest bfloat16 value (ties to even), as float64.

    bfloat16 keeps 8 significant bits and the fp32 exponent range; below
    2^-126 its step is fixed at 2^-133 (subnormals). Finite results only.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)  # |v| = m * 2^e, 0.5 <= m < 1 (e = 0 for v = 0)
    step_exp = np.maximum(e, -125) - 8
    step = np.ldexp(1.0, step_exp)
    return np.rint(v / step) * step  # v / step and the product are exact in float64


def silu_mul_bf16(x) -> np.ndarray:
    """x: [M, 2K] bf16-valued array -> float32 [M, K] holding bf16 values of
    bf16(silu(x[:, :K]) * x[:, K:])."""
    xf = np.asarray(x, dtype=np.float64)
    if xf.ndim != 2 or xf.shape[1] % 2 != 0:
        raise ValueError("expects a 2-D input with an even number of columns")
    k = xf.shape[1] // 2
    gate = xf[:, :k]
    up = xf[:, k:]
    with np.errstate(over="ignore"):
        silu = gate / (1.0 + np.exp(-gate))  # exp overflow -> inf -> silu = -0
    return bf16_round_exact(silu * up).astype(np.float32)
