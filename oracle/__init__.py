"""CPU oracle for the FP8 W8A8 quantized linear: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation of what the hot path
computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import it; the product package never does, and nothing here
imports the product package. It shares no code, table or constant generator
with the HIP path.

Sources (prhub.com.cn digests of three sglang pull requests):

* PR 34331 digest, "Tune FP8 GEMM Triton tiles on L40S and enable them by
  default" -- the channelwise scaled GEMM: per-token activation scale times
  per-output-channel weight scale, optional bias, output dtype (sections
  "Key source excerpts", ``apply_fp8_linear``).
* PR 31340 digest, "Fix FP8 Triton dtype selection on A100" -- names the FP8
  format as torch's ``float8_e4m3fn`` (section "Key source excerpts",
  ``fp8_dtype_to_triton``).
* PR 27896 digest, "Remove the per-call padding overhead of the FP8 blockwise
  GEMM" -- per-token-group quantization with eps, row alignment and
  column-major scales, and the blockwise linear (sections "Implementation",
  "Key source excerpts", "Risks and impact").

Readings taken where the pages are silent (each one is listed in the design
notes with its reason): OCP E4M3 with saturation at +-448, round to nearest
even, scale = max(absmax, eps) / 448 in fp32, element codes from a true fp32
division x / scale, signed zero kept, fp64 GEMM references.

Variants the pages name without a body, with the readings taken: the
quantizer's ``fuse_silu_and_mul`` flag (input [gate | up], quantized row
bf16(silu(gate) * up)), its ``scale_ue8m0`` flag (each fp32 scale rounded up
to a power of two), and a static per-tensor quantization with a given scale
(codes only) -- see ``activation.py`` and ``quant.py``; and its ``masked_m``
argument (per-expert valid row counts of an [E, M_max, K] batch, feeding a
grouped blockwise GEMM) -- see ``moe.py``.

Parity unpinned: behaviour on non-finite inputs (Inf/NaN), which the pages do
not define; every workload here is finite.
"""

from .e4m3 import E4M3_MAX, decode, decode_table, encode  # noqa: F401
from .activation import bf16_round_exact, silu_mul_bf16  # noqa: F401
from .quant import (  # noqa: F401
    padded_rows,
    pow2_ceil,
    quant_static,
    silu_mul_quant_per_token,
    silu_mul_quant_per_token_group,
    quant_per_token,
    quant_per_token_group,
    quant_weight_blockwise,
    quant_weight_per_channel,
    scales_col_major,
)
from .gemm import (  # noqa: F401
    bf16_round,
    scaled_mm_blockwise,
    scaled_mm_channelwise,
    summation_bound_blockwise,
    summation_bound_channelwise,
)
from .check import (  # noqa: F401
    Tolerance,
    check_gemm,
    gemm_tolerance_blockwise,
    gemm_tolerance_channelwise,
    mfma_truncation_blockwise,
    mfma_truncation_channelwise,
)
from .moe import masked_quant_per_token_group, scaled_mm_blockwise_masked  # noqa: F401
