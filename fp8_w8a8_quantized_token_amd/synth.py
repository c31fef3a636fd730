"""Seeded synthetic inputs for the FP8 W8A8 linear workloads.

This module only draws random numbers; it holds none of the quantization or
GEMM arithmetic. Tests feed the same tensors to the HIP path and to the CPU
oracle, and the benchmark draws its inputs here too.

Every tensor is drawn on the CPU from a ``torch.Generator`` seeded with
``zlib.crc32`` of a key naming the workload, the tensor and its shape; weight
keys leave out M, so the weight of a shape is the same at every M.

Workloads (all shapes [M, K] activations, [N, K] weights, bf16 out):

* ``small``       M=16 N=256 K=512, activations N(0,1), weights N(0,0.02).
* ``o_proj``      N=K=4096, M in 1..8192 (powers of two); activations N(0,1)
                  with 1% of the K columns (seeded) multiplied by 50 in every
                  row, standing in for outlier channels.
* ``qwen3_8b``    Qwen3-8B-style linears qkv (6144,4096), down (4096,12288),
                  gate_up (24576,4096) at M in {1,64,512,8192}, bias N(0,0.1).
* ``block_7168``  blockwise, N=K=7168, M in {1,2,3,5,7,13,31,64,256}.
* ``block_moe``   blockwise, (3072,4096) and (4096,1536), M in {1,4,16,64,4096}.
"""

import zlib

import torch

WORKLOADS = {
    "small": {"kind": "channelwise", "shapes": [(256, 512)], "ms": [16], "bias": False,
              "outliers": 0.0},
    "o_proj": {"kind": "channelwise", "shapes": [(4096, 4096)],
               "ms": [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192],
               "bias": False, "outliers": 0.01},
    "qwen3_8b": {"kind": "channelwise", "shapes": [(6144, 4096), (4096, 12288), (24576, 4096)],
                 "ms": [1, 64, 512, 8192], "bias": True, "outliers": 0.0},
    "block_7168": {"kind": "blockwise", "shapes": [(7168, 7168)],
                   "ms": [1, 2, 3, 5, 7, 13, 31, 64, 256], "bias": False, "outliers": 0.0},
    "block_moe": {"kind": "blockwise", "shapes": [(3072, 4096), (4096, 1536)],
                  "ms": [1, 4, 16, 64, 4096], "bias": False, "outliers": 0.0},
}


def seed_of(key: str) -> int:
    return zlib.crc32(key.encode("utf-8"))


def _gen(key: str) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_of(key))
    return g


def activations(workload: str, m: int, k: int, outlier_frac: float = 0.0,
                outlier_gain: float = 50.0, tag: str = "x") -> torch.Tensor:
    """bf16 [m, k] ~ N(0, 1); a seeded ``outlier_frac`` of the columns is
    multiplied by ``outlier_gain`` in every row."""
    x = torch.randn(m, k, generator=_gen(f"{workload}/{tag}/{k}/{m}"), dtype=torch.float32)
    n_out = int(round(outlier_frac * k))
    if n_out > 0:
        cols = torch.randperm(k, generator=_gen(f"{workload}/{tag}-outlier-cols/{k}"))[:n_out]
        x[:, cols] *= outlier_gain
    return x.to(torch.bfloat16)


def weights(workload: str, n: int, k: int, std: float = 0.02) -> torch.Tensor:
    """fp32 [n, k] ~ N(0, std^2), independent of M."""
    return torch.randn(n, k, generator=_gen(f"{workload}/w/{n}/{k}"), dtype=torch.float32) * std


def bias(workload: str, n: int, std: float = 0.1) -> torch.Tensor:
    """bf16 [n] ~ N(0, std^2)."""
    return (torch.randn(n, generator=_gen(f"{workload}/bias/{n}"), dtype=torch.float32)
            * std).to(torch.bfloat16)


def random_codes(key: str, shape) -> torch.Tensor:
    """uint8 codes drawn uniformly from the 254 finite E4M3 bit patterns
    (0x7F and 0xFF, the NaN patterns, are skipped)."""
    r = torch.randint(0, 254, tuple(shape), generator=_gen(key), dtype=torch.int32)
    r = r + (r >= 0x7F).to(torch.int32)  # skip 0x7F
    return r.to(torch.uint8)


def positive_scales(key: str, shape, lo: float = 2.0 ** -12, hi: float = 2.0 ** -4) -> torch.Tensor:
    """fp32 scales, log-uniform in [lo, hi)."""
    u = torch.rand(tuple(shape), generator=_gen(key), dtype=torch.float64)
    import math
    return torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).to(torch.float32)
