"""Build libfp8w8a8.so (gfx950) in-tree with hipcc.

Usage: python -m fp8_w8a8_quantized_token_amd.build   (or build() from Python)
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8w8a8.so")
SOURCES = ["quant.hip", "gemm.hip", "tile_table.cpp", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE-correct fp32 division: the quantizer's codes depend on it
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall",
    "-Wno-unused-function",
    # M0 is clobbered on purpose by the LDS-DMA loads (see gemm.hip)
    "-Wno-inline-asm",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs, "-ldl"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    noisy = [ln for ln in (res.stdout + res.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    if verbose and noisy:
        print("\n".join(noisy))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
