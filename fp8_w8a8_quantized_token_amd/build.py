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
# the device compiler's per-kernel register / scratch / LDS report of the
# last build (one "remark" block per kernel)
RESOURCE_REPORT = os.path.join(PKG, "_build", "resource_usage.txt")
SOURCES = ["quant.hip", "gemm.hip", "probes.hip", "tile_table.cpp", "api.cpp"]

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
    # per-kernel resource usage (VGPRs, scratch, LDS), kept in RESOURCE_REPORT
    "-Rpass-analysis=kernel-resource-usage",
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
    lines = (res.stdout + res.stderr).splitlines()
    remarks = [ln for ln in lines if "[-Rpass-analysis=kernel-resource-usage]" in ln]
    noisy = [ln for ln in lines
             if ln.strip() and "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln
             and "kernel-resource-usage" not in ln and not ln.lstrip().startswith(("|", "^"))
             and not ln.lstrip()[:1].isdigit()]
    if verbose and noisy:
        print("\n".join(noisy))
    os.makedirs(os.path.dirname(RESOURCE_REPORT), exist_ok=True)
    with open(RESOURCE_REPORT, "w") as f:
        f.write("\n".join(remarks) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
