"""Shared helpers of the GPU parity tests: seeded inputs (synth), oracle
fixtures cached per session, device transfer, and case logging (printed and
flushed before every GPU step so a failing case is named)."""
import functools

import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import synth


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a GPU (run with -m 'not gpu' on a CPU host)")
    return torch.device("cuda:0")


def say(*args):
    print("[case]", *args, flush=True)


def gpu(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)) if isinstance(x, np.ndarray) else x
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device())


@functools.lru_cache(maxsize=None)
def activations(workload, m, k, outliers=0.0):
    return synth.activations(workload, m, k, outlier_frac=outliers)


@functools.lru_cache(maxsize=None)
def act_per_token(workload, m, k, outliers=0.0):
    """Oracle per-token quant of the workload's activations: (codes, scales)."""
    x = activations(workload, m, k, outliers).float().numpy()
    return oracle.quant_per_token(x)


@functools.lru_cache(maxsize=None)
def act_group(workload, m, k, group=128):
    x = activations(workload, m, k).float().numpy()
    return oracle.quant_per_token_group(x, group)


@functools.lru_cache(maxsize=4)
def weight_channelwise(workload, n, k):
    return oracle.quant_weight_per_channel(synth.weights(workload, n, k).numpy())


@functools.lru_cache(maxsize=4)
def weight_blockwise(workload, n, k):
    return oracle.quant_weight_blockwise(synth.weights(workload, n, k).numpy())


def sample_rows(m, count=48, seed=0):
    """Rows of an M-row output checked against the oracle when the whole
    output is too large: the first and last row of every 256-row band (of
    every 64-row band up to M = 1024), so every output tile row of every
    kernel is seen, plus `count` seeded random rows."""
    if m <= count:
        return np.arange(m)
    rng = np.random.default_rng(seed + m)
    band = 64 if m <= 1024 else 256
    fixed = {0, 1, m // 2, m - 2, m - 1}
    for lo in range(0, m, band):
        fixed.update((lo, min(lo + band, m) - 1))
    rest = rng.choice(m, size=count, replace=False)
    return np.array(sorted(fixed | set(int(r) for r in rest)))


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)
