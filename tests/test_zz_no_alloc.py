"""fp8_scaled_mm_noalloc (the GEMMs on the library's static split-K scratch)
against the workspace-taking entry points, through the C ABI.

Two calls in a row per kind, the second on a smaller input, with split-K
configs so the static scratch is used; outputs must be bit-identical to those
of fp8_scaled_mm_channelwise_ex / fp8_scaled_mm_blockwise_ex with a caller
workspace and within the GEMM tolerance of the fp64 oracle. A plan that needs
more scratch than the library holds is refused before any device work.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import _lib, ops
from gpu_common import act_group, act_per_token, bf16_to_f64, device, gpu, say, weight_blockwise, weight_channelwise

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _noalloc(kind, a, b, sa, sa_ld, sb, bias, out, m, n, k, cfg):
    return _lib.load().fp8_scaled_mm_noalloc(kind, _p(a), _p(b), _p(sa), sa_ld, _p(sb), _p(bias), _p(out),
                                             m, n, k, a.stride(0), b.stride(0), out.stride(0),
                                             ctypes.byref(cfg), _stream())


def _with_workspace(kind, a, b, sa, sa_ld, sb, bias, out, m, n, k, cfg):
    lib = _lib.load()
    nws = lib.fp8_scaled_mm_workspace_size(kind, m, n, k, ctypes.byref(cfg))
    assert nws > 0, "the case must use split-K"
    ws = torch.zeros(nws, dtype=torch.uint8, device=device())
    if kind == ops.KIND_CHANNELWISE:
        st = lib.fp8_scaled_mm_channelwise_ex(_p(a), _p(b), _p(sa), _p(sb), _p(bias), _p(out), m, n, k,
                                              a.stride(0), b.stride(0), out.stride(0), _p(ws), nws,
                                              ctypes.byref(cfg), _stream())
    else:
        st = lib.fp8_scaled_mm_blockwise_ex(_p(a), _p(b), _p(sa), sa_ld, _p(sb), _p(bias), _p(out), m, n, k,
                                            a.stride(0), b.stride(0), out.stride(0), _p(ws), nws,
                                            ctypes.byref(cfg), _stream())
    torch.cuda.synchronize()
    return st, ws


CASES = [
    ("cw", "t64x64panel", 3, 300, 392, 2048),
    ("cw", "t64x32deep", 2, 100, 256, 1024),
    ("bw", "t256x128panel", 2, 301, 384, 1024),
    ("bw", "t64x64deep", 4, 64, 256, 512),
    ("cw", "decode", 3, 16, 4104, 12288),
    ("bw", "decode", 2, 3, 512, 2048),
]


def _run_case(kind_s, variant, split_k, m, n, k):
    cfg = ops.make_config(variant, split_k)
    if kind_s == "cw":
        kind = ops.KIND_CHANNELWISE
        a, sa = act_per_token("noalloc", m, k)
        b, sb = weight_channelwise("noalloc", n, k)
        a_d, sa_d, sa_ld = gpu(a), gpu(sa), 0
        ref = oracle.scaled_mm_channelwise(a, b, sa, sb)
        tau = oracle.gemm_tolerance_channelwise(a, b, sa, sb)
    else:
        kind = ops.KIND_BLOCKWISE
        a, sa = act_group("noalloc", m, k)
        b, sb = weight_blockwise("noalloc", n, k)
        m_pad = ops.padded_rows(m, 4)
        a_d = torch.zeros((m_pad, k), dtype=torch.uint8, device=device())
        a_d[:m] = gpu(a)
        s_store = torch.zeros((k // 128, m_pad), dtype=torch.float32, device=device())
        s_store[:, :m] = gpu(sa.T.copy())
        sa_d, sa_ld = s_store, m_pad
        ref = oracle.scaled_mm_blockwise(a, b, sa, sb)
        tau = oracle.gemm_tolerance_blockwise(a, b, sa, sb)
    b_d, sb_d = gpu(b), gpu(sb)
    out_ws = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=device())
    out_na = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=device())
    say("noalloc", kind_s, variant, split_k, m, n, k)
    st, _ = _with_workspace(kind, a_d, b_d, sa_d, sa_ld, sb_d, None, out_ws, m, n, k, cfg)
    assert st == 0, _lib.load().fp8_last_error()
    st = _noalloc(kind, a_d, b_d, sa_d, sa_ld, sb_d, None, out_na, m, n, k, cfg)
    assert st == 0, _lib.load().fp8_last_error()
    torch.cuda.synchronize()
    assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), "differs from the workspace entry"
    res = oracle.check_gemm(bf16_to_f64(out_na), ref, tau)
    assert res["ok"] and res["cosine"] > 0.9999, res


def test_noalloc_matches_workspace_entry_two_calls_in_a_row():
    # each kind: a larger call, then a smaller one on the same static scratch
    for case in CASES:
        _run_case(*case)


def test_noalloc_repeat_after_other_shapes_is_stable():
    # the counters the previous calls left at zero serve the next calls
    _run_case(*CASES[0])
    _run_case(*CASES[2])


def test_noalloc_refuses_plans_beyond_the_static_scratch():
    lib = _lib.load()
    m = n = k = 4096
    cfg = ops.make_config("t256x256panel", 8)
    need = lib.fp8_scaled_mm_workspace_size(ops.KIND_CHANNELWISE, m, n, k, ctypes.byref(cfg))
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    a = torch.zeros((m, k), dtype=torch.uint8, device=device())
    b = torch.zeros((n, k), dtype=torch.uint8, device=device())
    sa = torch.ones(m, dtype=torch.float32, device=device())
    sb = torch.ones(n, dtype=torch.float32, device=device())
    out = torch.full((m, n), 7.0, dtype=torch.bfloat16, device=device())
    st = _noalloc(ops.KIND_CHANNELWISE, a, b, sa, 0, sb, None, out, m, n, k, cfg)
    assert st == _lib.FP8_ERR_WORKSPACE
    assert b"static scratch" in lib.fp8_last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call must not touch the output"
