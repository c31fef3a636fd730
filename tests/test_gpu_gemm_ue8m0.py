"""GPU parity of the blockwise GEMM with UE8M0 (power-of-two) scales against
the fp64 blockwise oracle.

Activations and weights are quantized by the oracle with scale_ue8m0 (the
quantizer flag of the PR 27896 digest's kernel call; the GPU quantizer is
checked bit-exact against the same oracle elsewhere), and the same bytes go to
both sides. The 16x16 256x256 tile and the 256x128 and 128x64 (8-wave)
panel tiles apply the scales inside gfx950's block-scaled MFMA; the other
tiles run the fp32-promotion kernels. Acceptance
as for every GEMM (oracle.check_gemm): max|err| <= 1e-2 max|ref| and per
element |err| <= 2^-6 |ref| + tau.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import ops, synth
from gpu_common import activations, bf16_to_f64, device, gpu, sample_rows, say

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=8)
def _act(wl, m, k):
    return oracle.quant_per_token_group(activations(wl, m, k).float().numpy(), 128, scale_ue8m0=True)


@functools.lru_cache(maxsize=4)
def _weight(wl, n, k):
    return oracle.quant_weight_blockwise(synth.weights(wl, n, k).numpy(), scale_ue8m0=True)


def _case(wl, m, n, k, config=None, with_bias=False, poison=False, row_align=4):
    a, sa = _act(wl, m, k)
    b, sb = _weight(wl, n, k)
    assert np.all((sa.view(np.uint32) & 0x7FFFFF) == 0) and np.all((sb.view(np.uint32) & 0x7FFFFF) == 0)
    bias = synth.bias(wl, n) if with_bias else None
    m_pad = ops.padded_rows(m, row_align)
    a_dev = torch.full((m_pad, k), 0x7F if poison else 0, dtype=torch.uint8, device=device())
    a_dev[:m] = gpu(a)
    s_store = torch.full((k // 128, m_pad), float("nan") if poison else 1.0, dtype=torch.float32,
                         device=device())
    s_store[:, :m] = gpu(sa.T.copy())
    say("blockwise ue8m0", wl, m, n, k, "poison" if poison else "",
        config.as_dict() if config is not None else "")
    out = ops.scaled_mm_blockwise(a_dev, gpu(b), s_store.transpose(0, 1), gpu(sb),
                                  gpu(bias) if bias is not None else None, m=m, config=config,
                                  scale_ue8m0=True)
    torch.cuda.synchronize()
    rows = sample_rows(m) if m * n > 4_000_000 else np.arange(m)
    bias64 = bias.float().numpy() if bias is not None else None
    ref = oracle.scaled_mm_blockwise(a[rows], b, sa[rows], sb, bias64)
    tau = oracle.gemm_tolerance_blockwise(a[rows], b, sa[rows], sb)
    res = oracle.check_gemm(bf16_to_f64(out)[rows], ref, tau)
    say("ue8m0", wl, m, n, k, {kk: (round(v, 8) if isinstance(v, float) else v) for kk, v in res.items()})
    assert out.shape == (m, n)
    assert res["ok"], res
    assert res["cosine"] > 0.9999
    return out


BW16_CASES = [
    (1, 300, 384, 1024, False), (3, 300, 384, 1024, True), (1, 1, 128, 128, False),
    (1, 257, 256, 384, False), (2, 513, 640, 2048, True), (4, 129, 384, 4096, False),
    (1, 4096, 3072, 4096, False), (1, 8192, 4096, 4096, True)]


@pytest.mark.parametrize("split_k,m,n,k,bias", BW16_CASES,
                         ids=[f"sk{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}{'-bias' if c[4] else ''}"
                              for c in BW16_CASES])
def test_ue8m0_block_scaled_mfma_tile(split_k, m, n, k, bias):
    """The 256x256 ping-pong tile with the scales inside the MFMA: one to many
    stages, ragged M, N overhanging the tile, uneven split-K, bias, and the
    MoE-expert and o_proj prefill shapes."""
    _case("ue8m0-bw16", m, n, k, config=ops.make_config("t256x256bw16", split_k), with_bias=bias)


def test_ue8m0_weight_scale_table_limits():
    """UE8M0 exponents from the once-per-tile weight scale table (K = 32768)
    and from the per-stage copies beyond it (K = 33024)."""
    for k in (32768, 33024):
        _case("ue8m0-kb", 300, 384, k, config=ops.make_config("t256x256bw16"))


def test_ue8m0_poisoned_pad_rows_and_fallback():
    """NaN pad scales and 0x7F pad codes stay out of the outputs; an unaligned
    scale column (row alignment 1) runs the same tile with its scales copied
    one per lane."""
    _case("ue8m0-poison", 301, 512, 1024, config=ops.make_config("t256x256bw16", 2), poison=True)
    _case("ue8m0-ld", 301, 384, 1024, config=ops.make_config("t256x256bw16", 1), row_align=1)


DEFAULT_CASES = ([("block_7168", m, 7168, 7168) for m in (1, 13, 64, 256)]
                 + [("block_moe", m, n, k) for n, k in ((3072, 4096), (4096, 1536)) for m in (4, 64, 4096)])


@pytest.mark.parametrize("wl,m,n,k", DEFAULT_CASES, ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in DEFAULT_CASES])
def test_ue8m0_default_configs(wl, m, n, k):
    """Table / heuristic choice at the blockwise workloads' shapes: small M runs
    the fp32-promotion kernels on power-of-two scales, large M the MFMA-scaled
    tile."""
    _case(wl + "-ue8m0", m, n, k)


def test_ue8m0_matches_fp32_promotion_tile():
    """The same power-of-two inputs through the fp32-promotion 16x16 tile and
    the MFMA-scaled one: both within tolerance of the oracle and of each other."""
    m, n, k = 512, 1024, 2048
    out_e8 = _case("ue8m0-vs", m, n, k, config=ops.make_config("t256x256bw16"))
    a, sa = _act("ue8m0-vs", m, k)
    b, sb = _weight("ue8m0-vs", n, k)
    st = gpu(sa.T.copy())
    out_f32 = ops.scaled_mm_blockwise(gpu(a), gpu(b), st.transpose(0, 1), gpu(sb), m=m,
                                      config=ops.make_config("t256x256bw16"))
    torch.cuda.synchronize()
    d = (out_e8.float() - out_f32.float()).abs().max().item()
    ref_max = out_f32.float().abs().max().item()
    assert d <= 1e-2 * ref_max, (d, ref_max)


E8_PANEL_VARIANTS = [("t256x128panel", 1), ("t256x128panel", 3), ("t128x128panel", 1), ("t128x64panel", 2),
                     ("t64x64panel", 1), ("t64x64deep", 2), ("t128x64deep", 1), ("t128x128panel8", 2),
                     ("t128x64panel8", 1), ("t32x32deep", 2), ("t64x32deep", 1)]


@pytest.mark.parametrize("variant,split_k", E8_PANEL_VARIANTS, ids=[f"{v}-sk{s}" for v, s in E8_PANEL_VARIANTS])
def test_ue8m0_panel_tiles(variant, split_k):
    """Every 32x32-MFMA panel tile on power-of-two scales (the 256x128 and
    8-wave 128x64 tiles on the block-scaled MFMA, with no per-stage partial
    tile; the others promoting in fp32): ragged M, N not a multiple of the
    tile, several stages, split-K, bias."""
    _case("ue8m0-panel", 203, 384, 1536, config=ops.make_config(variant, split_k), with_bias=True)
