"""GPU parity of the scaled GEMMs against the fp64 oracle.

Inputs are quantized by the oracle (never by the HIP path) and the same bytes
go to both sides. Acceptance (oracle.check_gemm): max|err| <= 1e-2 max|ref| and
per element |err| <= 2^-6 |ref| + tau, tau being the fp32 summation bound of
the K-term accumulation. Full outputs are compared up to a few million
elements; larger workloads compare a sample of rows (rows are independent),
always including the first and last rows.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import ops, synth
from gpu_common import (act_group, act_per_token, bf16_to_f64, device, gpu, sample_rows, say,
                        weight_blockwise, weight_channelwise)

pytestmark = pytest.mark.gpu


def _check(out_rows, ref, tol, label):
    res = oracle.check_gemm(out_rows, ref, tol)
    say(label, {k: (round(v, 8) if isinstance(v, float) else v) for k, v in res.items()})
    assert res["ok"], (label, res)
    assert res["cosine"] > 0.9999
    return res


def _channelwise_case(wl, m, n, k, outliers, with_bias, config=None, sample=True):
    a, sa = act_per_token(wl, m, k, outliers)
    b, sb = weight_channelwise(wl, n, k)
    bias = synth.bias(wl, n) if with_bias else None
    say("channelwise", wl, m, n, k, config.as_dict() if config is not None else "table/default")
    out = ops.scaled_mm_channelwise(gpu(a), gpu(b), gpu(sa), gpu(sb),
                                    gpu(bias) if bias is not None else None, config=config)
    torch.cuda.synchronize()
    rows = sample_rows(m) if (sample and m * n > 4_000_000) else np.arange(m)
    bias64 = bias.float().numpy() if bias is not None else None
    ref = oracle.scaled_mm_channelwise(a[rows], b, sa[rows], sb, bias64)
    tau = oracle.gemm_tolerance_channelwise(a[rows], b, sa[rows], sb)
    got = bf16_to_f64(out)[rows]
    return _check(got, ref, tau, f"cw {wl} M={m} N={n} K={k}"), out


CW_CASES = (
    [("small", 16, 256, 512, 0.0, False)]
    + [("o_proj", m, 4096, 4096, 0.01, False)
       for m in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192)]
    + [("qwen3_8b", m, n, k, 0.0, True) for n, k in ((6144, 4096), (4096, 12288), (24576, 4096))
       for m in (1, 64, 512, 8192)]
    # M between the skinny kernel and the 64-row tiles: the tile table sends
    # some of these to the 32- and 64-wide deep-ring tiles
    + [("qwen3_8b", m, n, k, 0.0, True) for n, k in ((6144, 4096), (4096, 12288), (24576, 4096))
       for m in (8, 21, 32)]
    + [("small", m, 256, 512, 0.0, False) for m in (8, 32, 100)]
)


@pytest.mark.parametrize("wl,m,n,k,outl,bias", CW_CASES, ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in CW_CASES])
def test_channelwise_workloads(wl, m, n, k, outl, bias):
    _channelwise_case(wl, m, n, k, outl, bias)


def _blockwise_case(wl, m, n, k, config=None, with_bias=False, poison=False, row_align=4):
    a, sa = act_group(wl, m, k)
    b, sb = weight_blockwise(wl, n, k)
    bias = synth.bias(wl, n) if with_bias else None
    m_pad = ops.padded_rows(m, row_align)
    a_dev = torch.full((m_pad, k), 0x7F if poison else 0, dtype=torch.uint8, device=device())
    a_dev[:m] = gpu(a)
    s_store = torch.full((k // 128, m_pad), float("nan") if poison else 0.0, dtype=torch.float32,
                         device=device())
    s_store[:, :m] = gpu(sa.T.copy())
    say("blockwise", wl, m, n, k, "poison" if poison else "", config.as_dict() if config is not None else "")
    out = ops.scaled_mm_blockwise(a_dev, gpu(b), s_store.transpose(0, 1), gpu(sb),
                                  gpu(bias) if bias is not None else None, m=m, config=config)
    torch.cuda.synchronize()
    rows = sample_rows(m) if m * n > 4_000_000 else np.arange(m)
    bias64 = bias.float().numpy() if bias is not None else None
    ref = oracle.scaled_mm_blockwise(a[rows], b, sa[rows], sb, bias64)
    tau = oracle.gemm_tolerance_blockwise(a[rows], b, sa[rows], sb)
    got = bf16_to_f64(out)[rows]
    assert out.shape == (m, n)
    return _check(got, ref, tau, f"bw {wl} M={m} N={n} K={k}"), out


BW_CASES = ([("block_7168", m, 7168, 7168) for m in (1, 2, 3, 5, 7, 13, 31, 64, 256)]
            + [("block_moe", m, n, k) for n, k in ((3072, 4096), (4096, 1536)) for m in (1, 4, 16, 64, 4096)]
            + [("block_7168", m, 7168, 7168) for m in (16, 32, 48)])


@pytest.mark.parametrize("wl,m,n,k", BW_CASES, ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in BW_CASES])
def test_blockwise_workloads(wl, m, n, k):
    _blockwise_case(wl, m, n, k)


# ---------------------------------------------------------------- every kernel variant
VARIANT_CASES = [(v, sk) for v, sk in (("skinny", 1), ("t64x64", 1), ("t64x64", 3), ("t128x128", 1),
                                       ("t128x128", 2), ("t256x128", 1), ("t256x128", 4),
                                       ("t256x256", 1), ("t256x256", 2), ("t256x256w8", 1),
                                       ("t256x128w8", 2), ("t128x128w8", 1), ("t128x64k256", 1),
                                       ("t128x64k256", 3), ("t64x128k256", 2), ("t128x128k256", 1),
                                       ("t128x128k256", 2))]


@pytest.mark.parametrize("variant,split_k", VARIANT_CASES, ids=[f"{v}-sk{s}" for v, s in VARIANT_CASES])
def test_channelwise_variants_ragged(variant, split_k):
    """Ragged M, N and K tails (K a multiple of 16 but not of 128)."""
    m = 29 if variant == "skinny" else 300
    n, k = 392, 1040
    cfg = ops.make_config(variant, split_k)
    _channelwise_case("ragged", m, n, k, 0.0, True, config=cfg, sample=False)


BW_VARIANTS = [(v, sk) for v, sk in (("skinny", 1), ("t64x64", 1), ("t64x64", 2), ("t128x128", 1),
                                     ("t128x128", 3), ("t256x128", 2), ("t256x128w8", 1),
                                     ("t128x128w8", 2), ("t128x64k256", 1), ("t128x64k256", 2),
                                     ("t64x128k256", 1), ("t128x128k256", 2))]


@pytest.mark.parametrize("variant,split_k", BW_VARIANTS, ids=[f"{v}-sk{s}" for v, s in BW_VARIANTS])
def test_blockwise_variants(variant, split_k):
    m = 30 if variant == "skinny" else 200
    _blockwise_case("bw-variants", m, 640, 1280, config=ops.make_config(variant, split_k),
                    with_bias=True)


# ---------------------------------------------------------------- decode weight stream
# (M, N, K): one 128-deep block, whole 1 KB K stages and a 128- or 384-deep
# tail stage, a ragged last group of 16 columns (channelwise), one round of
# workgroups over the compute units (four-slot ring) and more groups than
# compute units (an 80 KB ring: four slots at M = 1, two at M = 16).
DECODE_CASES = [(m, n, k) for (m, n, k) in ((1, 256, 128), (3, 384, 1152), (8, 640, 4096), (16, 512, 2176),
                                             (13, 4224, 3200), (16, 4224, 1024), (1, 4224, 7168),
                                             (5, 392, 1408))]


# Two and four activation tiles (M <= 32, 64): ragged last tile, one and
# several blocks per wave; the blockwise M = 64 case does not fit its scale
# table beside the ring and runs the 64x64 tile instead.
DECODE_WIDE_CASES = [("cw", 17, 392, 1152), ("cw", 32, 4224, 2048), ("cw", 33, 512, 4096),
                     ("cw", 64, 4096, 1024), ("bw", 24, 384, 4096), ("bw", 40, 512, 1024),
                     ("bw", 64, 256, 2048)]


@pytest.mark.parametrize("kind,m,n,k", DECODE_WIDE_CASES, ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in DECODE_WIDE_CASES])
def test_decode_variant_wide_m(kind, m, n, k):
    cfg = ops.make_config("decode")
    if kind == "cw":
        _, o1 = _channelwise_case("decode-wide", m, n, k, 0.01, True, config=cfg, sample=False)
        if m <= 32:
            _, o2 = _channelwise_case("decode-wide", m, n, k, 0.01, True, config=ops.make_config("skinny"),
                                      sample=False)
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    else:
        _, o1 = _blockwise_case("decode-wide", m, n, k, config=cfg, with_bias=True)
        _, o3 = _blockwise_case("decode-wide", m, n, k, config=ops.make_config("decode", 2), with_bias=True)


@pytest.mark.parametrize("m,n,k", DECODE_CASES, ids=[f"M{m}-N{n}-K{k}" for m, n, k in DECODE_CASES])
def test_decode_variant_parity_and_same_bits_as_skinny(m, n, k):
    """The decode stream against the oracle, and bit-identical to the skinny
    kernel: both take the K blocks in the same order and sum the waves'
    partial tiles in wave order."""
    cfg, sk = ops.make_config("decode"), ops.make_config("skinny")
    _, o1 = _channelwise_case("decode", m, n, k, 0.01, True, config=cfg, sample=False)
    _, o2 = _channelwise_case("decode", m, n, k, 0.01, True, config=sk, sample=False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    if n % 128 == 0:
        _, b1 = _blockwise_case("decode", m, n, k, config=cfg, with_bias=True, row_align=4)
        _, b2 = _blockwise_case("decode", m, n, k, config=sk, with_bias=True, row_align=4)
        assert torch.equal(b1.view(torch.int16), b2.view(torch.int16))


DECODE_SPLIT_CASES = [("cw", 1, 4096, 4096, 2), ("cw", 16, 520, 12288, 3), ("cw", 5, 392, 1152, 2),
                      ("bw", 3, 4096, 7168, 4), ("bw", 16, 512, 2048, 2), ("bw", 1, 384, 4224, 5)]


@pytest.mark.parametrize("kind,m,n,k,split", DECODE_SPLIT_CASES,
                         ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}-sk{c[4]}" for c in DECODE_SPLIT_CASES])
def test_decode_variant_split_k(kind, m, n, k, split):
    """The decode stream split over K (each split a run of every wave's
    blocks, partials summed in split order): within the tolerance of the
    oracle, including splits of unequal length and a wave with no block in
    the last split, and the same bits on a repeat (the arrival counters
    reset)."""
    cfg = ops.make_config("decode", split)
    if kind == "cw":
        _, o1 = _channelwise_case("decode-split", m, n, k, 0.01, True, config=cfg, sample=False)
        _, o2 = _channelwise_case("decode-split", m, n, k, 0.01, True, config=cfg, sample=False)
    else:
        _, o1 = _blockwise_case("decode-split", m, n, k, config=cfg, with_bias=True)
        _, o2 = _blockwise_case("decode-split", m, n, k, config=cfg, with_bias=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_decode_variant_pad_rows_and_scale_stride():
    """Blockwise decode with NaN-poisoned pad rows and scales, and with an
    unaligned scale stride (row_alignment 1): the first M rows match a clean
    run bit for bit."""
    cfg = ops.make_config("decode")
    for m in (1, 3, 13):
        _, clean = _blockwise_case("decode-pad", m, 4224, 2048, config=cfg)
        _, dirty = _blockwise_case("decode-pad", m, 4224, 2048, config=cfg, poison=True)
        _, ld1 = _blockwise_case("decode-pad", m, 4224, 2048, config=cfg, row_align=1)
        assert torch.equal(clean.view(torch.int16), dirty.view(torch.int16)), m
        assert torch.equal(clean.view(torch.int16), ld1.view(torch.int16)), m


def test_blockwise_poisoned_pad_rows_do_not_leak():
    """Pad rows filled with NaN codes and NaN scales: the first M rows must be
    bit-identical to a run with zero pads (rows are independent)."""
    for m in (1, 3, 5, 13, 31):
        _, clean = _blockwise_case("block_7168", m, 7168, 7168)
        _, dirty = _blockwise_case("block_7168", m, 7168, 7168, poison=True)
        assert torch.equal(clean.view(torch.int16), dirty.view(torch.int16)), m


def test_deterministic_repeat():
    for cfg in (None, ops.make_config("t128x128", 4), ops.make_config("t64x64", 2)):
        _, o1 = _channelwise_case("o_proj", 256, 4096, 4096, 0.01, False, config=cfg, sample=False)
        _, o2 = _channelwise_case("o_proj", 256, 4096, 4096, 0.01, False, config=cfg, sample=False)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_split_k_agrees_within_tolerance():
    outs = []
    for cfg in (ops.make_config("t64x64", 1), ops.make_config("t64x64", 8)):
        _, o = _channelwise_case("o_proj", 128, 4096, 4096, 0.01, False, config=cfg, sample=False)
        outs.append(bf16_to_f64(o))
    diff = np.abs(outs[0] - outs[1])
    assert np.max(diff) <= 2.0 ** -6 * np.max(np.abs(outs[0]))


def test_exact_identities():
    """Bit-exact cases: all-ones operands with power-of-two scales; A = 0 gives
    bf16(bias); identity-pattern weight reproduces dec(A) * scales."""
    dev = device()
    k = 512
    a = torch.full((20, k), 0x38, dtype=torch.uint8, device=dev)
    b = torch.full((48, k), 0x38, dtype=torch.uint8, device=dev)
    sa = torch.full((20,), 2.0 ** -3, device=dev)
    sb = torch.full((48,), 2.0 ** -5, device=dev)
    for cfg in (ops.make_config("skinny"), ops.make_config("t64x64", 2)):
        out = ops.scaled_mm_channelwise(a, b, sa, sb, config=cfg)
        torch.cuda.synchronize()
        assert torch.all(out.float() == k * 2.0 ** -8)
    bias = synth.bias("ident", 48)
    z = torch.zeros((20, k), dtype=torch.uint8, device=dev)
    out = ops.scaled_mm_channelwise(z, b, sa, sb, gpu(bias))
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), bias.expand(20, 48).contiguous().view(torch.int16))
    codes = synth.random_codes("ident-a", (20, 128))
    eye = torch.zeros((128, 128), dtype=torch.uint8)
    eye[torch.arange(128), torch.arange(128)] = 0x38
    sa2 = torch.tensor([2.0 ** -(i % 5) for i in range(20)], dtype=torch.float32)
    out = ops.scaled_mm_channelwise(gpu(codes), gpu(eye), gpu(sa2), torch.full((128,), 4.0, device=dev))
    torch.cuda.synchronize()
    want = oracle.bf16_round(oracle.decode(codes.numpy()) * sa2.numpy()[:, None].astype(np.float64) * 4.0)
    assert np.array_equal(bf16_to_f64(out), want)


def test_blockwise_uniform_scales_match_channelwise():
    m, n, k = 64, 1024, 2048
    a = synth.random_codes("uni-a", (m, k))
    b = synth.random_codes("uni-b", (n, k))
    sa = synth.positive_scales("uni-sa", (m,))
    sbb = synth.positive_scales("uni-sb", (n // 128,))
    out_c = ops.scaled_mm_channelwise(gpu(a), gpu(b), gpu(sa), gpu(sbb.repeat_interleave(128)))
    s_store = gpu(sa[None, :].repeat(k // 128, 1).contiguous())
    out_b = ops.scaled_mm_blockwise(gpu(a), gpu(b), s_store.transpose(0, 1),
                                    gpu(sbb[:, None].repeat(1, k // 128).contiguous()))
    torch.cuda.synchronize()
    oc, ob = bf16_to_f64(out_c), bf16_to_f64(out_b)
    assert np.max(np.abs(oc - ob)) <= 2.0 ** -6 * np.max(np.abs(oc))


def test_empty_m_is_noop():
    dev = device()
    a = torch.empty((0, 512), dtype=torch.uint8, device=dev)
    b = torch.zeros((256, 512), dtype=torch.uint8, device=dev)
    out = ops.scaled_mm_channelwise(a, b, torch.empty(0, device=dev), torch.ones(256, device=dev))
    assert out.shape == (0, 256)


def test_linear_wrappers_match_oracle():
    """The user-facing linears (quant + GEMM) against the oracle pipeline."""
    x = synth.activations("linear", 37, 1024)
    w = synth.weights("linear", 384, 1024).numpy()
    bias = synth.bias("linear", 384)
    wq, ws = oracle.quant_weight_per_channel(w)
    say("linear_channelwise")
    y = ops.linear_channelwise(gpu(x), gpu(wq), gpu(ws), gpu(bias))
    torch.cuda.synchronize()
    aq, as_ = oracle.quant_per_token(x.float().numpy())
    ref = oracle.scaled_mm_channelwise(aq, wq, as_, ws, bias.float().numpy())
    tau = oracle.gemm_tolerance_channelwise(aq, wq, as_, ws)
    _check(bf16_to_f64(y), ref, tau, "linear_channelwise")
    bq, bs = oracle.quant_weight_blockwise(w)
    say("linear_blockwise")
    y = ops.linear_blockwise(gpu(x), gpu(bq), gpu(bs), gpu(bias))
    torch.cuda.synchronize()
    gq, gs = oracle.quant_per_token_group(x.float().numpy(), 128)
    ref = oracle.scaled_mm_blockwise(gq, bq, gs, bs, bias.float().numpy())
    tau = oracle.gemm_tolerance_blockwise(gq, bq, gs, bs)
    assert y.shape == (37, 384)
    _check(bf16_to_f64(y), ref, tau, "linear_blockwise")


def test_split_k_back_to_back_calls_see_fresh_partials():
    """Two split-K calls of the same shape on different data, back to back on
    one workspace: the second must not read the first call's partial tiles."""
    for cfg in (ops.make_config("t64x64", 4), ops.make_config("t128x128k256", 2)):
        _channelwise_case("o_proj", 192, 4096, 4096, 0.01, False, config=cfg, sample=False)
        _channelwise_case("qwen3_8b", 192, 4096, 4096, 0.0, True, config=cfg, sample=False)
        _channelwise_case("o_proj", 192, 4096, 4096, 0.01, False, config=cfg, sample=False)


DMA_CASES = [(v, sk, m, n, k) for v, sk, m, n, k in (
    ("t256x256dma", 1, 300, 392, 1024), ("t256x256dma", 3, 300, 392, 1024),
    ("t256x128dma", 1, 300, 392, 1024), ("t256x128dma", 2, 513, 200, 2048),
    ("t128x128dma", 1, 300, 392, 1024), ("t128x128dma", 4, 129, 392, 4096),
    ("t256x256dma", 1, 1, 256, 64), ("t256x256dma", 1, 4096, 4096, 4096))]


@pytest.mark.parametrize("variant,split_k,m,n,k", DMA_CASES,
                         ids=[f"{c[0]}-sk{c[1]}-M{c[2]}-N{c[3]}-K{c[4]}" for c in DMA_CASES])
def test_channelwise_dma_variants(variant, split_k, m, n, k):
    """The LDS-DMA pipelined tiles (K a multiple of 64): ragged M and N, one to
    many stages, split-K, and a full-size o_proj tile grid."""
    _channelwise_case("dma", m, n, k, 0.0, True, config=ops.make_config(variant, split_k))


def test_dma_variant_falls_back_when_k_not_multiple_of_64():
    _channelwise_case("dma-fallback", 200, 264, 1040, 0.0, True, config=ops.make_config("t256x256dma", 1),
                      sample=False)
    _blockwise_case("dma-fallback-bw", 64, 256, 1024, config=ops.make_config("t128x128dma", 1))


PANEL_CASES = [
    (1, 300, 392, 1024), (3, 300, 392, 1024), (2, 513, 200, 2048), (1, 1, 256, 128),
    (1, 257, 264, 256), (1, 300, 392, 384), (4, 129, 392, 4096), (3, 64, 520, 1280),
    (3, 300, 392, 384), (2, 1, 520, 256), (1, 4096, 4096, 4096)]


@pytest.mark.parametrize("split_k,m,n,k", PANEL_CASES,
                         ids=[f"sk{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in PANEL_CASES])
def test_channelwise_panel_variant(split_k, m, n, k):
    """The 256x256 ping-pong tile, channelwise (K a multiple of 128): one to
    many stages against its four-slot ring, ragged M and N, split-K with
    uneven splits and with one stage per split, and a full o_proj tile grid."""
    _channelwise_case("panel", m, n, k, 0.0, True, config=ops.make_config("t256x256panel", split_k))


def test_panel_variant_falls_back_when_k_not_multiple_of_128():
    _channelwise_case("panel-fallback", 200, 264, 1088, 0.0, True,
                      config=ops.make_config("t256x256panel", 2), sample=False)
    _blockwise_case("panel-fallback-bw", 64, 256, 1024, config=ops.make_config("t256x256panel", 1))


BW_PANEL_CASES = [
    (1, 300, 384, 1024, False), (3, 300, 384, 1024, True), (1, 1, 128, 128, False),
    (1, 257, 256, 384, False), (2, 513, 640, 2048, True), (4, 129, 384, 4096, False),
    (3, 257, 384, 384, True), (2, 2, 256, 256, False), (1, 4096, 4096, 4096, False)]


@pytest.mark.parametrize("split_k,m,n,k,bias", BW_PANEL_CASES,
                         ids=[f"sk{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}{'-bias' if c[4] else ''}"
                              for c in BW_PANEL_CASES])
def test_blockwise_panel_variant(split_k, m, n, k, bias):
    """The 256x128 panel-ring tile, blockwise: per-stage scales staged with the
    B panels, one to many stages, ragged M, uneven split-K, bias, full grid."""
    _blockwise_case("bw-panel", m, n, k, config=ops.make_config("t256x128panel", split_k), with_bias=bias)


@pytest.mark.parametrize("split_k,m,n,k,bias", BW_PANEL_CASES,
                         ids=[f"sk{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}{'-bias' if c[4] else ''}"
                              for c in BW_PANEL_CASES])
def test_blockwise_256x256_mfma16(split_k, m, n, k, bias):
    """The blockwise 256x256 ping-pong tile on 16x16x128 MFMAs (four-slot
    ring, one promotion per MFMA): the same stage counts, ragged shapes and
    splits, down to one stage per split."""
    _blockwise_case("bw16", m, n, k, config=ops.make_config("t256x256bw16", split_k), with_bias=bias)


def test_blockwise_256x256_mfma16_weight_scale_table_limits():
    """The tile's weight block scales come from a table filled once per tile
    for up to 256 K blocks (K = 32768: all four 64-block pieces of it), and
    with every stage beyond that (K = 33024)."""
    for k in (32768, 33024):
        _blockwise_case("bw16-kb", 300, 384, k, config=ops.make_config("t256x256bw16"), with_bias=True)
    _blockwise_case("bw16-kb-split", 257, 256, 32768, config=ops.make_config("t256x256bw16", 3))


def test_blockwise_256x256_mfma16_poison_and_fallbacks():
    """NaN pad rows stay out; an unaligned scale column (stride not a multiple
    of 4) runs the same tile with its scales copied one per lane; a
    channelwise request runs the channelwise form of the tile."""
    _blockwise_case("bw16-poison", 301, 512, 1024, config=ops.make_config("t256x256bw16", 2), poison=True)
    _blockwise_case("bw16-ld", 301, 384, 1024, config=ops.make_config("t256x256bw16", 2), row_align=1)
    _channelwise_case("bw16-cw", 300, 392, 1024, 0.0, True, config=ops.make_config("t256x256bw16", 2),
                      sample=False)


def test_blockwise_panel_poisoned_padding():
    """Padded activation rows hold NaN codes and NaN scales; no valid row may see them."""
    _blockwise_case("bw-panel-poison", 301, 384, 1024, config=ops.make_config("t256x128panel", 2),
                    poison=True)


UNALIGNED_SCALE_CASES = [(v, sk, m, ra) for v, sk, m, ra in (
    ("t256x128panel", 2, 301, 1), ("t256x256bw16", 1, 517, 1), ("t256x256bw16", 2, 301, 2),
    ("t128x128panel", 1, 131, 3), ("t128x64panel8", 3, 197, 1), ("t64x64panel", 2, 77, 2),
    ("t64x64deep", 1, 61, 1), ("t32x32deep", 2, 45, 3), ("t64x32deep", 1, 33, 1),
    ("t128x128panel8", 1, 129, 2), ("t128x64deep", 2, 150, 1))]


@pytest.mark.parametrize("variant,split_k,m,row_align", UNALIGNED_SCALE_CASES,
                         ids=[f"{c[0]}-sk{c[1]}-M{c[2]}-ra{c[3]}" for c in UNALIGNED_SCALE_CASES])
def test_blockwise_panel_unaligned_scale_column(variant, split_k, m, row_align):
    """Activation-scale column strides that are not a multiple of 4 (row
    alignment 1, 2 or 3 on a ragged M) on every blockwise panel tile: the
    per-stage scales travel one per lane instead of in 16-byte pieces."""
    _blockwise_case("bw-panel-ld", m, 384, 1024, config=ops.make_config(variant, split_k), row_align=row_align,
                    poison=True)


def test_blockwise_default_unaligned_scale_column_large_m():
    """M = 4097 with row alignment 1 at the default tile (the 256x256
    ping-pong tile): a column stride of 4097 scales."""
    _blockwise_case("bw-ld-4097", 4097, 4096, 4096, row_align=1)


CW_PANEL128_CASES = [(1, 300, 392, 1024), (2, 300, 392, 1024), (1, 2048, 4096, 4096)]


@pytest.mark.parametrize("split_k,m,n,k", CW_PANEL128_CASES,
                         ids=[f"sk{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in CW_PANEL128_CASES])
def test_channelwise_panel128_variant(split_k, m, n, k):
    _channelwise_case("cw-panel128", m, n, k, 0.0, True, config=ops.make_config("t256x128panel", split_k))


SMALL_PANEL_CASES = [(v, kind, sk, m, n, k) for v in ("t128x128panel", "t128x64panel", "t64x64panel")
                     for kind, sk, m, n, k in (("cw", 1, 300, 392, 1024), ("cw", 3, 129, 392, 4096),
                                               ("cw", 1, 1, 64, 128), ("bw", 2, 300, 384, 1024),
                                               ("bw", 1, 65, 256, 384))]


@pytest.mark.parametrize("variant,kind,split_k,m,n,k", SMALL_PANEL_CASES,
                         ids=[f"{c[0]}-{c[1]}-sk{c[2]}-M{c[3]}-N{c[4]}-K{c[5]}" for c in SMALL_PANEL_CASES])
def test_small_panel_variants(variant, kind, split_k, m, n, k):
    """The 4-wave panel-ring tiles, both kinds: ragged M and N, one to many
    stages, uneven split-K."""
    cfg = ops.make_config(variant, split_k)
    if kind == "cw":
        _channelwise_case("small-panel", m, n, k, 0.0, True, config=cfg)
    else:
        _blockwise_case("small-panel", m, n, k, config=cfg, with_bias=True)


DEEP_CASES = [(v, kind, sk, m, n, k) for v in ("t64x64deep", "t128x64deep", "t128x128panel8", "t128x64panel8",
                                                "t32x32deep", "t64x32deep")
              for kind, sk, m, n, k in (("cw", 1, 300, 392, 1024), ("cw", 2, 129, 392, 4096),
                                        ("cw", 1, 1, 64, 128), ("cw", 1, 65, 256, 768),
                                        ("bw", 2, 300, 384, 1024), ("bw", 1, 65, 256, 768),
                                        ("bw", 1, 70, 256, 4096))]


@pytest.mark.parametrize("variant,kind,split_k,m,n,k", DEEP_CASES,
                         ids=[f"{c[0]}-{c[1]}-sk{c[2]}-M{c[3]}-N{c[4]}-K{c[5]}" for c in DEEP_CASES])
def test_deep_ring_variants(variant, kind, split_k, m, n, k):
    """Deep-ring (7- to 17-slot) and 8-wave small panel tiles: stage counts
    below, at and above the ring depth, ragged M and N, split-K."""
    cfg = ops.make_config(variant, split_k)
    if kind == "cw":
        _channelwise_case("deep-panel", m, n, k, 0.0, True, config=cfg)
    else:
        _blockwise_case("deep-panel", m, n, k, config=cfg, with_bias=True)



def test_narrow_tiles_fall_back_when_k_not_multiple_of_128():
    """The register-staged 32x32 and 64x32 tiles behind the narrow panel
    variants (channelwise K % 128 != 0), with split-K on a ragged M."""
    _channelwise_case("narrow-fallback", 70, 200, 1088, 0.0, True, config=ops.make_config("t32x32deep", 2),
                      sample=False)
    _channelwise_case("narrow-fallback", 70, 200, 1088, 0.0, True, config=ops.make_config("t64x32deep", 3),
                      sample=False)


SPLIT4_CASES = [  # (variant, kind, split_k, M, N, K): split 4 as the tile tables choose it at M <= 128,
    # and requests the host clamps (more splits than 128-deep stages: K = 256 -> 2 splits,
    # K = 384 -> 3, K = 640 -> 3 uneven splits of 2, 2, 1 stages)
    ("t64x32deep", "cw", 4, 64, 392, 4096), ("t64x64deep", "cw", 4, 61, 256, 12288),
    ("t64x64panel", "bw", 4, 37, 384, 1024), ("t32x32deep", "bw", 4, 16, 7168, 7168),
    ("t128x64panel", "cw", 4, 100, 512, 4096), ("t32x32deep", "cw", 4, 20, 200, 256),
    ("t64x64deep", "bw", 4, 64, 256, 384), ("t64x32deep", "cw", 4, 33, 136, 640),
    ("t64x64", "cw", 8, 33, 128, 512), ("t128x64k256", "bw", 3, 70, 256, 256)]


@pytest.mark.parametrize("variant,kind,split_k,m,n,k", SPLIT4_CASES,
                         ids=[f"{c[0]}-{c[1]}-sk{c[2]}-M{c[3]}-N{c[4]}-K{c[5]}" for c in SPLIT4_CASES])
def test_split_k_four_and_clamped(variant, kind, split_k, m, n, k):
    """Split-K partials exchanged in 16-byte device-coherent pieces: split 4
    on the narrow deep-ring and panel tiles, and split requests above the
    number of K stages (the host lowers them)."""
    cfg = ops.make_config(variant, split_k)
    if kind == "cw":
        _channelwise_case("split4", m, n, k, 0.0, True, config=cfg)
    else:
        _blockwise_case("split4", m, n, k, config=cfg, with_bias=True)


def test_panel_split_k_deterministic_and_fresh_partials():
    """Panel-tile split-K: the same call twice gives the same bits, and calls
    on other data in between (same workspace, same tile count) leave nothing
    behind that the next call reads."""
    for cfg in (ops.make_config("t64x32deep", 4), ops.make_config("t64x64panel", 2)):
        _, o1 = _channelwise_case("o_proj", 96, 4096, 4096, 0.01, False, config=cfg, sample=False)
        _channelwise_case("qwen3_8b", 96, 4096, 4096, 0.0, True, config=cfg, sample=False)
        _, o2 = _channelwise_case("o_proj", 96, 4096, 4096, 0.01, False, config=cfg, sample=False)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


DEFAULT_SPLIT_CASES = [("cw", 64, 2048, 8192), ("cw", 100, 4096, 5120), ("bw", 96, 1536, 7168), ("bw", 48, 5120, 5120)]


@pytest.mark.parametrize("kind,m,n,k", DEFAULT_SPLIT_CASES,
                         ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in DEFAULT_SPLIT_CASES])
def test_default_heuristic_split_k(kind, m, n, k):
    """Shapes with no tile table, where the default heuristic splits K (2 or 4
    splits of the 64x64 tiles at 32 < M <= 128)."""
    kid = ops.KIND_CHANNELWISE if kind == "cw" else ops.KIND_BLOCKWISE
    cfg, hit = ops.tile_config(kid, n, k, m)
    assert not hit and cfg["split_k"] > 1, cfg
    if kind == "cw":
        _channelwise_case("default-split", m, n, k, 0.0, True)
    else:
        _blockwise_case("default-split", m, n, k, with_bias=True)


NARROW_DEFAULT_CASES = [("cw", 16, 14336, 4096, "t32x32deep"), ("cw", 32, 5120, 5120, "t32x32deep"),
                        ("bw", 32, 12288, 7168, "t32x32deep"), ("cw", 8, 5120, 5120, "decode"),
                        ("bw", 12, 5120, 5120, "decode"), ("cw", 3, 14336, 4096, "decode")]


@pytest.mark.parametrize("kind,m,n,k,variant", NARROW_DEFAULT_CASES,
                         ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in NARROW_DEFAULT_CASES])
def test_default_narrow_tile_on_wide_weights(kind, m, n, k, variant):
    """Untabled wide weights at M = 3..32: the default heuristic takes the
    decode stream (two workgroups per compute unit) up to 16 rows where the
    column groups run in at most ~3.5 rounds (any round count at M <= 4),
    else the 32x32 deep-ring tile (split over long K), instead of the
    register-staged weight stream."""
    kid = ops.KIND_CHANNELWISE if kind == "cw" else ops.KIND_BLOCKWISE
    cfg, hit = ops.tile_config(kid, n, k, m)
    assert not hit and cfg["variant"] == variant, cfg
    if kind == "cw":
        _channelwise_case("narrow-default", m, n, k, 0.0, True)
    else:
        _blockwise_case("narrow-default", m, n, k, with_bias=True)
