"""GPU parity of the quantizer variants against the oracle, codes and scales
bit-exact: SiLU-and-mul fused into the per-token and per-token-group
quantizers (the step between a gate/up projection and its down projection:
Qwen3-8B's 24576 -> 12288 and the MoE expert's 3072 -> 1536), UE8M0 scales,
and static per-tensor quantization with a given scale."""
import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import ops, synth
from gpu_common import activations, device, gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def _assert_codes(got_q, want_q):
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def _edge_rows(k):
    """Two [gate | up] rows (k >= 256). In row 0, group i of 16 columns has one
    special gate value: zeros of both signs, large positive gates, large
    negative gates on both sides of the -80 switch to fp64 and past fp32 (and
    fp64) overflow of e^-g, and tiny gates with huge up values; the up values
    of the group vary, so with 16-wide groups every group's own scale and codes
    show its values. Row 1 is ordinary data times 8."""
    x = synth.activations("silu-edge", 2, 2 * k).float().numpy()
    special = [(0.0, 1.0), (-0.0, 1.0), (90.0, 1.0), (1000.0, 0.5), (-79.5, 1.0), (-80.5, 1.0),
               (-85.0, 2.0), (-88.5, 3.0), (-89.0, 1.0), (-95.0, 1.0), (-100.0, 1.0),
               (-1000.0, 2.0), (1e-30, 1e25), (-1e-30, 1e25), (3.0e4, 1.0), (-3.0e4, 1.0)]
    for i, (g, mag) in enumerate(special):
        x[0, 16 * i:16 * (i + 1)] = g
        x[0, k + 16 * i:k + 16 * (i + 1)] *= mag
    x[1, :k] *= 8.0
    return torch.from_numpy(x).to(torch.bfloat16)


# ---------------------------------------------------------------- SiLU-and-mul
SILU_PT_CASES = (
    [("qwen3_8b_down_in", m, 12288) for m in (1, 64, 512, 2048)]
    + [("silu_small", m, k) for m, k in ((16, 512), (3, 48), (5, 16), (2, 20480), (1, 40960))]
)


@pytest.mark.parametrize("wl,m,k", SILU_PT_CASES, ids=[f"{c[0]}-M{c[1]}-K{c[2]}" for c in SILU_PT_CASES])
def test_silu_per_token_bit_exact(wl, m, k):
    x = activations(wl, m, 2 * k)
    say("silu_mul_quant_per_token", wl, m, k)
    q, s = ops.silu_mul_quant_per_token(gpu(x))
    torch.cuda.synchronize()
    want_q, want_s = oracle.silu_mul_quant_per_token(x.float().numpy())
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    _assert_codes(q.cpu().numpy(), want_q)


def test_silu_per_token_full_size_sampled_rows():
    """M = 8192 rows of the 24576-wide gate/up output; rows are independent, so
    sampled rows are checked against the oracle one by one."""
    m, k = 8192, 12288
    x = activations("qwen3_8b_down_in", m, 2 * k)
    say("silu_mul_quant_per_token full", m, k)
    q, s = ops.silu_mul_quant_per_token(gpu(x))
    torch.cuda.synchronize()
    rows = sample_rows(m, count=24)
    want_q, want_s = oracle.silu_mul_quant_per_token(x[rows].float().numpy())
    assert np.array_equal(s.cpu().numpy()[rows].view(np.uint32), want_s.view(np.uint32))
    _assert_codes(q.cpu().numpy()[rows], want_q)


SILU_GROUP_CASES = (
    [("block_moe_down_in", m, 1536, 128, 4) for m in (1, 4, 16, 64, 4096)]
    + [("qwen3_8b_down_in", m, 12288, 128, 4) for m in (1, 13, 256, 2048)]
    + [("silu_groups", m, 1024, g, ra) for g in (16, 32, 64) for m, ra in ((1, 4), (37, 4), (9, 8))]
)


@pytest.mark.parametrize("wl,m,k,g,ra", SILU_GROUP_CASES,
                         ids=[f"{c[0]}-M{c[1]}-K{c[2]}-G{c[3]}-ra{c[4]}" for c in SILU_GROUP_CASES])
def test_silu_group_bit_exact(wl, m, k, g, ra):
    x = activations(wl, m, 2 * k)
    say("silu_mul_quant_per_token_group", wl, m, k, g, ra)
    m_pad = ops.padded_rows(m, ra)
    q_buf = torch.full((m_pad, k), 0x7F, dtype=torch.uint8, device=device())
    s_buf = torch.full((k // g, m_pad), float("nan"), dtype=torch.float32, device=device())
    q, s = ops.silu_mul_quant_per_token_group(gpu(x), g, row_alignment=ra, out=q_buf,
                                              scale_storage=s_buf)
    torch.cuda.synchronize()
    assert q.shape == (m_pad, k) and s.shape == (m_pad, k // g) and s.stride() == (1, m_pad)
    want_q, want_s = oracle.silu_mul_quant_per_token_group(x.float().numpy(), g)
    flat_want = oracle.scales_col_major(want_s, m_pad)
    live = ~np.isnan(flat_want)
    got_s = s_buf.cpu().numpy().ravel()
    assert np.array_equal(got_s[live].view(np.uint32), flat_want[live].view(np.uint32))
    assert np.all(np.isnan(got_s[~live])), "pad scale entries were written"
    got_q = q.cpu().numpy()
    _assert_codes(got_q[:m], want_q)
    assert np.all(got_q[m:] == 0x7F), "pad rows were written"


@pytest.mark.parametrize("k", [256, 1536])
def test_silu_edge_gates(k):
    x = _edge_rows(k)
    say("silu edge gates", k)
    xg = gpu(x)
    q, s = ops.silu_mul_quant_per_token(xg)
    qg, sg = ops.silu_mul_quant_per_token_group(xg, 16, row_alignment=1)
    torch.cuda.synchronize()
    xf = x.float().numpy()
    want_q, want_s = oracle.silu_mul_quant_per_token(xf)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    _assert_codes(q.cpu().numpy(), want_q)
    want_qg, want_sg = oracle.silu_mul_quant_per_token_group(xf, 16)
    assert np.array_equal(sg.contiguous().cpu().numpy().view(np.uint32), want_sg.view(np.uint32))
    _assert_codes(qg.cpu().numpy(), want_qg)


def test_silu_strided_input():
    """Rows of x wider than 2K (ldx > 2K): only [0, 2K) of each row is read."""
    m, k = 9, 640
    base = activations("silu_strided", m, 2 * k + 64)
    x = gpu(base)[:, :2 * k]
    assert x.stride(0) == 2 * k + 64
    say("silu strided", m, k)
    q, s = ops.silu_mul_quant_per_token(x)
    qg, sg = ops.silu_mul_quant_per_token_group(x, 64, row_alignment=4)
    torch.cuda.synchronize()
    xf = base[:, :2 * k].float().numpy()
    want_q, want_s = oracle.silu_mul_quant_per_token(xf)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    _assert_codes(q.cpu().numpy(), want_q)
    want_qg, want_sg = oracle.silu_mul_quant_per_token_group(xf, 64)
    assert np.array_equal(sg[:m].contiguous().cpu().numpy().view(np.uint32), want_sg.view(np.uint32))
    _assert_codes(qg.cpu().numpy()[:m], want_qg)


# ---------------------------------------------------------------- UE8M0
UE_CASES = [("block_7168", m, 7168, 128) for m in (1, 5, 64)] + \
           [("ue_groups", m, 1024, g) for g in (16, 32, 64) for m in (3, 40)] + \
           [("block_moe", 4096, 4096, 128)]


@pytest.mark.parametrize("wl,m,k,g", UE_CASES, ids=[f"{c[0]}-M{c[1]}-K{c[2]}-G{c[3]}" for c in UE_CASES])
def test_ue8m0_group_bit_exact(wl, m, k, g):
    x = activations(wl, m, k)
    say("quant_per_token_group ue8m0", wl, m, k, g)
    q, s = ops.quant_per_token_group(gpu(x), g, scale_ue8m0=True)
    qs, ss = ops.silu_mul_quant_per_token_group(gpu(activations(wl + "_silu", m, 2 * k)), g,
                                                scale_ue8m0=True)
    torch.cuda.synchronize()
    want_q, want_s = oracle.quant_per_token_group(x.float().numpy(), g, scale_ue8m0=True)
    assert np.array_equal(s[:m].contiguous().cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    _assert_codes(q.cpu().numpy()[:m], want_q)
    want_qs, want_ss = oracle.silu_mul_quant_per_token_group(
        activations(wl + "_silu", m, 2 * k).float().numpy(), g, scale_ue8m0=True)
    assert np.array_equal(ss[:m].contiguous().cpu().numpy().view(np.uint32), want_ss.view(np.uint32))
    _assert_codes(qs.cpu().numpy()[:m], want_qs)


@pytest.mark.parametrize("m,k", [(1, 4096), (33, 4096), (7, 12288)])
def test_ue8m0_per_token_bit_exact(m, k):
    x = activations("ue_pt", m, k)
    say("quant_per_token ue8m0", m, k)
    q, s = ops.quant_per_token(gpu(x), scale_ue8m0=True)
    torch.cuda.synchronize()
    want_q, want_s = oracle.quant_per_token_group(x.float().numpy(), k, scale_ue8m0=True)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s[:, 0].view(np.uint32))
    _assert_codes(q.cpu().numpy(), want_q)


# ---------------------------------------------------------------- static
STATIC_CASES = [("o_proj", m, 4096, sc) for m in (1, 64, 1024) for sc in (0.03, 0.0071, 1.7)] + \
               [("static_edge", m, k, sc) for m, k, sc in ((3, 48, 2.0 ** -9), (5, 16, 0.01),
                                                            (8192, 4096, 0.02))]


@pytest.mark.parametrize("wl,m,k,sc", STATIC_CASES, ids=[f"{c[0]}-M{c[1]}-K{c[2]}-s{c[3]}" for c in STATIC_CASES])
def test_static_bit_exact(wl, m, k, sc):
    x = activations(wl, m, k, 0.01 if wl == "o_proj" else 0.0)
    xf = x.float().numpy().copy()
    # the division-sensitive value of the worked example, and a saturating one
    xf[0, :3] = [0.000732421875, 500.0, -500.0]
    x = torch.from_numpy(xf).to(torch.bfloat16)
    say("quant_static", wl, m, k, sc)
    scale = torch.tensor([sc], dtype=torch.float32, device=device())
    q = ops.quant_static(gpu(x), scale)
    torch.cuda.synchronize()
    rows = sample_rows(m, count=256)
    want = oracle.quant_static(x[rows].float().numpy(), np.float32(sc))
    _assert_codes(q.cpu().numpy()[rows], want)


# ---------------------------------------------------------------- composed with the GEMMs
@pytest.mark.parametrize("m", [1, 4, 64, 512])
def test_silu_quant_feeds_down_projection(m):
    """The gate/up output of Qwen3-8B (24576 wide) through the fused SiLU-and-mul
    per-token quantizer into the channelwise down projection (N=4096, K=12288),
    and the MoE expert's 3072-wide output through the group-128 form into its
    blockwise down projection (N=4096, K=1536): GEMM outputs within the GEMM
    tolerance of the oracle's composition."""
    from gpu_common import bf16_to_f64, weight_blockwise, weight_channelwise

    x = activations("silu_down", m, 2 * 12288)
    say("silu -> channelwise down", m)
    q, s = ops.silu_mul_quant_per_token(gpu(x))
    bq, bs = weight_channelwise("silu_down_w", 4096, 12288)
    out = ops.scaled_mm_channelwise(q, gpu(bq), s, gpu(bs))
    torch.cuda.synchronize()
    aq, as_ = oracle.silu_mul_quant_per_token(x.float().numpy())
    ref = oracle.scaled_mm_channelwise(aq, bq, as_, bs)
    tau = oracle.gemm_tolerance_channelwise(aq, bq, as_, bs)
    res = oracle.check_gemm(bf16_to_f64(out), ref, tau)
    assert res["ok"] and res["cosine"] > 0.9999, res

    x2 = activations("silu_down_moe", m, 2 * 1536)
    say("silu -> blockwise down", m)
    q2, s2 = ops.silu_mul_quant_per_token_group(gpu(x2), 128)
    wq, ws = weight_blockwise("silu_down_moe_w", 4096, 1536)
    out2 = ops.scaled_mm_blockwise(q2, gpu(wq), s2, gpu(ws), m=m)
    torch.cuda.synchronize()
    aq2, as2 = oracle.silu_mul_quant_per_token_group(x2.float().numpy(), 128)
    ref2 = oracle.scaled_mm_blockwise(aq2, wq, as2, ws)
    tau2 = oracle.gemm_tolerance_blockwise(aq2, wq, as2, ws)
    res2 = oracle.check_gemm(bf16_to_f64(out2), ref2, tau2)
    assert res2["ok"] and res2["cosine"] > 0.9999, res2


def _near_midpoint_pairs(count, seed=7):
    """bf16 (gate, up) pairs whose silu(gate) * up lies within 40 fp32 ulps of
    a bf16 rounding midpoint (the values the fp32 SiLU evaluation must hand to
    its exact fallback), gates over [-16, 20]."""
    rng = np.random.default_rng(seed)
    out_g, out_u = [], []
    while sum(len(a) for a in out_g) < count:
        g = torch.from_numpy(np.concatenate([rng.normal(0, 2, 1 << 20), rng.uniform(-16, 20, 1 << 18)])
                             .astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)
        u = torch.from_numpy(rng.normal(0, 1, g.size).astype(np.float32)).to(torch.bfloat16).float() \
            .numpy().astype(np.float64)
        y = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        low = y.view(np.uint32) & 0xFFFF
        near = (np.abs(low.astype(np.int64) - 0x8000) <= 40) & (y != 0)
        out_g.append(g[near])
        out_u.append(u[near])
    return np.concatenate(out_g)[:count], np.concatenate(out_u)[:count]


def test_silu_near_bf16_midpoints():
    """Each near-midpoint pair is the only nonzero of its 16-element group and
    of its row (the other gates are 0, so their products are 0): the group and
    row scales are then |bf16(silu(g) * u)| / 448 and show any one-ulp error of
    the bf16 product."""
    g, u = _near_midpoint_pairs(4096)
    m, k = g.size, 16
    x = np.zeros((m, 2 * k), dtype=np.float32)
    pos = np.arange(m) % k
    x[np.arange(m), pos] = g
    x[np.arange(m), k + pos] = u
    x[:, k:] += np.where(np.arange(k) == pos[:, None], 0.0, 1.0)  # up halves nonzero, gates zero
    xb = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xb.float().numpy(), x)
    say("silu near midpoints", m)
    q, s = ops.silu_mul_quant_per_token(gpu(xb))
    qg, sg = ops.silu_mul_quant_per_token_group(gpu(xb), 16, row_alignment=1)
    torch.cuda.synchronize()
    want_q, want_s = oracle.silu_mul_quant_per_token(x)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    _assert_codes(q.cpu().numpy(), want_q)
    want_qg, want_sg = oracle.silu_mul_quant_per_token_group(x, 16)
    assert np.array_equal(sg.contiguous().cpu().numpy().view(np.uint32), want_sg.view(np.uint32))
    _assert_codes(qg.cpu().numpy(), want_qg)
