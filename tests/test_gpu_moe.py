"""GPU parity of the MoE expert path against the oracle: the masked per-expert
group quantizer (codes and scales bit-exact on valid rows, every other row
untouched) and the grouped blockwise GEMM over E experts with per-expert
valid row counts in device memory (within the GEMM tolerance on valid rows,
other rows untouched), on the blockwise workload's expert shapes (gate/up
3072x4096, down 4096x1536, group 128)."""
import functools

import numpy as np
import pytest
import torch

import oracle
from fp8_w8a8_quantized_token_amd import ops, synth
from gpu_common import bf16_to_f64, device, gpu, say

pytestmark = pytest.mark.gpu


def _counts(e_n, m_max, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, m_max + 1, size=e_n)
    c[0] = m_max
    if e_n > 2:
        c[1] = 0
    return c.astype(np.int32)


def _batch(key, e_n, m_max, k):
    return torch.stack([synth.activations(f"{key}/{e}", m_max, k) for e in range(e_n)])


@functools.lru_cache(maxsize=4)
def _weights(key, e_n, n, k, ue8m0):
    ws = [oracle.quant_weight_blockwise(synth.weights(f"{key}/{e}", n, k).numpy(), scale_ue8m0=ue8m0)
          for e in range(e_n)]
    return np.stack([w[0] for w in ws]), np.stack([w[1] for w in ws])


QUANT_CASES = [(8, 4, 1536, 128, False, False), (8, 64, 4096, 128, False, False),
               (4, 37, 1024, 64, False, False), (8, 16, 1536, 128, True, False),
               (8, 64, 1536, 128, False, True), (3, 9, 512, 16, True, True)]


@pytest.mark.parametrize("e_n,m_max,k,g,silu,ue8m0", QUANT_CASES,
                         ids=[f"E{c[0]}-M{c[1]}-K{c[2]}-G{c[3]}{'-silu' if c[4] else ''}{'-ue8m0' if c[5] else ''}"
                              for c in QUANT_CASES])
def test_masked_quant_bit_exact(e_n, m_max, k, g, silu, ue8m0):
    width = 2 * k if silu else k
    x = _batch("moe-q", e_n, m_max, width)
    counts = _counts(e_n, m_max, m_max + k)
    say("masked quant", e_n, m_max, k, g, silu, ue8m0, counts.tolist())
    m_pad = ops.padded_rows(m_max, 4)
    q_buf = torch.full((e_n, m_pad, k), 0x7F, dtype=torch.uint8, device=device())
    s_buf = torch.full((e_n, k // g, m_pad), float("nan"), dtype=torch.float32, device=device())
    q, s = ops.masked_quant_per_token_group(gpu(x), gpu(counts), g, out=q_buf, scale_storage=s_buf,
                                            silu_mul=silu, scale_ue8m0=ue8m0)
    torch.cuda.synchronize()
    xf = x.float().numpy()
    if silu:
        want_q, want_s = oracle.masked_quant_per_token_group(
            np.stack([oracle.silu_mul_bf16(xf[e]) for e in range(e_n)]), counts, g, scale_ue8m0=ue8m0)
    else:
        want_q, want_s = oracle.masked_quant_per_token_group(xf, counts, g, scale_ue8m0=ue8m0)
    got_q = q.cpu().numpy()
    got_s = s.cpu().numpy()  # [E, M_pad, K/G] view
    for e in range(e_n):
        r = counts[e]
        assert np.array_equal(got_q[e, :r], want_q[e, :r]), e
        assert np.array_equal(got_s[e, :r].view(np.uint32), want_s[e, :r].view(np.uint32)), e
        assert np.all(got_q[e, r:] == 0x7F), f"expert {e}: rows past masked_m were written"
        assert np.all(np.isnan(got_s[e, r:])), f"expert {e}: scales past masked_m were written"


GEMM_CASES = [  # (E, M_max, N, K, variant, ue8m0)
    (8, 4, 3072, 4096, None, False), (8, 64, 3072, 4096, None, False), (8, 64, 4096, 1536, None, False),
    (4, 256, 4096, 1536, None, False), (4, 512, 3072, 4096, None, False),
    (8, 16, 4096, 1536, "t32x32deep", False), (8, 100, 3072, 4096, "t64x32deep", False),
    (6, 300, 384, 1024, "t256x256bw16", False), (6, 300, 384, 1024, "t256x256bw16", True),
    (4, 200, 1024, 2048, "t128x128panel", False), (4, 200, 1024, 2048, "t256x128panel", True),
    (2, 4096, 3072, 4096, None, True),
    # the 7168x7168 blockwise table names split-K tiles at these M: the grouped
    # path drops the split under the default config
    (3, 16, 7168, 7168, None, False), (2, 64, 7168, 7168, None, True)]


@pytest.mark.parametrize("e_n,m_max,n,k,variant,ue8m0", GEMM_CASES,
                         ids=[f"E{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}-{c[4] or 'default'}{'-ue8m0' if c[5] else ''}"
                              for c in GEMM_CASES])
def test_grouped_gemm(e_n, m_max, n, k, variant, ue8m0):
    counts = _counts(e_n, m_max, m_max * 7 + n)
    x = _batch("moe-mm", e_n, m_max, k)
    a, sa = oracle.masked_quant_per_token_group(x.float().numpy(), counts, 128, scale_ue8m0=ue8m0)
    b, sb = _weights("moe-w", e_n, n, k, ue8m0)
    m_pad = ops.padded_rows(m_max, 4)
    a_dev = torch.full((e_n, m_pad, k), 0x7F, dtype=torch.uint8, device=device())
    s_store = torch.full((e_n, k // 128, m_pad), float("nan"), dtype=torch.float32, device=device())
    for e in range(e_n):
        r = counts[e]
        a_dev[e, :r] = gpu(a[e, :r])
        s_store[e, :, :r] = gpu(sa[e, :r].T.copy())
    out = torch.full((e_n, m_max, n), float("nan"), dtype=torch.bfloat16, device=device())
    cfg = ops.make_config(variant) if variant else None
    say("grouped gemm", e_n, m_max, n, k, variant, ue8m0, counts.tolist())
    ops.scaled_mm_blockwise_masked(a_dev, gpu(b), s_store.transpose(1, 2), gpu(sb), gpu(counts),
                                   m_max=m_max, out=out, config=cfg, scale_ue8m0=ue8m0)
    torch.cuda.synchronize()
    got = bf16_to_f64(out.reshape(e_n * m_max, n)).reshape(e_n, m_max, n)
    for e in range(e_n):
        r = int(counts[e])
        assert np.all(np.isnan(got[e, r:])), f"expert {e}: rows past masked_m were written"
        if r == 0:
            continue
        rows = np.arange(r) if r * n <= 2_000_000 else np.unique(np.r_[0, r - 1, np.linspace(0, r - 1, 24).astype(int)])
        ref = oracle.scaled_mm_blockwise(a[e, rows], b[e], sa[e, rows], sb[e])
        tau = oracle.gemm_tolerance_blockwise(a[e, rows], b[e], sa[e, rows], sb[e])
        res = oracle.check_gemm(got[e, rows], ref, tau)
        assert res["ok"], (e, res)
        assert res["cosine"] > 0.9999, (e, res)


def test_out_of_range_counts_are_clamped():
    """masked_m lives in device memory, so the host cannot check it: the
    kernels clamp every count into [0, M_max]. Negative counts act as 0, counts
    past M_max as M_max, and nothing outside the expert slabs is written (the
    buffers carry a guard expert on each side)."""
    e_n, m_max, n, k = 4, 24, 256, 512
    raw = np.array([-3, 30, 7, m_max + 1000], dtype=np.int32)
    clamped = np.clip(raw, 0, m_max)
    x = _batch("moe-clamp", e_n, m_max, k)
    say("clamped counts", raw.tolist())
    m_pad = ops.padded_rows(m_max, 4)
    # experts 1..e_n of e_n + 2 slabs; slabs 0 and e_n + 1 are guards
    q_all = torch.full((e_n + 2, m_pad, k), 0x7F, dtype=torch.uint8, device=device())
    s_all = torch.full((e_n + 2, k // 128, m_pad), float("nan"), dtype=torch.float32, device=device())
    q, s = ops.masked_quant_per_token_group(gpu(x), gpu(raw), 128, out=q_all[1:e_n + 1],
                                            scale_storage=s_all[1:e_n + 1])
    torch.cuda.synchronize()
    want_q, want_s = oracle.masked_quant_per_token_group(x.float().numpy(), clamped, 128)
    got_q, got_s = q.cpu().numpy(), s.cpu().numpy()
    for e in range(e_n):
        r = clamped[e]
        assert np.array_equal(got_q[e, :r], want_q[e, :r])
        assert np.array_equal(got_s[e, :r].view(np.uint32), want_s[e, :r].view(np.uint32))
        assert np.all(got_q[e, r:] == 0x7F) and np.all(np.isnan(got_s[e, r:]))
    for guard in (0, e_n + 1):
        assert np.all(q_all[guard].cpu().numpy() == 0x7F)
        assert np.all(np.isnan(s_all[guard].cpu().numpy()))

    b, sb = _weights("moe-clamp-w", e_n, n, k, False)
    out_all = torch.full((e_n + 2, m_max, n), float("nan"), dtype=torch.bfloat16, device=device())
    ops.scaled_mm_blockwise_masked(q, gpu(b), s, gpu(sb), gpu(raw), m_max=m_max,
                                   out=out_all[1:e_n + 1])
    torch.cuda.synchronize()
    got = bf16_to_f64(out_all.reshape(-1, n)).reshape(e_n + 2, m_max, n)
    assert np.all(np.isnan(got[0])) and np.all(np.isnan(got[e_n + 1]))
    for e in range(e_n):
        r = int(clamped[e])
        assert np.all(np.isnan(got[e + 1, r:]))
        if r:
            ref = oracle.scaled_mm_blockwise(want_q[e, :r], b[e], want_s[e, :r], sb[e])
            tau = oracle.gemm_tolerance_blockwise(want_q[e, :r], b[e], want_s[e, :r], sb[e])
            assert oracle.check_gemm(got[e + 1, :r], ref, tau)["ok"]
