"""Per-shape measurement of the FP8 linear on one MI355X (gfx950).

For every (kind, N, K, M) of the workloads in ``synth.WORKLOADS`` this times,
call by call with HIP events on the launch stream (warm-up calls first, then
the timed ones):

* ``gemm``   -- the scaled GEMM alone (the metric),
* ``quant``  -- the activation quantizer alone (per token for channelwise,
  group 128 with row alignment 4 for blockwise),
* ``linear`` -- the whole linear through ``fp8_linear_*`` (quantizer then GEMM,
  or the single fused launch where M is small),

cycling through enough distinct buffer sets (activations, codes, scales,
weights) that at least 1 GiB of weights is touched, four times the 256 MB
last-level cache, so every call's weight comes from HBM; and ``hot``, the
same GEMM repeated on one buffer set. Reported per row: medians with p10 and
p90 over the timed calls, TFLOP/s, algorithmic GB/s (the bytes the method
must move: codes, weight, scales, bias, output; no padding rows or re-reads)
and the fractions of HBM (8 TB/s) and dense FP8 MFMA (5.0 PFLOP/s) peak.

Inputs are the seeded synthetic tensors of ``synth`` (no dataset); weights
are quantized by the library itself, blockwise weight scales are synthetic
(timing does not depend on their values).

Usage: python -m fp8_w8a8_quantized_token_amd.measure [--workloads small,o_proj,...]
       [--calls 100] [--warmup 20] [--out FILE]
"""
import argparse
import json
import os
import math
import sys
import time

import torch

from . import _lib, ops, synth

PEAK_GBPS = 8000.0
PEAK_TFLOPS = 5000.0
ROTATE_BYTES = 1 << 30
MAX_SETS = 64


def gemm_bytes(kind, m, n, k, bias):
    b = m * k + n * k + 2 * m * n + (2 * n if bias else 0)
    if kind == "channelwise":
        return b + 4 * m + 4 * n
    return b + 4 * m * (k // 128) + 4 * (n // 128) * (k // 128)


def quant_bytes(kind, m, k):
    return 3 * m * k + 4 * m * (1 if kind == "channelwise" else k // 128)


def percentile(xs, p):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))
    return xs[i]


class _Filler:
    """Device copies queued ahead of the timed calls, so the host has enqueued
    every call before the GPU reaches the first one: the events then time the
    kernels, not the host's launch rate."""

    def __init__(self, dev):
        self.a = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
        self.b = torch.empty_like(self.a)

    def __call__(self, calls):
        for _ in range(max(4, calls // 3)):  # ~90 us per 256 MiB copy
            self.b.copy_(self.a)


def time_calls(fns, warmup, calls, filler):
    """Per-call durations (us) of fns cycled round-robin: events around each call."""
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    filler(calls)
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        fns[i % len(fns)]()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]


class ShapeBuffers:
    """Weight copies of one (kind, N, K), enough of them to cover >= 1 GiB."""

    def __init__(self, cfg, kind, n, k, with_bias, dev):
        self.kind, self.n, self.k, self.dev = kind, n, k, dev
        self.sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / (n * k))))
        w = synth.weights(f"measure/{cfg}", n, k).to(torch.bfloat16).to(dev)
        if kind == "channelwise":
            wq, ws = ops.quant_per_token(w)
        else:
            wq, _ = ops.quant_per_token_group(w, 128, row_alignment=1)
            wq = wq.contiguous()
            ws = synth.positive_scales(f"measure/{cfg}/{n}/{k}", (n // 128, k // 128)).to(dev)
        del w
        self.w = [(wq.clone(), ws.clone()) for _ in range(self.sets)]
        self.bias = synth.bias(f"measure/{cfg}", n).to(dev) if with_bias else None


def measure_m(buf, cfg, m, outliers, warmup, calls, filler):
    kind, n, k, dev, sets = buf.kind, buf.n, buf.k, buf.dev, buf.sets
    x0 = synth.activations(f"measure/{cfg}", m, k, outlier_frac=outliers).to(dev)
    m_pad = ops.padded_rows(m, 4) if kind == "blockwise" else m
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    xs, qs, ss = [], [], []
    for _ in range(sets):
        xs.append(x0.clone())
        qs.append(torch.empty((m_pad, k), dtype=torch.uint8, device=dev))
        ss.append(torch.empty((m,), dtype=torch.float32, device=dev) if kind == "channelwise"
                  else torch.empty((k // 128, m_pad), dtype=torch.float32, device=dev))
    quant, gemm, linear = [], [], []
    for i in range(sets):
        wq, ws = buf.w[i]
        if kind == "channelwise":
            quant.append(ops.prepare("quant_per_token", xs[i], out=qs[i], scale=ss[i]))
            quant[-1]()
            gemm.append(ops.prepare("scaled_mm_channelwise", qs[i], wq, ss[i], ws, bias=buf.bias,
                                    out=out))
            linear.append(ops.prepare("linear_channelwise", xs[i], wq, ws, bias=buf.bias, out=out,
                                      q=qs[i], scale=ss[i]))
        else:
            quant.append(ops.prepare("quant_per_token_group", xs[i], 128, row_alignment=4,
                                     out=qs[i], scale_storage=ss[i]))
            quant[-1]()
            gemm.append(ops.prepare("scaled_mm_blockwise", qs[i], wq, ss[i].transpose(0, 1), ws,
                                    bias=buf.bias, m=m, out=out))
            linear.append(ops.prepare("linear_blockwise", xs[i], wq, ws, bias=buf.bias,
                                      row_alignment=4, out=out, q=qs[i], scale=ss[i]))
    torch.cuda.synchronize()
    kid = ops.KIND_CHANNELWISE if kind == "channelwise" else ops.KIND_BLOCKWISE
    cfg_d, hit = ops.tile_config(kid, n, k, m)
    res = {
        "gemm": time_calls(gemm, warmup, calls, filler),
        "quant": time_calls(quant, warmup, calls, filler),
        "linear": time_calls(linear, warmup, calls, filler),
        "hot": time_calls(gemm[:1], warmup, calls, filler),
        "rot_gib": min(sets, calls) * n * k / (1 << 30),
        "variant": cfg_d["variant"], "split_k": cfg_d["split_k"], "table": hit,
        "launches": ops.linear_launches(kid, m, n, k),
    }
    return res


# Quantizer variants: (name, K, M values). SiLU-and-mul inputs are [M, 2K]
# (the gate/up projection's output), the quantized rows K wide.
QUANT_VARIANTS = [
    ("silu_per_token", 12288, (1, 64, 512, 8192)),     # Qwen3-8B 24576 -> down K = 12288
    ("per_token", 12288, (1, 64, 512, 8192)),          # the same rows without SiLU-and-mul
    ("silu_group128", 12288, (1, 64, 512, 8192)),
    ("silu_group128", 1536, (1, 4, 16, 64, 4096)),     # MoE expert 3072 -> down K = 1536
    ("group128", 1536, (1, 4, 16, 64, 4096)),
    ("ue8m0_group128", 7168, (1, 64, 256)),
    ("ue8m0_group128", 4096, (4096,)),
    ("static", 4096, (1, 64, 1024, 8192)),
]


def quant_variant_bytes(name, m, k):
    """Algorithmic bytes: bf16 input (2K wide with SiLU-and-mul), codes, scales."""
    read = (4 if name.startswith("silu") else 2) * m * k
    if name == "static":
        return read + m * k + 4
    scales = 4 * m * (k // 128) if "group128" in name else 4 * m
    return read + m * k + scales


def _quant_variant_call(name, x, q, s, scale):
    if name == "silu_per_token":
        return ops.prepare("silu_mul_quant_per_token", x, out=q, scale=s)
    if name == "per_token":
        return ops.prepare("quant_per_token", x, out=q, scale=s)
    if name == "static":
        return ops.prepare("quant_static", x, scale, out=q)
    kw = dict(row_alignment=4, out=q, scale_storage=s)
    if name == "silu_group128":
        return ops.prepare("silu_mul_quant_per_token_group", x, 128, **kw)
    if name == "ue8m0_group128":
        return ops.prepare("quant_per_token_group", x, 128, scale_ue8m0=True, **kw)
    return ops.prepare("quant_per_token_group", x, 128, **kw)


def measure_quant_variants(warmup, calls, filler):
    """Average launch time of each quantizer variant over `calls` back-to-back
    launches cycling through buffer sets that cover >= 1 GiB of input where
    the shape allows (at most MAX_SETS sets), timed as one batch with HIP
    events: per-call event pairs would add their own ~4 us."""
    dev = torch.device("cuda:0")
    head = ("| variant | K | M | input MB | sets | µs per launch | GB/s | frac HBM |")
    lines = [head, "|---|---|---|---|---|---|---|---|"]
    print(head, flush=True)
    print(lines[1], flush=True)
    scale = torch.tensor([0.02], dtype=torch.float32, device=dev)
    for name, k, ms in QUANT_VARIANTS:
        width = 2 * k if name.startswith("silu") else k
        for m in ms:
            x0 = synth.activations(f"measure/quant/{name}", m, width).to(dev)
            sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / x0.numel() / 2)))
            m_pad = ops.padded_rows(m, 4)
            fns, keep = [], []
            for _ in range(sets):
                x = x0.clone()
                q = torch.empty((m_pad, k), dtype=torch.uint8, device=dev)
                s = torch.empty((k // 128, m_pad) if "group" in name else (m,), dtype=torch.float32,
                                device=dev)
                keep.append((x, q, s))
                fns.append(_quant_variant_call(name, x, q, s, scale))
            for i in range(warmup):
                fns[i % sets]()
            torch.cuda.synchronize()
            filler(calls)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(calls):
                fns[i % sets]()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / calls
            gb = quant_variant_bytes(name, m, k) / us / 1e3
            line = (f"| {name} | {k} | {m} | {x0.numel() * 2 / 1e6:.2f} | {sets} | {us:.2f} | "
                    f"{gb:.0f} | {gb / PEAK_GBPS:.2f} |")
            lines.append(line)
            print(line, flush=True)
            del keep, fns, x0
            torch.cuda.empty_cache()
    return lines


# Blockwise GEMMs timed with fp32 scales (promotion per 128-deep block) and
# with power-of-two scales (block-scaled MFMA), on the 16x16 256x256 tile.
UE8M0_SHAPES = [(4096, 4096, (2048, 4096, 8192)), (3072, 4096, (4096,)), (4096, 1536, (4096,)),
                (7168, 7168, (4096,))]


def measure_ue8m0_gemm(warmup, calls, filler):
    dev = torch.device("cuda:0")
    head = "| N×K | M | tile | scales | weight sets | µs per launch | TFLOP/s | frac MFMA |"
    lines = [head, "|---|---|---|---|---|---|---|---|"]
    print(head, flush=True)
    print(lines[1], flush=True)
    cfg = ops.make_config("t256x256bw16")
    for n, k, ms in UE8M0_SHAPES:
        sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / (n * k))))
        w = synth.weights("measure/ue8m0", n, k).to(torch.bfloat16).to(dev)
        wq, _ = ops.quant_per_token_group(w, 128, row_alignment=1)
        wq = wq.contiguous()
        del w
        ws = synth.positive_scales(f"measure/ue8m0/{n}/{k}", (n // 128, k // 128)).to(dev)
        ws_e8 = torch.exp2(torch.ceil(torch.log2(ws)))  # powers of two
        weights = [wq.clone() for _ in range(sets)]
        for m in ms:
            x = synth.activations("measure/ue8m0", m, k).to(dev)
            out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            for ue8m0 in (False, True):
                q, st = ops.quant_per_token_group(x, 128, row_alignment=4, scale_ue8m0=ue8m0)
                bs = ws_e8 if ue8m0 else ws
                fns = [ops.prepare("scaled_mm_blockwise", q, wt, st, bs, m=m, out=out, config=cfg,
                                   scale_ue8m0=ue8m0) for wt in weights]
                for i in range(warmup):
                    fns[i % sets]()
                torch.cuda.synchronize()
                filler(calls)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(calls):
                    fns[i % sets]()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / calls
                tf = 2 * m * n * k / us / 1e6
                line = (f"| {n}×{k} | {m} | t256x256bw16 | {'ue8m0 (MFMA-scaled)' if ue8m0 else 'fp32 (promotion)'} "
                        f"| {sets} | {us:.1f} | {tf:.0f} | {tf / PEAK_TFLOPS:.3f} |")
                lines.append(line)
                print(line, flush=True)
        del weights
        torch.cuda.empty_cache()
    return lines


# MoE experts (the blockwise workload's expert shapes): E experts of M_max
# rows each, every expert full or a seeded random count in [0, M_max].
MOE_SHAPES = [(3072, 4096), (4096, 1536)]
MOE_MAX = (4, 16, 64, 256, 512)
MOE_E = 8


def measure_moe(warmup, calls, filler):
    """Grouped blockwise GEMM (and the masked quantizer feeding it) over
    MOE_E experts, weight sets rotated to cover >= 1 GiB, batch-timed."""
    dev = torch.device("cuda:0")
    head = ("| N×K | E | M_max | rows (valid) | GEMM µs | TFLOP/s (valid rows) | weight GB/s | "
            "masked quant µs |")
    lines = [head, "|---|---|---|---|---|---|---|---|"]
    print(head, flush=True)
    print(lines[1], flush=True)
    gen = torch.Generator().manual_seed(5)
    for n, k in MOE_SHAPES:
        wbytes = MOE_E * n * k
        sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / wbytes)))
        w = synth.weights("measure/moe", n, k).to(torch.bfloat16).to(dev)
        wq, _ = ops.quant_per_token_group(w, 128, row_alignment=1)
        wq = wq.contiguous()
        del w
        ws = synth.positive_scales(f"measure/moe/{n}/{k}", (n // 128, k // 128)).to(dev)
        weights = [(wq.unsqueeze(0).repeat(MOE_E, 1, 1), ws.unsqueeze(0).repeat(MOE_E, 1, 1).contiguous())
                   for _ in range(sets)]
        for m_max in MOE_MAX:
            for full in (True, False):
                counts = torch.full((MOE_E,), m_max, dtype=torch.int32) if full else \
                    torch.randint(0, m_max + 1, (MOE_E,), generator=gen, dtype=torch.int32)
                valid = int(counts.sum())
                cd = counts.to(dev)
                x = torch.stack([synth.activations(f"measure/moe/{e}", m_max, k) for e in range(MOE_E)]).to(dev)
                q, st = ops.masked_quant_per_token_group(x, cd, 128)
                out = torch.empty((MOE_E, m_max, n), dtype=torch.bfloat16, device=dev)
                fns = [lambda wt=wt, sc=sc: ops.scaled_mm_blockwise_masked(q, wt, st, sc, cd, m_max=m_max,
                                                                          out=out)
                       for wt, sc in weights]
                tq = []
                for fn_set, dst in ((fns, None), ([lambda: ops.masked_quant_per_token_group(x, cd, 128, out=q,
                                                  scale_storage=st.transpose(1, 2))], tq)):
                    for i in range(warmup):
                        fn_set[i % len(fn_set)]()
                    torch.cuda.synchronize()
                    filler(calls)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for i in range(calls):
                        fn_set[i % len(fn_set)]()
                    e1.record()
                    torch.cuda.synchronize()
                    t = e0.elapsed_time(e1) * 1e3 / calls
                    if dst is None:
                        us = t
                    else:
                        dst.append(t)
                line = (f"| {n}×{k} | {MOE_E} | {m_max} | {valid} ({'full' if full else 'random'}) | "
                        f"{us:.1f} | {2 * valid * n * k / us / 1e6:.0f} | "
                        f"{wbytes / us / 1e3:.0f} | {tq[0]:.1f} |")
                lines.append(line)
                print(line, flush=True)
        del weights
        torch.cuda.empty_cache()
    return lines


HEADER = ("| workload | kind | N×K | M | tile config | weight GiB rotated | GEMM µs p50 (p10–p90) | "
          "TFLOP/s | GB/s | frac HBM | frac MFMA | quant µs p50 (GB/s) | linear µs p50 (launches) | "
          "hot GEMM µs p50 |")


def _batch_us(fns, warmup, calls, filler):
    """Average µs per call of `calls` back-to-back calls cycling through fns,
    timed as one batch with HIP events behind queued device copies."""
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    filler(calls)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(calls):
        fns[i % len(fns)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / calls


def measure_stream_ceiling(warmup, calls, filler):
    """What plain HBM streams reach at the byte counts the small-M linears
    move, beside the skinny GEMM itself: torch's device copy (reads and writes
    the size) and max-reduction (reads it once) from 8.4 MB to 268 MB, and the
    o_proj channelwise GEMM (N = K = 4096, a 16.8 MB weight) at M = 1 and 16,
    each over distinct buffers covering >= 1 GiB so every call starts from
    HBM."""
    dev = torch.device("cuda:0")
    head = "| op | MB moved per call | buffers | µs per call | GB/s | frac of 8 TB/s |"
    lines = [head, "|---|---|---|---|---|---|"]
    print(head, flush=True)
    print(lines[1], flush=True)

    def emit(name, nbytes, sets, us):
        line = (f"| {name} | {nbytes / 1e6:.1f} | {sets} | {us:.2f} | {nbytes / us / 1e3:.0f} | "
                f"{nbytes / us / 1e3 / PEAK_GBPS:.2f} |")
        lines.append(line)
        print(line, flush=True)

    n = k = 4096
    sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / (n * k))))
    w = synth.weights("measure/stream", n, k).to(torch.bfloat16).to(dev)
    wq, ws = ops.quant_per_token(w)
    del w
    weights = [(wq.clone(), ws.clone()) for _ in range(sets)]
    for m in (1, 16):
        a, sa = ops.quant_per_token(synth.activations("measure/stream", m, k).to(dev))
        outs = [torch.empty((m, n), dtype=torch.bfloat16, device=dev) for _ in range(sets)]
        fns = [ops.prepare("scaled_mm_channelwise", a, wb, sa, wsb, out=o)
               for (wb, wsb), o in zip(weights, outs)]
        emit(f"channelwise GEMM M={m} N=K=4096", gemm_bytes("channelwise", m, n, k, False),
             sets, _batch_us(fns, warmup, calls, filler))
        del fns, outs
    del weights
    torch.cuda.empty_cache()
    for size in (2048 * 4096, 4096 * 4096, 2 * 4096 * 4096, 4 * 4096 * 4096, 8 * 4096 * 4096,
                 16 * 4096 * 4096):
        sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / size)))
        src = [torch.full((size // 4,), i, dtype=torch.int32, device=dev) for i in range(sets)]
        dst = [torch.empty_like(t) for t in src]
        red = torch.empty((), dtype=torch.int32, device=dev)
        emit(f"copy {size / 1e6:.1f} MB", 2 * size, sets,
             _batch_us([lambda i=i: dst[i].copy_(src[i]) for i in range(sets)], warmup, calls, filler))
        emit(f"max-reduce {size / 1e6:.1f} MB", size, sets,
             _batch_us([lambda i=i: torch.amax(src[i], dim=0, out=red) for i in range(sets)],
                       warmup, calls, filler))
        del src, dst
        torch.cuda.empty_cache()
    return lines


def measure_library_reference(warmup, calls, filler):
    """Context for the large-M tiles: the same channelwise GEMMs through the
    vendor library (torch._scaled_mm, hipBLASLt on ROCm) beside this library's
    default tile, on the same E4M3 operands with row-wise fp32 scales and with
    unit tensor-wise scales, weights rotated over >= 1 GiB of copies. Not part
    of the path; a measurement of the practical ceiling on this chip."""
    dev = torch.device("cuda:0")
    head = ("| N×K | M | this library µs (TFLOP/s) | library, row-wise scales µs (TFLOP/s) | "
            "library, tensor-wise scales µs (TFLOP/s) |")
    lines = [head, "|---|---|---|---|---|"]
    print(head, flush=True)
    print(lines[1], flush=True)
    for n, k, m in ((4096, 4096, 4096), (4096, 4096, 8192), (6144, 4096, 8192), (4096, 12288, 8192),
                    (24576, 4096, 8192), (3072, 4096, 4096)):
        sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / (n * k))))
        w = synth.weights("measure/libref", n, k).to(torch.bfloat16).to(dev)
        wq, ws = ops.quant_per_token(w)
        del w
        a, sa = ops.quant_per_token(synth.activations("measure/libref", m, k).to(dev))
        ws_row = ws.reshape(1, n)
        sa_col = sa.reshape(m, 1)
        one = torch.ones((), dtype=torch.float32, device=dev)
        wts = [wq.clone() for _ in range(sets)]
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        fl = 2.0 * m * n * k
        ours = _batch_us([ops.prepare("scaled_mm_channelwise", a, wb, sa, ws, out=out) for wb in wts],
                         warmup, calls, filler)
        a8 = a.view(torch.float8_e4m3fn)
        cells = []
        for sc_a, sc_b in ((sa_col, ws_row), (one, one)):
            try:
                fns = [lambda wb=wb: torch._scaled_mm(a8, wb.view(torch.float8_e4m3fn).t(), scale_a=sc_a,
                                                      scale_b=sc_b, out_dtype=torch.bfloat16) for wb in wts]
                us = _batch_us(fns, warmup, calls, filler)
                cells.append(f"{us:.1f} ({fl / us / 1e6:.0f})")
            except Exception as ex:  # noqa: BLE001 - the library may lack a scaling mode
                cells.append(f"unavailable ({type(ex).__name__})")
        line = f"| {n}×{k} | {m} | {ours:.1f} ({fl / ours / 1e6:.0f}) | {cells[0]} | {cells[1]} |"
        lines.append(line)
        print(line, flush=True)
        del wts, out
        torch.cuda.empty_cache()
    return lines


def measure_probes(warmup, calls, filler):
    """Ceilings from the library's own probe kernels (batch-timed, HIP events
    around each batch): the read-only HBM stream at the small-M weight sizes
    (cold: distinct buffers covering >= 1 GiB, at two grid sizes), the
    L2-to-compute-unit feed with register and LDS-DMA loads (one and two
    workgroups per compute unit, a 512 KB window every workgroup re-reads),
    and the dense FP8 MFMA rate with the clock it implies."""
    import ctypes
    dev = torch.device("cuda:0")
    lib = _lib.load()
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # noqa: E731
    sink = torch.zeros(4096 * 256, dtype=torch.int32, device=dev)
    sp = ctypes.c_void_p(sink.data_ptr())
    head = "| probe | size | grid | µs per call | rate | note |"
    lines = [head, "|---|---|---|---|---|---|"]
    print(head, flush=True)
    print(lines[1], flush=True)

    def emit(*cells):
        line = "| " + " | ".join(str(c) for c in cells) + " |"
        lines.append(line)
        print(line, flush=True)

    # read-only HBM stream at the weight sizes of the small-M linears (and above)
    for size in (6291456, 16777216, 50331648, 100663296, 268435456):
        sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / size)))
        bufs = [torch.full((size // 4,), i, dtype=torch.int32, device=dev) for i in range(sets)]
        for wgs in (1024, 2048):
            fns = [lambda b=b, w=wgs: _lib.check(lib.fp8_probe_stream_read(
                ctypes.c_void_p(b.data_ptr()), size, sp, w, stream())) for b in bufs]
            us = _batch_us(fns, warmup, calls, filler)
            emit("HBM read (cold)", f"{size / 1e6:.1f} MB", f"{wgs}x256", f"{us:.2f}",
                 f"{size / us / 1e3:.0f} GB/s ({size / us / 1e3 / PEAK_GBPS:.2f} of 8 TB/s)", f"{sets} buffers")
        del bufs
        torch.cuda.empty_cache()
    # the same bytes read as row pieces: the weight-panel access of the GEMM tiles
    for rows, rb in ((4096, 4096), (4096, 12288)):
        size = rows * rb
        sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / size)))
        bufs = [torch.full((size // 4,), i, dtype=torch.int32, device=dev) for i in range(sets)]
        for rpw in (16, 32):
            for piece in (64, 128, 256, 512, 1024):
                if (rpw * piece) % 1024:
                    continue
                fns = [lambda b=b, r=rpw, pc=piece: _lib.check(lib.fp8_probe_strided_read(
                    ctypes.c_void_p(b.data_ptr()), rows, rb, r, pc, sp, stream())) for b in bufs]
                us = _batch_us(fns, warmup, calls, filler)
                emit("HBM read in row pieces (cold)", f"{rows}x{rb} B, {piece} B pieces",
                     f"{rows // rpw}x256 ({rpw} rows each)", f"{us:.2f}",
                     f"{size / us / 1e3:.0f} GB/s ({size / us / 1e3 / PEAK_GBPS:.2f} of 8 TB/s)", f"{sets} buffers")
        del bufs
        torch.cuda.empty_cache()
    # read rate against waves per compute unit and pieces in flight per wave
    size = 50331648
    sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / size)))
    bufs = [torch.full((size // 4,), i, dtype=torch.int32, device=dev) for i in range(sets)]
    for dma in (0, 1):
        for threads, depth in ((256, 4), (256, 8), (256, 16), (512, 4), (512, 8), (512, 16), (1024, 4), (1024, 8)):
            for wgs in (256, 512):
                fns = [lambda b=b, t=threads, d=depth, w=wgs, dm=dma: _lib.check(lib.fp8_probe_wave_read(
                    ctypes.c_void_p(b.data_ptr()), size, t, d, dm, sp, w, stream())) for b in bufs]
                us = _batch_us(fns, warmup, calls, filler)
                waves_cu = wgs * threads // 64 // 256
                emit("HBM read by waves (cold)", f"{size / 1e6:.1f} MB", f"{wgs}x{threads}", f"{us:.2f}",
                     f"{size / us / 1e3:.0f} GB/s ({size / us / 1e3 / PEAK_GBPS:.2f})",
                     f"{'LDS-DMA' if dma else 'register'}; {waves_cu} waves/CU x {depth} KB in flight "
                     f"= {waves_cu * depth} KB/CU")
    del bufs
    torch.cuda.empty_cache()
    # L2 -> compute unit feed: every workgroup re-reads a 512 KB window
    win = 512 << 10
    src = torch.full((win // 4,), 3, dtype=torch.int32, device=dev)
    for dma in (0, 1):
        for wgs in (256, 512):
            reps = 64
            fn = lambda w=wgs, d=dma: _lib.check(lib.fp8_probe_l2_feed(  # noqa: E731
                ctypes.c_void_p(src.data_ptr()), win, reps, d, sp, w, stream()))
            us = _batch_us([fn], max(2, warmup // 4), max(4, calls // 10), filler)
            moved = wgs * reps * win
            emit("L2 feed, " + ("LDS-DMA" if dma else "register") + " loads", "512 KB window",
                 f"{wgs}x256", f"{us:.1f}", f"{moved / us / 1e3:.0f} GB/s total, "
                 f"{moved / us / 1e3 / 256:.1f} GB/s per CU", f"{reps} passes per workgroup")
    # the panel tiles' feed pattern: 64-row panels of 4 KB rows, alone, with
    # LDS reads of the landed stages, with a barrier per stage, with both
    row_bytes, panels, stages = 4096, 32, 2048
    pbuf = torch.full((panels * 64 * row_bytes // 4,), 5, dtype=torch.int32, device=dev)
    for mode, what in ((0, "LDS-DMA alone"), (1, "+ LDS reads"), (2, "+ barrier per stage"),
                       (3, "+ LDS reads + barrier")):
        fn = lambda md=mode: _lib.check(lib.fp8_probe_panel_feed(  # noqa: E731
            ctypes.c_void_p(pbuf.data_ptr()), row_bytes, panels, stages, md, sp, 256, stream()))
        us = _batch_us([fn], 2, 5, filler)
        moved = 256 * stages * 8192
        emit("L2 feed, 64-row panels", "8 MB, 4 KB rows", "256x256", f"{us:.1f}",
             f"{moved / us / 1e3 / 256:.1f} GB/s per CU", what)
    del pbuf
    # LDS read rate per compute unit
    for threads, wgs in ((256, 256), (512, 256), (256, 512), (256, 1024)):
        iters = 4000
        fn = lambda t=threads, w=wgs: _lib.check(lib.fp8_probe_lds(iters, t, sp, w, stream()))  # noqa: E731
        us = _batch_us([fn], 2, 5, filler)
        moved = wgs * threads * iters * 128
        emit("LDS reads (ds_read_b128)", "64 KB per workgroup", f"{wgs}x{threads}", f"{us:.1f}",
             f"{moved / us / 1e3 / 256:.0f} GB/s per CU", "divide by the clock for bytes per cycle")
    # dense FP8 MFMA
    iters = 20000
    for wgs in (256, 512, 1024):
        fn = lambda w=wgs: _lib.check(lib.fp8_probe_mfma(iters, ctypes.c_void_p(sink.data_ptr()), w,  # noqa: E731
                                                          stream()))
        us = _batch_us([fn], 2, 5, filler)
        flops = wgs * 4 * iters * 4 * 131072
        tf = flops / us / 1e6
        emit("FP8 MFMA 32x32x64", f"{iters} x 4 per wave", f"{wgs}x256", f"{us:.1f}",
             f"{tf:.0f} TFLOP/s ({tf / PEAK_TFLOPS:.2f} of 5.0 PF)",
             f"clock {tf * 1e12 / (256 * 8192) / 1e9:.2f} GHz")
    return lines


# Down projections fed straight from a gated MLP's [gate | up] output: the
# decode linears with SiLU-and-mul through the linear call (one launch where
# the library fuses; FP8W8A8_FUSED_LINEAR=all fuses at every M <= 4) and as the
# flagged quantizer followed by the GEMM.
SILU_LINEAR_SHAPES = [("channelwise", 4096, 12288), ("blockwise", 4096, 1536), ("blockwise", 7168, 2048)]


def measure_silu_linear(warmup, calls, filler):
    dev = torch.device("cuda:0")
    head = "| kind | N×K | M | path | launches | weight sets | µs per call | GB/s (weight + 2K-wide input) |"
    lines = [head, "|---|---|---|---|---|---|---|---|"]
    print(head, flush=True)
    print(lines[1], flush=True)
    for kind, n, k in SILU_LINEAR_SHAPES:
        sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / (n * k))))
        w = synth.weights(f"measure/silu/{kind}", n, k).to(torch.bfloat16).to(dev)
        if kind == "channelwise":
            wq, ws = ops.quant_per_token(w)
        else:
            wq, _ = ops.quant_per_token_group(w, 128, row_alignment=1)
            wq = wq.contiguous()
            ws = synth.positive_scales(f"measure/silu/{n}/{k}", (n // 128, k // 128)).to(dev)
        del w
        weights = [(wq.clone(), ws.clone()) for _ in range(sets)]
        for m in (1, 2, 4):
            x = synth.activations(f"measure/silu/{kind}", m, 2 * k).to(dev)
            m_pad = ops.padded_rows(m, 4)
            out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            q = torch.empty((m if kind == "channelwise" else m_pad, k), dtype=torch.uint8, device=dev)
            s = torch.empty((m,) if kind == "channelwise" else (k // 128, m_pad), dtype=torch.float32,
                            device=dev)
            if kind == "channelwise":
                one = [ops.prepare("linear_channelwise", x, wb, wsb, out=out, q=q, scale=s, silu_mul=True)
                       for wb, wsb in weights]
                quant = ops.prepare("silu_mul_quant_per_token", x, out=q, scale=s)
                gemms = [ops.prepare("scaled_mm_channelwise", q, wb, s, wsb, out=out) for wb, wsb in weights]
            else:
                one = [ops.prepare("linear_blockwise", x, wb, wsb, out=out, q=q, scale=s, row_alignment=4,
                                   silu_mul=True) for wb, wsb in weights]
                quant = ops.prepare("silu_mul_quant_per_token_group", x, 128, row_alignment=4, out=q,
                                    scale_storage=s)
                gemms = [ops.prepare("scaled_mm_blockwise", q, wb, s.transpose(0, 1), wsb, m=m, out=out)
                         for wb, wsb in weights]
            two = []
            for g in gemms:
                two.append(lambda g=g: (quant(), g()))
            nbytes = n * k + 4 * m * k
            kid = ops.KIND_CHANNELWISE if kind == "channelwise" else ops.KIND_BLOCKWISE
            nl1 = ops.linear_launches(kid, m, n, k, silu_mul=True)
            name1 = "linear call" + (" (single launch)" if nl1 == 1 else "")
            for name, fns, nl in ((name1, one, nl1), ("quantizer + GEMM", two, 2)):
                us = _batch_us(fns, warmup, calls, filler)
                line = (f"| {kind} | {n}×{k} | {m} | {name} | {nl} | {sets} | {us:.2f} | "
                        f"{nbytes / us / 1e3:.0f} |")
                lines.append(line)
                print(line, flush=True)
        del weights
        torch.cuda.empty_cache()
    return lines


def row(cfg, kind, n, k, m, r, bias):
    g = r["gemm"]
    p50 = percentile(g, 50)
    qp50 = percentile(r["quant"], 50)
    fl = 2 * m * n * k
    by = gemm_bytes(kind, m, n, k, bias)
    tf = fl / p50 / 1e6
    gb = by / p50 / 1e3
    conf = f"{r['variant']}" + (f" sk{r['split_k']}" if r["split_k"] > 1 else "") + \
        (" (table)" if r["table"] else "")
    return (f"| {cfg} | {kind} | {n}×{k} | {m} | `{conf}` | {r['rot_gib']:.2f} | "
            f"{p50:.1f} ({percentile(g, 10):.1f}–"
            f"{percentile(g, 90):.1f}) | {tf:.0f} | {gb:.0f} | {gb / PEAK_GBPS:.2f} | "
            f"{tf / PEAK_TFLOPS:.3f} | {qp50:.1f} ({quant_bytes(kind, m, k) / qp50 / 1e3:.0f} GB/s) | "
            f"{percentile(r['linear'], 50):.1f} ({r['launches']}) | {percentile(r['hot'], 50):.1f} |")


COUNTER_CASES = ("cw:4096:4096:64,cw:4096:4096:128,cw:4096:4096:256,bw:4096:4096:64,bw:4096:4096:128,"
                 "bw:4096:4096:256,bw:3072:4096:64,bw:4096:1536:64,cw:4096:12288:64,bw:7168:7168:64")
COUNTER_CALLS = 3


def counter_run(cases):
    """Driver for rocprofv3 counter and trace runs: a plain 256 MiB device
    copy (the byte counters' calibration), then, for every kind:N:K:M case,
    COUNTER_CALLS GEMMs with the default tile config, each on its own weight
    copy (so the weight comes from HBM), synchronised one by one."""
    dev = torch.device("cuda:0")
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for case in cases.split(","):
        kind_s, n, k, m = case.split(":")
        n, k, m = int(n), int(k), int(m)
        w = synth.weights("counters", n, k).to(torch.bfloat16).to(dev)
        x = synth.activations("counters", m, k).to(dev)
        if kind_s == "cw":
            wq, ws = ops.quant_per_token(w)
            a, sa = ops.quant_per_token(x)
            copies = [(wq.clone(), ws.clone()) for _ in range(COUNTER_CALLS)]
            cfg, _ = ops.tile_config(ops.KIND_CHANNELWISE, n, k, m)
            run = [lambda b=b, s_=s_: ops.scaled_mm_channelwise(a, b, sa, s_) for b, s_ in copies]
        else:
            wq, _ = ops.quant_per_token_group(w, 128, row_alignment=1)
            ws = synth.positive_scales(f"counters/{n}/{k}", (n // 128, k // 128)).to(dev)
            a, sa = ops.quant_per_token_group(x, 128, row_alignment=4)
            copies = [(wq.contiguous().clone(), ws.clone()) for _ in range(COUNTER_CALLS)]
            cfg, _ = ops.tile_config(ops.KIND_BLOCKWISE, n, k, m)
            run = [lambda b=b, s_=s_: ops.scaled_mm_blockwise(a, b, sa, s_, m=m) for b, s_ in copies]
        torch.cuda.synchronize()
        for f in run:
            f()
            torch.cuda.synchronize()
        print(json.dumps({"case": case, "variant": cfg["variant"], "split_k": cfg["split_k"]}), flush=True)
        del copies, w, x
        torch.cuda.empty_cache()


def counter_summary(fetch_csv, write_csv, trace_csv, cases, command):
    """Table of the counter_run dispatches: per case the kernel, its average
    duration (kernel trace), workgroups, and HBM bytes per call from
    FETCH_SIZE and WRITE_SIZE scaled by the calibration copy, against the
    algorithmic bytes."""
    import csv
    import re

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    def per_dispatch(path):
        d = {}
        for r in rows(path):
            key = int(r["Dispatch_Id"])
            d.setdefault(key, [re.sub(r"\(.*", "", r["Kernel_Name"]), int(r["Grid_Size"]), 0.0])
            d[key][2] += float(r["Counter_Value"])
        return [v for _, v in sorted(d.items())]

    def gemm_only(ds):
        # the calibration copy (the copy dispatch with the largest count)
        # first, then every case's quantizer launches and GEMMs; keep the GEMMs
        ci = max((i for i, v in enumerate(ds) if "copyBuffer" in v[0]), key=lambda i: ds[i][2])
        return ds[ci][2], [v for v in ds[ci + 1:] if "gemm_" in v[0]]

    cf, fetch = gemm_only(per_dispatch(fetch_csv))
    cw, write = gemm_only(per_dispatch(write_csv))
    ff, fw = 262144.0 / cf, 262144.0 / cw
    trace = [r for r in rows(trace_csv)]
    trace.sort(key=lambda r: int(r["Dispatch_Id"]))
    ci = max((i for i, r in enumerate(trace) if "copyBuffer" in r["Kernel_Name"]),
             key=lambda i: int(trace[i]["End_Timestamp"]) - int(trace[i]["Start_Timestamp"]))
    gemms = [r for r in trace[ci + 1:] if "gemm_" in r["Kernel_Name"]]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in gemms]
    wgs = [int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])) * int(r["Grid_Size_Y"]) *
           int(r["Grid_Size_Z"]) for r in gemms]
    out = [command, "",
           f"calibration: plain 256 MiB device copy reads FETCH_SIZE {cf:.1f} KiB (factor {ff:.4f}), "
           f"WRITE_SIZE {cw:.1f} KiB (factor {fw:.4f})", "",
           "| case | kernel | workgroups | us per call | HBM MB per call | algorithmic MB | ratio | GB/s (algorithmic) |",
           "|---|---|---|---|---|---|---|---|"]
    per = COUNTER_CALLS
    for i, case in enumerate(cases.split(",")):
        kind_s, n, k, m = case.split(":")
        n, k, m = int(n), int(k), int(m)
        sl = slice(i * per, (i + 1) * per)
        f, w, d = fetch[sl], write[sl], durs[sl]
        if not f:
            break
        hbm = sum(x[2] * ff + y[2] * fw for x, y in zip(f, w)) * 1024 / len(f)
        alg = m * k + n * k + 2 * m * n + (4 * m + 4 * n if kind_s == "cw" else
                                             4 * m * (k // 128) + 4 * (n // 128) * (k // 128))
        us = sum(d) / len(d)
        name = re.sub(r"^void fp8w8a8::", "", f[0][0])
        out.append(f"| {kind_s} {n}x{k} M={m} | `{name}` | {wgs[i * per]} | {us:.2f} | {hbm / 1e6:.2f} | "
                   f"{alg / 1e6:.2f} | {hbm / alg:.2f} | {alg / us / 1e3:.0f} |")
    return "\n".join(out) + "\n"


def step_table(bench_json, trace_csv, steps):
    """The per-(kind, M) table of the benchmark step from a kernel trace of
    ``bench.py --per-m --steps S --no-per-config --no-cpu-baseline``: the
    step's launches (one kernel each, in the order of the JSON's per_m) are
    the last S x L kernel dispatches; each row is the median over the S timed
    steps, with the launch's algorithmic flops and bytes."""
    import csv
    import re
    import statistics

    with open(bench_json) as f:
        line = [ln for ln in f if ln.startswith("{")][-1]
    per_m = json.loads(line)["per_m"]
    keys = list(per_m)
    with open(trace_csv) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    rows = [r for r in rows if "copyBuffer" not in r["Kernel_Name"] and "zero_words" not in r["Kernel_Name"]]
    n = len(keys)
    last = rows[-steps * n:]
    out = ["| config | kind | M | kernel | GPU median µs | TFLOP/s | GB/s | f_bw | f_mfma | roofline µs | quant µs (GB/s) |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    med = {}
    name = {}
    for j, key in enumerate(keys):
        us = [(int(last[s * n + j]["End_Timestamp"]) - int(last[s * n + j]["Start_Timestamp"])) / 1e3
              for s in range(steps)]
        med[key] = statistics.median(us)
        name[key] = re.sub(r"^void fp8w8a8::", "", re.sub(r"\(.*", "", last[j]["Kernel_Name"]))
    for kind in ("channelwise", "blockwise"):
        ms = sorted({int(k.split("M=")[1]) for k in keys if k.startswith(kind + "/")})
        for m in ms:
            g = f"{kind}/gemm/M={m}" if f"{kind}/gemm/M={m}" in per_m else f"{kind}/linear/M={m}"
            q = f"{kind}/quant/M={m}"
            us, fl, by = med[g], per_m[g]["flops"], per_m[g]["bytes"]
            roof = max(fl / 5e15, by / 8e12) * 1e6
            qcol = "fused" if q not in per_m else f"{med[q]:.1f} ({per_m[q]['bytes'] / med[q] / 1e3:.0f})"
            out.append(f"| o_proj 4096×4096 | {kind} | {m} | `{name[g]}` | {us:.1f} | {fl / us / 1e6:.0f} | "
                       f"{by / us / 1e3:.0f} | {by / us / 8e6:.2f} | {fl / us / 5e9:.3f} | {roof:.2f} | {qcol} |")
    total = sum(med.values())
    out.append("")
    out.append(f"sum of the step's kernel medians: {total:.0f} µs")
    return "\n".join(out) + "\n"


def traffic_summary(fetch_csv, write_csv, label, symbol, n, k, bm, bn, threads, command_tail):
    """Summary text of two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE,
    csv) of ``bench.py --profile-label LABEL``: the counters of each labelled
    dispatch after the 256 MiB calibration copy, scaled by what the copy
    reads (FETCH_SIZE) and writes (WRITE_SIZE) per KiB, against the
    algorithmic bytes of the launch (M from its grid: BM x BN tiles of
    `threads` threads)."""
    import csv
    import re

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench  # noqa: E402

    def agg(path):
        d = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (int(r["Dispatch_Id"]), re.sub(r"\(.*", "", r["Kernel_Name"]), int(r["Grid_Size"]))
                d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
        return sorted(d.items())

    copy_grid = (256 << 20) // 16 // 128  # the calibration copy's grid (16 bytes per lane)

    def pick(items):
        idx = max(i for i, ((_, kn, g), _) in enumerate(items) if "copyBuffer" in kn and g == copy_grid)
        return items[idx][1], [(kn, g, v) for (_, kn, g), v in items[idx + 1:] if symbol in kn]

    cf, lf = pick(agg(fetch_csv))
    cw, lw = pick(agg(write_csv))
    ff, fw = 262144.0 / cf, 262144.0 / cw

    def alg(m):
        return m * k + n * k + 2 * m * n + 4 * m * (k // 128) + 4 * (n // 128) * (k // 128)

    def m_of(grid):
        return grid // threads // ((n + bn - 1) // bn) * bm

    rows, tot = [], 0.0
    for i, ((_, g, f), (_, _, w)) in enumerate(zip(lf, lw)):
        t = (f * ff + w * fw) * 1024
        tot += t
        rows.append(f"  {i:4d}  {m_of(g):6d}  {f:11.1f}  {w:11.1f}  {t / 1e6:10.1f}  {alg(m_of(g)) / 1e6:10.1f}")
    cmd = f'python -u bench.py --profile-label "{label}"'
    return "\n".join([
        f"# HBM traffic of {label} ({command_tail})",
        "",
        "commands:",
        f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o f -- {cmd}",
        f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o w -- {cmd}",
        "  python -m fp8_w8a8_quantized_token_amd.measure --traffic-summary "
        "gpurun_out/pmc_fetch/f_counter_collection.csv gpurun_out/pmc_write/w_counter_collection.csv",
        "",
        f"calibration: plain 256 MiB device copy reads FETCH_SIZE {cf:.1f} KiB (factor {ff:.4f}), "
        f"WRITE_SIZE {cw:.1f} KiB (factor {fw:.4f})",
        "",
        "launch       M    FETCH_KiB    WRITE_KiB  traffic_MB  algorithmic_MB",
        *rows,
        "",
        f"label: {label}",
        f"kernel_symbol: {symbol}",
        f"traffic_bytes_per_launch: {int(round(tot / max(1, len(lf))))}",
        f"algorithmic_bytes_per_launch: {int(round(sum(alg(m_of(g)) for _, g, _ in lf) / max(1, len(lf))))}",
        f"source_sha256: {bench.kernel_source_hash()}",
        "note: FETCH_SIZE counts L2 misses, which includes reads the 256 MB last-level cache serves",
        "",
    ])


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default=",".join(synth.WORKLOADS))
    ap.add_argument("--calls", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--out", default="")
    ap.add_argument("--quant-variants", action="store_true",
                    help="time the quantizer variants (SiLU-and-mul, UE8M0, static) instead")
    ap.add_argument("--ue8m0-gemm", action="store_true",
                    help="time the 16x16 blockwise tile with fp32 and with power-of-two scales")
    ap.add_argument("--moe", action="store_true",
                    help="time the masked quantizer and grouped blockwise GEMM over MoE experts")
    ap.add_argument("--silu-linear", action="store_true",
                    help="time the decode down projection with SiLU-and-mul: one launch against two")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="time plain device copies and reductions at the small-M linears' byte counts")
    ap.add_argument("--library-reference", action="store_true",
                    help="time the large-M channelwise GEMMs through torch._scaled_mm (hipBLASLt) "
                         "beside this library's default tile (context, not part of the path)")
    ap.add_argument("--probes", action="store_true",
                    help="run the probe kernels: HBM read stream, L2 feed, FP8 MFMA rate and clock")
    ap.add_argument("--counter-run", nargs="?", const=COUNTER_CASES, default=None,
                    help="run the kind:N:K:M GEMMs (default: the mid-M cases) after a calibration "
                         "copy, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE and --kernel-trace runs")
    ap.add_argument("--counter-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "TRACE_CSV"),
                    help="summarise those three runs (no GPU needed)")
    ap.add_argument("--step-table", nargs=3, metavar=("BENCH_JSON_LOG", "TRACE_CSV", "STEPS"),
                    help="per-(kind, M) table of the benchmark step from a kernel trace (no GPU needed)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs of the benchmark's "
                         "dominant kernel (written to profiles/, no GPU needed)")
    args = ap.parse_args(argv)
    if args.step_table:
        print(step_table(args.step_table[0], args.step_table[1], int(args.step_table[2])))
        return 0
    if args.counter_summary:
        print(counter_summary(*args.counter_summary, COUNTER_CASES, ""))
        return 0
    if args.counter_run is not None:
        _lib.load()
        counter_run(args.counter_run)
        return 0
    if args.traffic_summary:
        txt = traffic_summary(*args.traffic_summary, label="gemm_blockwise[t256x256bw16]",
                              symbol="gemm_pingpong_kernel<1>", n=4096, k=4096,
                              bm=256, bn=256, threads=512, command_tail="o_proj N=K=4096 step launches")
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        with open(os.path.join(root, "profiles", "gemm_blockwise_t256x256bw16_o_proj_traffic.txt"), "w") as f:
            f.write(txt)
        print(txt)
        return 0
    _lib.load()
    dev = torch.device("cuda:0")
    want = args.workloads.split(",")
    filler = _Filler(dev)
    if (args.quant_variants or args.ue8m0_gemm or args.moe or args.stream_ceiling or args.silu_linear
            or args.probes or args.library_reference):
        t0 = time.time()
        mode = (measure_quant_variants if args.quant_variants else
                measure_ue8m0_gemm if args.ue8m0_gemm else
                measure_moe if args.moe else
                measure_probes if args.probes else
                measure_library_reference if args.library_reference else
                measure_silu_linear if args.silu_linear else measure_stream_ceiling)
        lines = mode(args.warmup, args.calls, filler)
        if args.stream_ceiling or args.silu_linear or args.probes or args.library_reference:
            note = (f"\n{args.calls} calls per row after {args.warmup} warm-up calls, timed as one "
                    f"batch with HIP events behind queued device copies (average per call); "
                    f"buffers rotated to cover >= 1 GiB. {time.time() - t0:.0f} s.")
        else:
            note = (f"\n{args.calls} launches per row after {args.warmup} warm-up launches, timed as "
                    f"one batch with HIP events (average per launch); GB/s from algorithmic bytes "
                    f"(bf16 input, codes, scales); weight sets rotated to cover >= 1 GiB. "
                    f"{time.time() - t0:.0f} s.")
        print(note, flush=True)
        if args.out:
            with open(args.out, "w") as f:
                f.write("\n".join(lines) + "\n" + note + "\n")
        return 0
    lines = [HEADER, "|" + "---|" * 14]
    print(HEADER, flush=True)
    print(lines[1], flush=True)
    t0 = time.time()
    floor = percentile(time_calls([lambda: None], args.warmup, args.calls, filler), 50)
    for cfg in want:
        w = synth.WORKLOADS[cfg]
        kind, with_bias = w["kind"], w["bias"]
        for n, k in w["shapes"]:
            buf = ShapeBuffers(cfg, kind, n, k, with_bias, dev)
            for m in w["ms"]:
                r = measure_m(buf, cfg, m, w["outliers"], args.warmup, args.calls, filler)
                line = row(cfg, kind, n, k, m, r, with_bias)
                lines.append(line)
                print(line, flush=True)
                torch.cuda.empty_cache()
            del buf
            torch.cuda.empty_cache()
    note = (f"\n{args.calls} timed calls after {args.warmup} warm-up calls per mode; HIP events "
            f"around each call, all calls queued behind device copies; up to {MAX_SETS} weight "
            f"sets rotated (GiB column: distinct weight bytes the timed calls touch; hot: one "
            f"set repeated). An event pair around no launch measures {floor:.1f} us (p50). "
            f"{time.time() - t0:.0f} s.")
    print(note, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write("\n".join(lines) + "\n" + note + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
