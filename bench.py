"""Benchmark of the FP8 W8A8 linear hot path on one MI355X.

One step = one pass of the whole hot path over the o_proj workload (N = K =
4096, M in 8192, 4096, ..., 1): for every M, the channelwise linear (per-token
quant, tile-config lookup, channelwise scaled GEMM with its fused epilogue and
in-launch split-K reduction) and the blockwise linear (row-padded group-128
quant, lookup, blockwise scaled GEMM). For M <= 4 each linear is one launch,
the quantization fused into the skinny GEMM (it still writes the codes and
scales); above, the quantizer and the GEMM are two launches. Inputs are synthetic and resident in HBM
before timing starts; every (M, kind) has its own weight copy, so a step
touches ~1 GB and the 256 MB last-level cache cannot serve the weights.

Output: one JSON line. ``value`` is the step's GEMM TFLOP/s (sum of 2MNK over
the step time, quant included in the time). ``roofline`` reports the kernel
with the largest share of GPU time: an untimed pass with HIP events around
every launch picks it, and inside the timed steps HIP events (on the stream
the kernels run on) bracket only that kernel's launches, so the step time is
not inflated by per-launch event records. ``cpu_baseline`` times the CPU
oracle on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-GEMM TFLOP/s and GB/s vs roofline, Qwen3-8B shapes, M=1..8192"
PEAK_TFLOPS_FP8 = 5000.0  # MI355X dense FP8 MFMA
PEAK_GBPS = 8000.0        # MI355X HBM3E
ID_PASSES = 3  # identification steps before the timed region
RIDGE = PEAK_TFLOPS_FP8 * 1e12 / (PEAK_GBPS * 1e9)
MS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192]
N = K = 4096


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-(shape, M) pass over the other workloads")
    ap.add_argument("--per-m", action="store_true", help="also print a per-(M, kind) table")
    ap.add_argument("--profile-label", default="",
                    help="run only the step's launches with this label (after a plain 256 MiB "
                         "device copy used to calibrate HBM byte counters), for rocprofv3 --pmc")
    return ap.parse_args()


def gemm_bytes(kind, m, n, k, bias=False):
    b = m * k + n * k + 2 * m * n + (2 * n if bias else 0)
    if kind == "channelwise":
        b += 4 * m + 4 * n
    else:
        b += 4 * m * (k // 128) + 4 * (n // 128) * (k // 128)
    return b


def quant_bytes(m, k, group):
    return 3 * m * k + 4 * m * (k // group)


class Launch:
    """One kernel launch of the step with its label and algorithmic cost."""

    def __init__(self, label, fn, flops, nbytes):
        self.label, self.fn, self.flops, self.nbytes = label, fn, flops, nbytes


def build_step(torch, ops, synth, dev):
    launches = []
    w_host = synth.weights("o_proj", N, K).to(torch.bfloat16)
    # largest M first: while the GPU runs the long GEMMs the host queues every
    # later launch, so the short kernels at the end run back to back and the
    # events around each launch time the kernel, not the host's launch cost
    for kind in ("channelwise", "blockwise"):
        for m in sorted(MS, reverse=True):
            x = synth.activations("o_proj", m, K, outlier_frac=0.01).to(dev)
            w = w_host.to(dev)
            kind_id = ops.KIND_CHANNELWISE if kind == "channelwise" else ops.KIND_BLOCKWISE
            fused = ops.linear_launches(kind_id, m, N, K) == 1
            if kind == "channelwise":
                wq, ws = ops.quant_per_token(w)           # per-output-channel weight quant
                q = torch.empty((m, K), dtype=torch.uint8, device=dev)
                s = torch.empty((m,), dtype=torch.float32, device=dev)
                out = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                cfg, _ = ops.tile_config(0, N, K, m)
                label_q = "quant_per_token"
                label_g = f"gemm_channelwise[{cfg['variant']}]"

                if fused:
                    fl = ops.prepare("linear_channelwise", x, wq, ws, out=out, q=q, scale=s)
                else:
                    fq = ops.prepare("quant_per_token", x, out=q, scale=s)
                    fg = ops.prepare("scaled_mm_channelwise", q, wq, s, ws, out=out)
                qb = quant_bytes(m, K, K)
            else:
                # codes from the group-128 quant of the weight rows, scales as
                # synthetic 128x128 block scales (timing does not depend on them)
                wq, _ = ops.quant_per_token_group(w, 128, row_alignment=1)
                wq = wq.contiguous()
                ws = synth.positive_scales("o_proj/wblk", (N // 128, K // 128)).to(dev)
                m_pad = ops.padded_rows(m, 4)
                q = torch.empty((m_pad, K), dtype=torch.uint8, device=dev)
                st = torch.empty((K // 128, m_pad), dtype=torch.float32, device=dev)
                out = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                cfg, _ = ops.tile_config(1, N, K, m)
                label_q = "quant_per_token_group"
                label_g = f"gemm_blockwise[{cfg['variant']}]"

                if fused:
                    fl = ops.prepare("linear_blockwise", x, wq, ws, row_alignment=4, out=out, q=q,
                                     scale=st)
                else:
                    fq = ops.prepare("quant_per_token_group", x, 128, row_alignment=4, out=q,
                                     scale_storage=st)
                    fg = ops.prepare("scaled_mm_blockwise", q, wq, st.transpose(0, 1), ws, m=m,
                                     out=out)
                qb = quant_bytes(m, K, 128)
            if fused:
                # x read once, codes and scales still written, codes not re-read
                step = [Launch(f"linear_{kind}_fused[{cfg['variant']}]", fl, 2 * m * N * K,
                               qb + gemm_bytes(kind, m, N, K) - m * K)]
                step[0].part = "linear"
            else:
                step = [Launch(label_q, fq, 0, qb),
                        Launch(label_g, fg, 2 * m * N * K, gemm_bytes(kind, m, N, K))]
                step[0].part, step[1].part = "quant", "gemm"
            for l in step:
                l.m, l.kind = m, kind
            launches += step
    torch.cuda.synchronize()
    return launches


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "fp8_w8a8_quantized_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(label):
    """HBM bytes per launch of `label` from a committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (profiles/*_traffic.txt), or None when there is none or
    the kernel sources changed since the counters were taken."""
    import glob
    cur = kernel_source_hash()
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt")):
        kv = {}
        with open(path) as fh:
            for line in fh:
                if ": " in line and not line.startswith(" "):
                    k, v = line.rstrip("\n").split(": ", 1)
                    kv[k] = v
        if kv.get("label") == label and kv.get("source_sha256") == cur:
            return float(kv["traffic_bytes_per_launch"])
    return None


# The other workloads, measured after the timed steps (not part of `value`):
# (config label, kind, N, K, M values, bias, outlier fraction)
PER_CONFIG = [
    ("small 256x512", "channelwise", 256, 512, [16], False, 0.0),
    ("qkv 6144x4096", "channelwise", 6144, 4096, [1, 64, 512, 8192], True, 0.0),
    ("down 4096x12288", "channelwise", 4096, 12288, [1, 64, 512, 8192], True, 0.0),
    ("gate_up 24576x4096", "channelwise", 24576, 4096, [1, 64, 512, 8192], True, 0.0),
    ("block 7168x7168", "blockwise", 7168, 7168, [1, 2, 3, 5, 7, 13, 31, 64, 256], False, 0.0),
    ("block 3072x4096", "blockwise", 3072, 4096, [1, 4, 16, 64, 4096], False, 0.0),
    ("block 4096x1536", "blockwise", 4096, 1536, [1, 4, 16, 64, 4096], False, 0.0),
]


def _sig(x, d=4):
    return float(f"{x:.{d}g}")


def per_config(torch, ops, synth, dev, warmup=10, calls=40):
    """GEMM, quantizer and whole-linear time of every (shape, M) of the other
    workloads: each timed as one batch of back-to-back calls behind queued
    device copies (HIP events around the batch, not per call), the GEMM's
    weight rotating over copies that cover >= 1 GiB so every call reads it
    from HBM. frac = roofline time (max of 2MNK / 5 PFLOP/s and algorithmic
    bytes / 8 TB/s) / GEMM time."""
    import math

    from fp8_w8a8_quantized_token_amd import measure

    filler = measure._Filler(dev)
    out = {}
    rows = []
    for label, kind, n, k, ms, with_bias, outl in PER_CONFIG:
        sets = max(2, min(64, math.ceil((1 << 30) / (n * k))))
        w = synth.weights(f"bench/{label}", n, k).to(torch.bfloat16).to(dev)
        if kind == "channelwise":
            wq, ws = ops.quant_per_token(w)
        else:
            wq, _ = ops.quant_per_token_group(w, 128, row_alignment=1)
            wq = wq.contiguous()
            ws = synth.positive_scales(f"bench/{label}/wblk", (n // 128, k // 128)).to(dev)
        del w
        weights = [(wq.clone(), ws.clone()) for _ in range(sets)]
        bias = synth.bias(f"bench/{label}", n).to(dev) if with_bias else None
        rec = {"kind": kind, "M": [], "variant": [], "gemm_us": [], "quant_us": [], "linear_us": [],
               "tflops": [], "gbps": [], "bound": [], "frac": []}
        for m in ms:
            x = synth.activations(f"bench/{label}", m, k, outlier_frac=outl).to(dev)
            m_pad = ops.padded_rows(m, 4) if kind == "blockwise" else m
            o = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            q = torch.empty((m_pad, k), dtype=torch.uint8, device=dev)
            st = (torch.empty((m,), dtype=torch.float32, device=dev) if kind == "channelwise"
                  else torch.empty((k // 128, m_pad), dtype=torch.float32, device=dev))
            if kind == "channelwise":
                fq = ops.prepare("quant_per_token", x, out=q, scale=st)
                fq()
                fg = [ops.prepare("scaled_mm_channelwise", q, wb, st, wsb, bias=bias, out=o)
                      for wb, wsb in weights]
                fl = [ops.prepare("linear_channelwise", x, wb, wsb, bias=bias, out=o, q=q, scale=st)
                      for wb, wsb in weights]
            else:
                fq = ops.prepare("quant_per_token_group", x, 128, row_alignment=4, out=q, scale_storage=st)
                fq()
                fg = [ops.prepare("scaled_mm_blockwise", q, wb, st.transpose(0, 1), wsb, bias=bias, m=m,
                                  out=o) for wb, wsb in weights]
                fl = [ops.prepare("linear_blockwise", x, wb, wsb, bias=bias, row_alignment=4, out=o, q=q,
                                  scale=st) for wb, wsb in weights]
            g_us = measure._batch_us(fg, warmup, calls, filler)
            q_us = measure._batch_us([fq], warmup, calls, filler)
            l_us = measure._batch_us(fl, warmup, calls, filler)
            flops = 2 * m * n * k
            nbytes = gemm_bytes(kind, m, n, k, with_bias)
            t_roof = max(flops / (PEAK_TFLOPS_FP8 * 1e12), nbytes / (PEAK_GBPS * 1e9))
            cfg, _ = ops.tile_config(ops.KIND_CHANNELWISE if kind == "channelwise" else ops.KIND_BLOCKWISE,
                                     n, k, m)
            rec["M"].append(m)
            rec["variant"].append(cfg["variant"] + (f"/sk{cfg['split_k']}" if cfg["split_k"] > 1 else ""))
            rec["gemm_us"].append(_sig(g_us))
            rec["quant_us"].append(_sig(q_us))
            rec["linear_us"].append(_sig(l_us))
            rec["tflops"].append(_sig(flops / g_us / 1e6))
            rec["gbps"].append(_sig(nbytes / g_us / 1e3))
            rec["bound"].append("mfma" if flops / nbytes >= RIDGE else "hbm")
            rec["frac"].append(_sig(t_roof * 1e6 / g_us, 3))
            rows.append(f"{label:20s} {kind:11s} M={m:5d} {rec['variant'][-1]:18s} gemm {g_us:8.2f} us  "
                        f"quant {q_us:6.2f}  linear {l_us:8.2f}  {flops / g_us / 1e6:7.1f} TF/s  "
                        f"{nbytes / g_us / 1e3:6.0f} GB/s  frac {t_roof * 1e6 / g_us:.3f} ({rec['bound'][-1]})")
            print(rows[-1], file=sys.stderr, flush=True)
            del fq, fg, fl
        out[label] = rec
        del weights
        torch.cuda.empty_cache()
    return out


def cpu_baseline():
    """The oracle (numpy, fp64 GEMM) on a bounded sample of the same workload."""
    import numpy as np
    import threadpoolctl

    import oracle
    from fp8_w8a8_quantized_token_amd import synth

    cores = len(os.sched_getaffinity(0))
    with threadpoolctl.threadpool_limits(limits=cores):
        threads = max([d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()] or [1])
        w = synth.weights("o_proj", N, K).numpy()
        wq_c, ws_c = oracle.quant_weight_per_channel(w)
        wq_b, ws_b = oracle.quant_weight_blockwise(w)
        sample = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192]
        flops = 0
        t0 = time.perf_counter()
        for m in sample:
            x = synth.activations("o_proj", m, K, outlier_frac=0.01).float().numpy()
            q, s = oracle.quant_per_token(x)
            oracle.scaled_mm_channelwise(q, wq_c, s, ws_c)
            qg, sg = oracle.quant_per_token_group(x, 128)
            oracle.scaled_mm_blockwise(qg, wq_b, sg, ws_b)
            flops += 2 * (2 * m * N * K)
        dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"o_proj N=K=4096, M in {sample}, channelwise + blockwise linear "
                      f"(quant + fp64 GEMM), {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is described in the design notes but not built.", flush=True)
        sys.exit(2)
    import torch

    from fp8_w8a8_quantized_token_amd import _lib, ops, synth

    _lib.load()
    dev = torch.device("cuda:0")
    launches = build_step(torch, ops, synth, dev)
    if args.profile_label:
        # counter collection: a plain copy of known size, then the labelled launches
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        sel = [l for l in launches if l.label == args.profile_label]
        if not sel:
            sys.exit(f"no launch labelled {args.profile_label}")
        for l in sel:
            l.fn()
        torch.cuda.synchronize()
        print(json.dumps({"profiled": args.profile_label, "launches": len(sel),
                          "m": [getattr(l, "m", None) for l in sel],
                          "bytes": [l.nbytes for l in sel], "flops": [l.flops for l in sel]}),
              flush=True)
        return
    flops_step = sum(l.flops for l in launches)
    bytes_step = sum(l.nbytes for l in launches)

    for _ in range(args.warmup):
        for l in launches:
            l.fn()
    torch.cuda.synchronize()

    # Identification passes (untimed): events around every launch give each
    # kernel's share of the step (summed over ID_PASSES steps, so one slow
    # launch cannot decide it) and the per-(kind, M) table (median).
    probe = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in launches] for _ in range(ID_PASSES)]
    for row in probe:
        for (e0, e1), l in zip(row, launches):
            e0.record()
            l.fn()
            e1.record()
    torch.cuda.synchronize()
    share = {}
    per_m = {}
    for i, l in enumerate(launches):
        us_all = sorted(row[i][0].elapsed_time(row[i][1]) * 1e3 for row in probe)
        share[l.label] = share.get(l.label, 0.0) + sum(us_all)
        key = f"{l.kind}/{l.part}/M={l.m}"
        per_m[key] = {"us_event": us_all[len(us_all) // 2], "flops": l.flops, "bytes": l.nbytes}
    dom_label = max(share, key=share.get)
    dom_idx = [i for i, l in enumerate(launches) if l.label == dom_label]

    # Timed region: K whole steps; HIP events (on the launch stream, torch's
    # current stream) bracket only the dominant kernel's launches.
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in dom_idx] for _ in range(args.steps)]
    dom_set = set(dom_idx)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        j = 0
        for i, l in enumerate(launches):
            if i in dom_set:
                ev[s][j][0].record()
                l.fn()
                ev[s][j][1].record()
                j += 1
            else:
                l.fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps

    dom = {"count": 0, "time": 0.0, "flops": 0, "bytes": 0}
    for s in range(args.steps):
        for j, i in enumerate(dom_idx):
            dom["count"] += 1
            dom["time"] += ev[s][j][0].elapsed_time(ev[s][j][1]) * 1e-3
            dom["flops"] += launches[i].flops
            dom["bytes"] += launches[i].nbytes
    avg = dom["time"] / dom["count"]
    flops_launch = dom["flops"] / dom["count"]
    bytes_launch = dom["bytes"] / dom["count"]
    if flops_launch > 0 and flops_launch / bytes_launch >= RIDGE:
        roof = {"bound": "mfma", "achieved": flops_launch / avg / 1e12, "peak": PEAK_TFLOPS_FP8,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": bytes_launch / avg / 1e9, "peak": PEAK_GBPS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom_label)
    roof["kernel"] = dom_label
    roof["avg_launch_us"] = avg * 1e6
    roof["launches_per_step"] = dom["count"] // args.steps

    result = {
        "metric": METRIC,
        "value": flops_step / step_s / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "o_proj N=K=4096, M in 1..8192 (powers of 2); channelwise and "
                               "blockwise FP8 linear (quant + scaled GEMM) per M",
                   "gemm_gflop_per_step": flops_step / 1e9, "bytes_per_step": bytes_step},
        "gbps": bytes_step / step_s / 1e9,
        "roofline": roof,
    }
    if args.per_m:
        result["per_m"] = per_m
    if not args.no_per_config:
        result["per_config"] = per_config(torch, ops, synth, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
