"""Offline tile-config sweep on gfx950: fills the per-(N, K) tables.

The PR 34331 digest ("Tune FP8 GEMM Triton tiles on L40S and enable them by
default", sections "Motivation" and "Implementation" step 5) describes an
offline scan of tile configurations per weight shape and token count whose
winners go into one JSON table per (N, K, device, dtype), M -> config, with
null entries where the default path wins. This script does the same for this
library's compiled gfx950 kernels: for every (kind, N, K) and every M of the
grid it times each candidate kernel variant / split-K factor, keeps the
fastest, and writes ``configs/N={N},K={K},device_name=gfx950,dtype=fp8_w8a8_{kind}.json``.

Timing: prepared launches (no host work per launch) cycling over enough
copies of the weight to exceed the 256 MB last-level cache, so the weight is
read from HBM as in a real forward pass; HIP events around the whole sequence
on the launch stream; the median of several repetitions.

Usage: python -m fp8_w8a8_quantized_token_amd.sweep [--kinds channelwise,blockwise]
       [--shapes 4096x4096,...] [--ms 1,2,4,...] [--out DIR] [--merge]
"""
import argparse
import json
import os
import statistics
import sys

import torch

from . import _lib, ops, synth

PKG = os.path.dirname(os.path.abspath(__file__))

SHAPES = {
    "channelwise": [(256, 512), (4096, 4096), (6144, 4096), (4096, 12288), (24576, 4096)],
    "blockwise": [(7168, 7168), (3072, 4096), (4096, 1536), (4096, 4096)],
}
MS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192]


def candidates(kind, m, n, k):
    """Kernel variants worth timing at this M: register-staged tiles always;
    the LDS-DMA tiles where their K condition holds (64-byte stages:
    channelwise, K % 64 == 0; panel rings: K % 128 == 0); the blockwise
    256x256 register-staged tiles run out of registers and are left out."""
    k128 = k % 128 == 0
    if m <= 32:
        # the skinny kernel re-reads all M activation rows per 16 weight rows;
        # from M = 8 the 32- and 64-wide deep-ring tiles can win on large N;
        # up to 64 rows the LDS-DMA decode stream
        c = [("skinny", 1)]
        if k128:
            c += [("decode", 1)]
        if m >= 8 and k128:
            c += [("t32x32deep", 1), ("t32x32deep", 2), ("t32x32deep", 4), ("t64x32deep", 1),
                  ("t64x32deep", 2), ("t64x32deep", 4), ("t64x64deep", 1), ("t64x64deep", 2),
                  ("t64x64deep", 4), ("t64x64panel", 1), ("t64x64panel", 2), ("t64x64panel", 4)]
        return c
    c = [("decode", 1)] if (k128 and m <= 64) else []
    if m <= 1024:
        c += [("t64x64", 1), ("t128x64k256", 1), ("t64x128k256", 1), ("t128x128k256", 1)]
        if k128:
            c += [("t64x64panel", 1), ("t64x64panel", 2), ("t64x64panel", 4), ("t128x64panel", 1),
                  ("t128x64panel", 2), ("t128x64panel", 4), ("t64x64deep", 1), ("t64x64deep", 2),
                  ("t64x64deep", 4), ("t128x64deep", 1), ("t128x64deep", 2)]
            if m <= 256:
                c += [("t32x32deep", 1), ("t32x32deep", 2), ("t32x32deep", 4), ("t64x32deep", 1),
                      ("t64x32deep", 2), ("t64x32deep", 4)]
    if m >= 256:
        c += [("t128x128", 1), ("t128x128k256", 1), ("t256x128w8", 1)]
        if kind == "channelwise" and k % 64 == 0:
            c += [("t128x128dma", 1), ("t256x128dma", 1)]
        if k128:
            c += [("t128x64panel", 1), ("t128x128panel", 1), ("t256x128panel", 1),
                  ("t128x64panel8", 1), ("t128x128panel8", 1), ("t128x128panel", 2),
                  ("t128x128panel8", 2)]
    if m >= 1024:
        c += [("t256x128", 1)]
        if k128:
            c += [("t256x128panel", 2)]
        if kind == "blockwise" and k128:
            c += [("t256x256bw16", 1), ("t256x256bw16", 2)]
        if kind == "channelwise":
            c += [("t256x256w8", 1)]
            if k % 64 == 0:
                c += [("t256x256dma", 1)]
            if k128:
                c += [("t256x256panel", 1)]
    out = []
    for v in c:
        if v not in out:
            out.append(v)
    return out


class Shape:
    """Device buffers for one (kind, N, K): rotating weight copies."""

    def __init__(self, kind, n, k, dev):
        self.kind, self.n, self.k, self.dev = kind, n, k, dev
        w = synth.weights(f"sweep/{kind}", n, k).to(torch.bfloat16).to(dev)
        copies = max(2, min(16, (512 << 20) // (n * k) + 1))
        self.w = []
        for _ in range(copies):
            if kind == "channelwise":
                q, s = ops.quant_per_token(w)
            else:
                q, _ = ops.quant_per_token_group(w, 128, row_alignment=1)
                q = q.contiguous()
                s = synth.positive_scales(f"sweep/{n}/{k}", (n // 128, k // 128)).to(dev)
            self.w.append((q, s))
        del w

    def launches(self, m, cfg):
        dev, n, k = self.dev, self.n, self.k
        x = synth.activations(f"sweep/{self.kind}", m, k).to(dev)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        fns = []
        if self.kind == "channelwise":
            a, sa = ops.quant_per_token(x)
            for q, s in self.w:
                fns.append(ops.prepare("scaled_mm_channelwise", a, q, sa, s, out=out, config=cfg))
        else:
            a, sa = ops.quant_per_token_group(x, 128, row_alignment=4)
            for q, s in self.w:
                fns.append(ops.prepare("scaled_mm_blockwise", a, q, sa, s, m=m, out=out, config=cfg))
        return fns


def time_launches(fns, min_launches=24, reps=5):
    for f in fns:
        f()
    torch.cuda.synchronize()
    rounds = max(1, -(-min_launches // len(fns)))
    per = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(rounds):
            for f in fns:
                f()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / (rounds * len(fns)))
    return statistics.median(per)


def sweep_shape(kind, n, k, ms, dev, log):
    shp = Shape(kind, n, k, dev)
    kid = _lib.KIND_CHANNELWISE if kind == "channelwise" else _lib.KIND_BLOCKWISE
    table = {}
    for m in ms:
        default = ops.default_tile_config(kid, n, k, m)
        cands = candidates(kind, m, n, k)
        dkey = (default["variant"], default["split_k"])
        if dkey not in cands:
            cands = [dkey] + cands
        results = {}
        for v, sk in cands:
            try:
                fns = shp.launches(m, ops.make_config(v, sk))
            except _lib.Fp8Error as e:
                log(f"  {kind} N={n} K={k} M={m} {v} sk={sk}: rejected ({e})")
                continue
            results[(v, sk)] = time_launches(fns)
        best = min(results, key=results.get)
        t_best, t_def = results[best], results.get(dkey, float("inf"))
        # null: the default heuristic is as fast (within 2%) -- keep the default
        if t_def <= t_best * 1.02:
            table[str(m)] = None
        else:
            table[str(m)] = {"variant": best[0], "split_k": best[1], "us": round(t_best, 2)}
        log(f"  {kind} N={n} K={k} M={m}: best {best[0]} sk={best[1]} {t_best:.2f} us, "
            f"default {dkey[0]} sk={dkey[1]} {t_def:.2f} us -> "
            f"{'null' if table[str(m)] is None else best[0]}")
    return table


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--kinds", default="channelwise,blockwise")
    ap.add_argument("--shapes", default="", help="NxK list, e.g. 4096x4096,6144x4096")
    ap.add_argument("--ms", default=",".join(map(str, MS)))
    ap.add_argument("--out", default=os.path.join(PKG, "configs"))
    ap.add_argument("--merge", action="store_true",
                    help="keep the existing table's entries for the M not swept")
    args = ap.parse_args(argv)
    dev = torch.device("cuda:0")
    ms = [int(x) for x in args.ms.split(",")]
    os.makedirs(args.out, exist_ok=True)

    def log(msg):
        print(msg, flush=True)

    # time the kernels alone: tables must not steer the candidates' configs
    os.environ["FP8W8A8_TUNED_CONFIGS"] = "0"
    for kind in args.kinds.split(","):
        shapes = SHAPES[kind]
        if args.shapes:
            shapes = [tuple(int(v) for v in s.split("x")) for s in args.shapes.split(",")]
        for n, k in shapes:
            log(f"sweeping {kind} N={n} K={k}")
            table = sweep_shape(kind, n, k, ms, dev, log)
            path = os.path.join(args.out, f"N={n},K={k},device_name=gfx950,dtype=fp8_w8a8_{kind}.json")
            if args.merge and os.path.exists(path):
                with open(path) as f:
                    old = json.load(f)
                old.update(table)
                table = {str(m): old[str(m)] for m in sorted(int(x) for x in old)}
            with open(path, "w") as f:
                json.dump(table, f, indent=1)
            log(f"wrote {path}")
            torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
