#!/usr/bin/env python3
"""Benchmark of the LoRA linear layer (forward + backward) on one MI355X.

A step is one forward and one backward pass of the LoRA linear layer for both
projection shapes of the LLaMA-8B-like workload (m = 8192 tokens,
k = 4096 -> n = 4096 and k = 4096 -> n = 14336, r = 16, alpha = 2, p = 0.1),
inputs already resident in HBM.  Every step runs the whole path: dropout mask
and down-projection, base GEMM with the fused LoRA epilogue, dS/dB, dA, and the
input-gradient GEMM with the fused masked LoRA term.

Prints one JSON line: tokens/s (m / step time), per-step milliseconds, the
roofline of the dominant kernel (algorithmic FLOPs per launch / its average
launch time from HIP events on the launch stream), the same-GEMM frozen layer
for the slowdown ratio, and the CPU oracle timed on a bounded row sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA-linear fwd+bwd tokens/sec at 1 MI355X; % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows (tokens) of the workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shapes", default="4096,14336", help="n of each projection (k = 4096)")
    ap.add_argument("--m", type=int, default=8192)
    ap.add_argument("--r", type=int, default=16)
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB (byte-counter calibration)")
    ap.add_argument("--unfused-only", action="store_true",
                    help="time only the eager PyTorch LoRA sequence (for its byte counters)")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the headline step: the mixed-adapter workloads and the rank/token "
                         "sweep, fused vs frozen, one JSON line per case")
    ap.add_argument("--pack", action="store_true",
                    help="instead of the headline step: the host packer (greedy token-capacity "
                         "packing and segment tables) on a synthetic global batch; no GPU")
    ap.add_argument("--dora", action="store_true",
                    help="instead of the headline step: the DoRA norm of W + alpha A B per output "
                         "feature at 8192 x 8192, ranks 16, 64 and 256 (one JSON line each)")
    ap.add_argument("--concat", action="store_true",
                    help="instead of the headline step: at p = 0, the library's forward against the "
                         "concatenated down-projection X [W | A] plus a separate Y += alpha S B pass")
    return ap.parse_args()


def concat_report(args):
    """The concatenated down-projection for p = 0: S comes out of the base GEMM
    as r extra output columns (X [W | A]), so X is read once, but the LoRA term
    then needs its own pass over Y (Y += alpha S B, read and write of Y) because
    no work-group holds S for its rows before its epilogue.  Timed from its
    parts on the headline shapes: this library's GEMM on the k x (n + r) weight
    (its 256-column tiles give the r extra columns a tile of their own), and
    torch.addmm for the update (hipBLASLt with beta = 1).  Beside it, the
    library's forward at p = 0 (the mask-free F1 pass over X, then the GEMM
    with the LoRA term in its epilogue)."""
    import torch

    import lora_fine_tuning_amd as lf

    lf.load()
    m, k, r, alpha = args.m, 4096, args.r, 2.0
    g = torch.Generator(device="cuda").manual_seed(3)

    def timed(fn, iters):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    for n in (int(v) for v in args.shapes.split(",")):
        X = torch.randn(m, k, device="cuda", generator=g).bfloat16()
        W = (torch.randn(k, n, device="cuda", generator=g) / k ** 0.5).bfloat16()
        A = (torch.randn(k, r, device="cuda", generator=g) / k ** 0.5).bfloat16()
        B = (torch.randn(r, n, device="cuda", generator=g) * 0.02 ** 0.5).bfloat16()
        Wc = torch.cat([W, A], dim=1).contiguous()
        Y = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
        Yc = torch.empty(m, n + r, device="cuda", dtype=torch.bfloat16)
        S = torch.empty(m, r, device="cuda", dtype=torch.float32)
        ws = torch.empty(max(lf.lora_linear_fwd_workspace_size(m, k, n, r), 1), dtype=torch.uint8, device="cuda")
        Sb = torch.randn(m, r, device="cuda", generator=g).bfloat16()
        fused = timed(lambda: lf.lora_linear_fwd(X, W, A, B, alpha, 0.0, Y=Y, S=S, workspace=ws), args.steps)
        gemm_cat = timed(lambda: lf.lora_frozen_fwd(X, Wc, Y=Yc), args.steps)
        gemm = timed(lambda: lf.lora_frozen_fwd(X, W, Y=Y), args.steps)
        update = timed(lambda: Y.addmm_(Sb, B, alpha=alpha), args.steps)
        print(json.dumps({"metric": "forward ms at p = 0: fused path vs concatenated down-projection",
                          "config": {"workload": f"m {m} k {k} n {n} r {r}"},
                          "fused_fwd_ms": fused, "frozen_gemm_ms": gemm,
                          "concat_gemm_ms": gemm_cat, "update_pass_ms": update,
                          "concat_total_ms": gemm_cat + update,
                          "concat_over_fused": (gemm_cat + update) / fused}), flush=True)
        del X, W, A, B, Wc, Y, Yc, S, ws, Sb


def dora_report(args):
    """DoRA norm on the page's 8192 x 8192 weight shape.  One pass over W is the
    compulsory traffic (bytes = 2kn + 2kr + 2rn + 4n per call); the kernel is
    reported against HBM.  Beside it: the eager PyTorch form that builds the
    dense A B (torch.linalg.vector_norm(W + alpha A B, dim=0) in fp32), and
    the oracle on a column sample."""
    import torch

    import lora_fine_tuning_amd as lf

    lf.load()
    k = n = 8192
    for r in (16, 64, 256):
        g = torch.Generator(device="cuda").manual_seed(7 + r)
        W = (torch.randn(k, n, device="cuda", generator=g) / k ** 0.5).bfloat16()
        A = (torch.randn(k, r, device="cuda", generator=g) / k ** 0.5).bfloat16()
        B = (torch.randn(r, n, device="cuda", generator=g) * 0.02 ** 0.5).bfloat16()
        norm = torch.empty(n, dtype=torch.float32, device="cuda")
        ws = torch.empty(lf.lora_dora_norm_workspace_size(k, n, r), dtype=torch.uint8, device="cuda")

        def fused():
            lf.lora_dora_norm(W, A, B, 2.0, norm=norm, workspace=ws)

        def eager():
            return torch.linalg.vector_norm(W.float() + 2.0 * (A.float() @ B.float()), dim=0)

        for _ in range(args.warmup):
            fused()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fused()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        # the pass over W alone: HIP events the library records on its launch stream
        lf.lora_profiling_enable(True, capacity=4 * args.steps + 16)
        lf.lora_profiling_reset()
        for _ in range(args.steps):
            fused()
        c, tot = lf.lora_profiling_query("dora_norm_pass")
        kern_ms = tot / max(c, 1)
        lf.lora_profiling_enable(False)
        for _ in range(2):
            eager()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            eager()
        e1.record()
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / 5
        nbytes = 2 * k * n + 2 * k * r + 2 * r * n + 4 * n
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        line = {"metric": "DoRA norm of W + alpha A B per output feature, GB/s of compulsory traffic",
                "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms": ms, "steps": args.steps,
                "warmup": args.warmup, "higher_is_better": True, "dtype": "bf16 in, fp32 sums",
                "data": "synthetic", "config": {"workload": f"W {k} x {n}, r {r}"},
                "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": achieved / PEAK_HBM_GBS, "traffic": None},
                "eager_torch": {"ms": eager_ms, "speedup": eager_ms / ms}}
        if not args.no_cpu_baseline:
            import numpy as np

            import oracle
            cols = np.arange(0, n, n // 16, dtype=np.int64)
            Wc, Ac, Bc = (t.to("cpu", torch.float64).numpy() for t in (W, A, B))
            t0 = time.perf_counter()
            oracle.dora_norm(Wc, Ac, Bc, 2.0, cols=cols)
            to = time.perf_counter() - t0
            line["cpu_baseline"] = {"value": (len(cols) / n) * nbytes / to / 1e9, "unit": "GB/s",
                                    "cores": oracle.num_threads(), "kind": "oracle",
                                    "sample": f"{len(cols)} of {n} columns"}
        print(json.dumps(line), flush=True)
        del W, A, B, ws


def pack_report(args):
    """Host packer throughput: 25,600 samples (the largest scheduling run on the
    pages) of four adapters, lognormal lengths (median 900 tokens, sigma 0.75,
    clipped to [128, 4096]), packed into microbatches of 16,384 tokens, then
    every microbatch's segment table.  The oracle's plain first-fit scan is
    timed beside it on a 2,560-sample slice."""
    import math

    import numpy as np

    import lora_fine_tuning_amd as lf

    n, cap, na = 25600, 16384, 4
    rng = np.random.Generator(np.random.PCG64(2002))
    lengths = [int(v) for v in np.clip(np.rint(rng.lognormal(math.log(900.0), 0.75, n)), 128, 4096)]
    adapters = [int(v) for v in rng.integers(0, na, n)]

    import ctypes
    lib = lf.load()
    c_len = (ctypes.c_int32 * n)(*lengths)
    c_ad = (ctypes.c_int32 * n)(*adapters)
    c_mb = (ctypes.c_int32 * n)()
    c_order = (ctypes.c_int32 * n)()
    c_so = (ctypes.c_int64 * (na + 1))()
    c_sa = (ctypes.c_int32 * na)()
    c_cnt, c_nm, c_ns = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)

    def run():  # straight through the C ABI, host arrays marshalled once
        assert lib.lora_pack_greedy(c_len, n, cap, c_mb, ctypes.byref(c_cnt)) == 0
        segs = 0
        for q in range(c_cnt.value):
            assert lib.lora_microbatch_segments(c_len, c_ad, c_mb, n, na, q, c_order, ctypes.byref(c_nm),
                                                c_so, c_sa, ctypes.byref(c_ns)) == 0
            segs += c_ns.value
        return c_cnt.value, segs

    times = []
    for _ in range(5):
        t0 = time.perf_counter()
        count, segs = run()
        times.append(time.perf_counter() - t0)
    t = sorted(times)[len(times) // 2]
    line = {"metric": "greedy packer + segment tables, samples/s (host)", "value": n / t,
            "unit": "samples/s", "ms": t * 1e3, "higher_is_better": True, "data": "synthetic",
            "config": {"workload": "25600 samples, 4 adapters, lognormal median 900 clip [128, 4096], "
                                   "capacity 16384", "microbatches": count, "segments": segs,
                       "mean_fill": sum(lengths) / (count * cap),
                       "lower_bound_microbatches": math.ceil(sum(lengths) / cap)}}
    if not args.no_cpu_baseline:
        from oracle import packing
        sl = lengths[:2560]
        t0 = time.perf_counter()
        packing.pack_ffd(sl, cap)
        to = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": len(sl) / to, "unit": "samples/s", "cores": 1, "kind": "oracle",
                                "sample": "first 2560 samples, packing only"}
    print(json.dumps(line), flush=True)


KERNELS = ("router", "f1_mask_down", "sum_s_partials", "gemm_f2_fwd_lora", "b1_ds_db", "reduce_ds_db",
           "b2_da", "reduce_da", "gemm_b3_bwd_dx")


def config_report(args):
    """Fused fwd+bwd against the frozen layer (ours and torch.matmul) for the
    mixed-adapter workloads (4 adapters r 16, k = n 8192, 16384 packed tokens;
    8 adapters r 8..128 on k 28672 -> n 8192, 8192 tokens), the seven
    projections of a LLaMA-8B-shaped decoder layer, and the rank/token sweep
    (k = n 4096, r 8..128, m 2048..32768).  Same synthetic inputs as the
    parity tests' workloads; per-kernel averages from the library's HIP events."""
    import torch

    import lora_fine_tuning_amd as lf
    from synth import AdapterSpec, Workload, make_tensors_device, workload

    lf.load()
    stream = torch.cuda.current_stream()

    def timed(fn, steps=args.steps, warmup=args.warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def kernels(fn):
        lf.lora_profiling_enable(True, capacity=8192)
        lf.lora_profiling_reset()
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        out = {}
        for nm in KERNELS:
            c, t = lf.lora_profiling_query(nm)
            if c:
                out[nm] = round(t / c * 1e3, 1)
        lf.lora_profiling_enable(False)
        return out

    def report(w, fused):
        t = tensors[w.name]
        X, W, dY = t["X"], t["W"], t["dY"]
        Yf = torch.empty(w.m, w.n, device="cuda", dtype=torch.bfloat16)
        dXf = torch.empty_like(X)
        Wt = W.t().contiguous()

        def ours():
            lf.lora_frozen_fwd(X, W, Y=Yf, stream=stream)
            lf.lora_frozen_bwd(dY, W, dX=dXf, stream=stream)

        def tor():
            torch.matmul(X, W, out=Yf)
            torch.matmul(dY, Wt, out=dXf)

        f, o, tt = timed(fused), timed(ours), timed(tor)
        print(json.dumps({"workload": w.name, "m": w.m, "k": w.k, "n": w.n,
                          "ranks": [a.r for a in w.adapters],
                          "segments": 0 if w.seg_off is None else len(w.seg_off) - 1,
                          "fused_ms": round(f, 4), "frozen_ours_ms": round(o, 4),
                          "frozen_torch_ms": round(tt, 4), "fused_over_frozen": round(f / min(o, tt), 4),
                          "kernel_us": kernels(fused)}), flush=True)

    tensors = {}
    for cid in (2, 4):
        w = workload(cid)
        t = tensors[w.name] = make_tensors_device(w, "cuda")
        As, Bs = t["A"], t["B"]
        dAs = [torch.empty_like(a) for a in As]
        dBs = [torch.empty_like(b) for b in Bs]
        table = lf.adapter_table(As, Bs, [a.alpha for a in w.adapters], [a.p for a in w.adapters], dAs, dBs)
        so = torch.as_tensor(w.seg_off).cuda()
        sa = torch.as_tensor(w.seg_adapter).cuda()

        def fused(t=t, table=table, so=so, sa=sa, w=w):
            Y, S, keep = lf.multi_lora_linear_fwd(t["X"], t["W"], table, len(t["A"]), so, sa, w.r_max, 0, 0,
                                                  stream=stream)
            lf.multi_lora_linear_bwd(t["dY"], t["X"], t["W"], table, len(t["A"]), so, sa, S, keep, w.r_max,
                                     stream=stream)
        report(w, fused)
        del tensors[w.name]
        torch.cuda.empty_cache()
    # the seven LoRA projections of one LLaMA-8B-shaped decoder layer (q, k, v, o,
    # gate, up, down; m 8192, r 16; synthetic weights, no attention), run back to
    # back as one step
    proj = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
            ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
    layer = []
    for vi, (nm, kk, nn) in enumerate(proj):
        wl = Workload(f"{nm} m8192 k{kk} n{nn} r16", 1, 10 + vi, 8192, kk, nn, [AdapterSpec(16, 2.0, 0.1)])
        layer.append(make_tensors_device(wl, "cuda"))

    def layer_fused():
        for t in layer:
            Y, S, keep = lf.lora_linear_fwd(t["X"], t["W"], t["A"][0], t["B"][0], 2.0, 0.1, 0, 0, stream=stream)
            lf.lora_linear_bwd(t["dY"], t["X"], t["W"], t["A"][0], t["B"][0], S, keep, 2.0, 0.1, stream=stream)

    outs = [(torch.empty(t["X"].shape[0], t["W"].shape[1], device="cuda", dtype=torch.bfloat16),
             torch.empty_like(t["X"]), t["W"].t().contiguous()) for t in layer]

    def layer_ours():
        for t, (yf, dxf, _) in zip(layer, outs):
            lf.lora_frozen_fwd(t["X"], t["W"], Y=yf, stream=stream)
            lf.lora_frozen_bwd(t["dY"], t["W"], dX=dxf, stream=stream)

    def layer_torch():
        for t, (yf, dxf, wt) in zip(layer, outs):
            torch.matmul(t["X"], t["W"], out=yf)
            torch.matmul(t["dY"], wt, out=dxf)

    f, o, tt = timed(layer_fused), timed(layer_ours), timed(layer_torch)
    print(json.dumps({"workload": "llama8b-layer q k v o gate up down, m 8192, r 16", "m": 8192,
                      "projections": [f"{nm} {kk}->{nn}" for nm, kk, nn in proj],
                      "fused_ms": round(f, 4), "frozen_ours_ms": round(o, 4), "frozen_torch_ms": round(tt, 4),
                      "fused_over_frozen": round(f / min(o, tt), 4), "kernel_us": kernels(layer_fused)}),
          flush=True)
    del layer, outs
    torch.cuda.empty_cache()
    for m in (2048, 8192, 32768):
        for r in (8, 16, 32, 64, 128):
            w = workload(3, m=m, r=r)
            t = tensors[w.name] = make_tensors_device(w, "cuda")
            ad = w.adapters[0]

            def fused(t=t, ad=ad):
                Y, S, keep = lf.lora_linear_fwd(t["X"], t["W"], t["A"][0], t["B"][0], ad.alpha, ad.p, 0, 0,
                                                stream=stream)
                lf.lora_linear_bwd(t["dY"], t["X"], t["W"], t["A"][0], t["B"][0], S, keep, ad.alpha, ad.p,
                                   stream=stream)
            report(w, fused)
            del tensors[w.name]
            torch.cuda.empty_cache()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_llama8b_m8192_hbm_traffic.md")


def source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm_kernels.hip", "device_common.hpp"):
        with open(os.path.join(ROOT, "lora_fine_tuning_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if
    it was taken on the current GEMM source; else None."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    digest, vals = None, {}
    for ln in lines:
        ln = ln.strip().strip("`")
        if ln.startswith("source_digest:"):
            digest = ln.split(":", 1)[1].strip()
        elif ln.startswith("traffic_bytes_per_launch["):
            name = ln[len("traffic_bytes_per_launch["):ln.index("]")]
            vals[name] = float(ln.split(":", 1)[1])
    if digest != source_digest():
        return None
    return vals.get(kernel)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding over several GPUs is described, not implemented", file=sys.stderr)
        sys.exit(2)
    if args.pack:
        pack_report(args)
        return

    import torch

    import lora_fine_tuning_amd as lf
    from synth import AdapterSpec, Workload, make_tensors_device

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.configs:
        config_report(args)
        return
    if args.dora:
        dora_report(args)
        return
    if args.concat:
        concat_report(args)
        return
    lf.load()
    dev = "cuda"
    m, k, r, alpha, p = args.m, 4096, args.r, 2.0, 0.1
    ns = [int(v) for v in args.shapes.split(",")]

    shapes = []
    for vi, n in enumerate(ns):
        w = Workload(f"m{m} k{k} n{n}", 1, vi, m, k, n, [AdapterSpec(r, alpha, p)])
        t = make_tensors_device(w, dev)
        X, W, A, B, dY = t["X"], t["W"], t["A"][0], t["B"][0], t["dY"]
        st = {
            "n": n, "X": X, "W": W, "A": A, "B": B, "dY": dY,
            "Y": torch.empty((m, n), dtype=torch.bfloat16, device=dev),
            "S": torch.empty((m, r), dtype=torch.float32, device=dev),
            "keep": torch.empty((m, (k + 31) // 32), dtype=torch.int32, device=dev),
            "dX": torch.empty((m, k), dtype=torch.bfloat16, device=dev),
            "dA": torch.empty((k, r), dtype=torch.bfloat16, device=dev),
            "dB": torch.empty((r, n), dtype=torch.bfloat16, device=dev),
            "wsf": torch.empty(max(1, lf.lora_linear_fwd_workspace_size(m, k, n, r)),
                               dtype=torch.uint8, device=dev),
            "wsb": torch.empty(max(1, lf.lora_linear_bwd_workspace_size(m, k, n, r)),
                               dtype=torch.uint8, device=dev),
        }
        shapes.append(st)
    stream = torch.cuda.current_stream()

    def step():
        for st in shapes:
            lf.lora_linear_fwd(st["X"], st["W"], st["A"], st["B"], alpha, p, 0, 0, Y=st["Y"],
                               S=st["S"], keep_bits=st["keep"], workspace=st["wsf"], stream=stream)
            lf.lora_linear_bwd(st["dY"], st["X"], st["W"], st["A"], st["B"], st["S"], st["keep"],
                               alpha, p, dX=st["dX"], dA=st["dA"], dB=st["dB"],
                               workspace=st["wsb"], stream=stream)

    def frozen_step(kind):
        for st in shapes:
            if kind == "ours":
                lf.lora_frozen_fwd(st["X"], st["W"], Y=st["Y"], stream=stream)
                lf.lora_frozen_bwd(st["dY"], st["W"], dX=st["dX"], stream=stream)
            else:
                torch.matmul(st["X"], st["W"], out=st["Y"])
                torch.matmul(st["dY"], st["W"].t(), out=st["dX"])

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # The unfused comparator: the eager PyTorch LoRA layer (dropout, three
    # matmuls, scale, add; backward by autograd), bf16, same shapes.  Its mask
    # comes from torch's own generator; only its time and bytes are used.
    unfused = []
    for st in shapes:
        ua = st["A"].detach().clone().requires_grad_(True)
        ub = st["B"].detach().clone().requires_grad_(True)
        unfused.append((st, ua, ub))

    def unfused_step():
        for st, ua, ub in unfused:
            ua.grad = None
            ub.grad = None
            xg = st["X"].detach().requires_grad_(True)
            xd = torch.nn.functional.dropout(xg, p=p, training=True)
            y = xg @ st["W"] + alpha * ((xd @ ua) @ ub)
            y.backward(st["dY"])

    def copy_calibration():
        # ends a counter run with device copies of known size (byte-counter scale)
        if not args.copy_calib_mib:
            return
        nel = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {args.copy_calib_mib} MiB read + written per copy, 3 copies",
              file=sys.stderr, flush=True)

    if args.unfused_only:
        ms_u = timed(unfused_step, args.steps, args.warmup)
        copy_calibration()
        print(json.dumps({"unfused_torch_ms": round(ms_u, 4), "steps": args.steps, "warmup": args.warmup}))
        return

    print(f"[bench] warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    ms = timed(step, args.steps, args.warmup)
    print(f"[bench] fused fwd+bwd {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # per-kernel HIP events on the launch stream, over a second timed region
    lf.lora_profiling_enable(True, capacity=64 * args.steps + 64)
    lf.lora_profiling_reset()
    ms_prof = timed(step, args.steps, 0)
    kernels = {}
    for name in ("f1_mask_down", "sum_s_partials", "gemm_f2_fwd_lora", "b1_ds_db", "sum_ds_partials",
                 "reduce_db", "reduce_ds_db", "b2_da", "reduce_da", "gemm_b3_bwd_dx"):
        cnt, tot = lf.lora_profiling_query(name)
        kernels[name] = {"launches": cnt, "total_ms": tot,
                         "avg_us": (tot / cnt * 1e3) if cnt else None}
    lf.lora_profiling_enable(False)

    ms_frozen_ours = timed(lambda: frozen_step("ours"), args.steps, args.warmup)
    ms_frozen_torch = timed(lambda: frozen_step("torch"), args.steps, args.warmup)
    print(f"[bench] frozen ours {ms_frozen_ours:.3f} ms, torch {ms_frozen_torch:.3f} ms",
          file=sys.stderr, flush=True)
    ms_unfused = timed(unfused_step, args.steps, args.warmup)
    print(f"[bench] unfused torch LoRA {ms_unfused:.3f} ms", file=sys.stderr, flush=True)

    # algorithmic FLOPs per launch (both shapes): F2 2mkn + 2mrn; B3 2mnk + 2mrk
    flops = {
        "gemm_f2_fwd_lora": sum(2.0 * m * k * st["n"] + 2.0 * m * r * st["n"] for st in shapes),
        "gemm_b3_bwd_dx": sum(2.0 * m * st["n"] * k + 2.0 * m * r * k for st in shapes),
    }
    dom = max(flops, key=lambda nm: kernels[nm]["total_ms"])
    kd = kernels[dom]
    achieved = flops[dom] / (kd["total_ms"] / args.steps * 1e-3) / 1e12  # TFLOP/s
    traffic = committed_traffic(dom)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else round(traffic)}
    # HBM-bound kernels: algorithmic bytes per launch (both shapes) / event time
    kw = (k + 31) // 32
    hbm_bytes = {
        "f1_mask_down": sum(m * k * 2 + m * kw * 4 + m * r * 4 + k * r * 2 for _ in shapes),
        "b1_ds_db": sum(m * st["n"] * 2 + 2 * m * r * 4 + 2 * r * st["n"] * 2 for st in shapes),
        "b2_da": sum(m * k * 2 + m * kw * 4 + m * r * 4 + k * r * 2 for _ in shapes),
    }
    hbm = {}
    for nm, b in hbm_bytes.items():
        t = kernels[nm]["total_ms"] / args.steps * 1e-3
        hbm[nm] = {"GB/s": round(b / t / 1e9, 1), "frac": round(b / t / 1e9 / PEAK_HBM_GBS, 4)}

    tokens_per_s = m / (ms * 1e-3)
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"LoRA linear fwd+bwd, m={m} tokens through k={k}->n="
                               f"{'+'.join(str(n) for n in ns)} (r={r}, alpha={alpha}, p={p})",
                   "m": m, "k": k, "n": ns, "r": r, "alpha": alpha, "p": p},
        "roofline": roofline,
        "frozen": {"ours_ms": round(ms_frozen_ours, 4), "torch_matmul_ms": round(ms_frozen_torch, 4),
                   "fused_over_frozen": round(ms / min(ms_frozen_ours, ms_frozen_torch), 4)},
        "unfused_torch": {"ms": round(ms_unfused, 4), "fused_speedup": round(ms_unfused / ms, 4)},
        "kernels": {nm: {kk: (round(v, 3) if isinstance(v, float) else v) for kk, v in d.items()}
                    for nm, d in kernels.items()},
        "ms_per_step_with_kernel_events": round(ms_prof, 4),
        "hbm_kernels": hbm,
        "gemm_source_digest": source_digest(),
    }
    copy_calibration()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(m, k, ns, r, alpha, p, args.cpu_rows)
    print(json.dumps(result), flush=True)


def cpu_baseline(m, k, ns, r, alpha, p, rows):
    """The oracle (fp64 C, OpenMP) timed on `rows` tokens of the same workload:
    forward and backward of both projections for those rows; the per-adapter
    reductions run over the sampled rows only."""
    import numpy as np
    import torch

    import oracle
    from synth import AdapterSpec, Workload, make_tensors

    oracle.build(force=False)
    total = 0.0
    for vi, n in enumerate(ns):
        w = Workload(f"m{rows} k{k} n{n}", 1, vi, rows, k, n, [AdapterSpec(r, alpha, p)])
        t = make_tensors(w)
        X, W, A, B, dY = (np.ascontiguousarray(v.to(torch.float64).numpy())
                          for v in (t["X"], t["W"], t["A"][0], t["B"][0], t["dY"]))
        t0 = time.perf_counter()
        oracle.lora_fwd(X, W, A, B, alpha, np.float32(p), 0, 0)
        oracle.lora_bwd(dY, X, W, A, B, alpha, np.float32(p), 0, 0)
        total += time.perf_counter() - t0
    return {"value": round(rows / total, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{rows} of {m} tokens, fwd+bwd of both projections (fp64 C oracle; "
                      f"{total:.1f} s)"}


if __name__ == "__main__":
    main()
