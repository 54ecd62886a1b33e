#!/usr/bin/env python3
"""Benchmark of the LoRA linear layer (forward + backward) on one MI355X.

A step is one forward and one backward pass of the mixed-adapter LoRA linear
layer on the 70B MLP down_proj shape (m = 8192 tokens, k = 28672 -> n = 8192,
8 adapters of ranks 8, 16, 16, 32, 32, 64, 64, 128 over 8 Dirichlet(1)
segments, alpha 2, p 0.1), inputs already resident in HBM.  Every step runs
the whole path: router, dropout mask and down-projection, base GEMM with the
fused LoRA epilogue, dS/dB, dA, and the input-gradient GEMM with the fused
masked LoRA term.  Each step is timed by its own HIP events with the caches
flushed before it; the reported time is the median.

Prints one JSON line: tokens/s (m / median step time), the roofline of the
dominant kernel (algorithmic FLOPs per launch / its average launch time from
HIP events on the launch stream), the frozen layer (this library's GEMM and
torch.matmul, the faster of W^T as a view and as a contiguous copy) for the
slowdown ratio, the LLaMA-8B projections and the small
workload as extra keys, and the CPU oracle timed on a row sample.
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="rows (tokens) of the headline workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shapes", default="4096,14336", help="--concat: n of each projection (k = 4096)")
    ap.add_argument("--m", type=int, default=8192, help="--concat: tokens")
    ap.add_argument("--r", type=int, default=16, help="--concat: rank")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB (byte-counter calibration)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload (no other workloads; for counter runs)")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the headline step: the mixed-adapter workloads and the rank/token "
                         "sweep, fused vs frozen, one JSON line per case")
    ap.add_argument("--pack", action="store_true",
                    help="instead of the headline step: the host packer (greedy token-capacity "
                         "packing and segment tables) on a synthetic global batch; no GPU")
    ap.add_argument("--dora", action="store_true",
                    help="instead of the headline step: the DoRA norm of W + alpha A B per output "
                         "feature at 8192 x 8192, ranks 16, 64 and 256 (one JSON line each)")
    ap.add_argument("--hbm", action="store_true",
                    help="instead of the headline step: the practical HBM ceiling of this part (a 2 GiB "
                         "device copy and a 4 GiB read-only reduction, median of flushed trials)")
    ap.add_argument("--concat", action="store_true",
                    help="instead of the headline step: the forward at p = 0, concatenated [W | A] "
                         "(one GEMM launch) against the split path and the frozen GEMM")
    return ap.parse_args()


def concat_report(args):
    """The forward at p = 0, three ways, on the projection shapes (median of
    cache-flushed event-timed trials):
    * concatenated: lora_linear_fwd_concat, one GEMM launch in which every
      256 x 256 tile also forms the 256 x r block of S = X A its rows need
      (A's rows ride along with W's in the K loop) and adds alpha S B in its
      epilogue -- no separate pass over X, no second pass over Y;
    * split: lora_linear_fwd at p = 0, the pass over X that forms S, then the
      GEMM with alpha S B in its epilogue;
    * from parts (context): the frozen GEMM on the k x (n + r) weight [W | A]
      gives S as r extra output columns, then torch.addmm adds alpha S B in a
      second pass over Y.
    Beside them, the frozen GEMM X W alone."""
    import torch

    import lora_fine_tuning_amd as lf

    lf.load()
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    m, k, r, alpha = args.m, 4096, args.r, 2.0
    g = torch.Generator(device="cuda").manual_seed(3)

    def med(fn):
        return timer.median(fn, args.steps, args.warmup)

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
        concat = med(lambda: lf.lora_linear_fwd_concat(X, W, A, B, alpha, Y=Y, S=S, stream=stream))
        split = med(lambda: lf.lora_linear_fwd(X, W, A, B, alpha, 0.0, Y=Y, S=S, workspace=ws, stream=stream))
        gemm = med(lambda: lf.lora_frozen_fwd(X, W, Y=Y, stream=stream))
        parts = med(lambda: (lf.lora_frozen_fwd(X, Wc, Y=Yc, stream=stream), Y.addmm_(Sb, B, alpha=alpha)))
        print(json.dumps({"metric": "forward ms at p = 0: concatenated [W | A] vs split (pass over X, then GEMM)",
                          "config": {"workload": f"m {m} k {k} n {n} r {r}"},
                          "concat_fwd_ms": round(concat, 4), "split_fwd_ms": round(split, 4),
                          "frozen_gemm_ms": round(gemm, 4), "from_parts_ms": round(parts, 4),
                          "concat_over_split": round(concat / split, 4),
                          "concat_over_frozen": round(concat / gemm, 4)}), flush=True)
        del X, W, A, B, Wc, Y, Yc, S, ws, Sb


def hbm_report(args):
    """What a plain streaming kernel reaches on this part, for the HBM-bound
    kernels' fractions: a device-to-device copy of 2 GiB (bytes read + bytes
    written per second) and torch.sum over 4 GiB of fp32 (bytes read per
    second), median of cache-flushed event-timed trials."""
    import torch

    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    n = (2 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    copy_ms = timer.median(lambda: b.copy_(a), args.steps, args.warmup)
    del a, b
    x = torch.ones((4 << 30) // 4, dtype=torch.float32, device="cuda")
    sum_ms = timer.median(lambda: x.sum(), args.steps, args.warmup)
    del x
    copy_gbs = 2 * (2 << 30) / (copy_ms * 1e-3) / 1e9
    read_gbs = (4 << 30) / (sum_ms * 1e-3) / 1e9
    print(json.dumps({"metric": "practical HBM bandwidth (plain streaming kernels)",
                      "copy_2GiB": {"ms": round(copy_ms, 4), "GB/s": round(copy_gbs, 1),
                                    "frac_of_8TBs": round(copy_gbs / PEAK_HBM_GBS, 4)},
                      "sum_read_4GiB": {"ms": round(sum_ms, 4), "GB/s": round(read_gbs, 1),
                                        "frac_of_8TBs": round(read_gbs / PEAK_HBM_GBS, 4)}}), flush=True)


def copy_calibration(torch, args):
    """Ends a counter run with device copies of known size (--copy-calib-mib),
    the scale for the byte counters."""
    if not args.copy_calib_mib:
        return
    nel = args.copy_calib_mib * (1 << 20) // 4
    src = torch.ones(nel, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {args.copy_calib_mib} MiB read + written per copy, 3 copies",
          file=sys.stderr, flush=True)
    del src, dst


def dora_report(args):
    """DoRA norm on the page's 8192 x 8192 weight shape.  One pass over W is the
    compulsory traffic (bytes = 2kn + 2kr + 2rn + 4n per call); the kernel is
    reported against HBM, timed as the median of flushed event-timed trials.
    Beside it: the eager PyTorch form that builds the
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

        # median of flushed event-timed trials (W, A and B come from HBM each
        # time, not from the Infinity Cache, which would hold a 128 MiB W)
        timer = Timer(torch, torch.cuda.current_stream())
        ms = timer.median(fused, args.steps, args.warmup)
        ms_b2b = sum(timer.trials(fused, args.steps, 0, flush=False)) / args.steps
        # the pass over W alone: HIP events the library records on its launch
        # stream, over flushed trials
        lf.lora_profiling_enable(True, capacity=4 * args.steps + 16)
        lf.lora_profiling_reset()
        timer.trials(fused, args.steps, 0)
        c, tot = lf.lora_profiling_query("dora_norm_pass")
        kern_ms = tot / max(c, 1)
        lf.lora_profiling_enable(False)
        eager_ms = timer.median(eager, 5, 2)
        nbytes = 2 * k * n + 2 * k * r + 2 * r * n + 4 * n
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        line = {"metric": "DoRA norm of W + alpha A B per output feature, GB/s of compulsory traffic",
                "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms": ms, "steps": args.steps,
                "warmup": args.warmup, "higher_is_better": True, "dtype": "bf16 in, fp32 sums",
                "data": "synthetic", "config": {"workload": f"W {k} x {n}, r {r}"},
                "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": achieved / PEAK_HBM_GBS, "traffic": None},
                "timing": "median of event-timed trials, 512 MiB read between trials (cache flush)",
                "ms_back_to_back": ms_b2b,
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
    parity tests' workloads.  Times are medians of cache-flushed event-timed
    trials (Timer); torch.matmul counts as the faster of W^T as a view and as a
    contiguous copy; per-kernel averages come from the library's HIP events over
    three back-to-back calls."""
    import torch

    import lora_fine_tuning_amd as lf
    from synth import DECODER_PROJECTIONS, decoder_projection, make_tensors_device, workload

    lf.load()
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)

    def timed(fn, steps=args.steps, warmup=args.warmup):
        return timer.median(fn, steps, warmup)

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

        # torch.matmul with W^T as a view and as a contiguous copy; the faster counts
        def tor_view():
            torch.matmul(X, W, out=Yf)
            torch.matmul(dY, W.t(), out=dXf)

        def tor_copy():
            torch.matmul(X, W, out=Yf)
            torch.matmul(dY, Wt, out=dXf)

        f, o = timed(fused), timed(ours)
        tt = min(timed(tor_view), timed(tor_copy))
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
    proj = DECODER_PROJECTIONS
    layer = [make_tensors_device(decoder_projection(vi), "cuda") for vi in range(len(proj))]

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

    def layer_torch_copy():
        for t, (yf, dxf, wt) in zip(layer, outs):
            torch.matmul(t["X"], t["W"], out=yf)
            torch.matmul(t["dY"], wt, out=dxf)

    def layer_torch_view():
        for t, (yf, dxf, _) in zip(layer, outs):
            torch.matmul(t["X"], t["W"], out=yf)
            torch.matmul(t["dY"], t["W"].t(), out=dxf)

    f, o = timed(layer_fused), timed(layer_ours)
    tt = min(timed(layer_torch_view), timed(layer_torch_copy))
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


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_b3_70b_downproj_m8192_hbm_traffic.md")


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


class Timer:
    """Per-step HIP-event timing on one stream.  Each trial is bracketed by its
    own event pair; between trials (outside the events) a 512 MiB scratch
    buffer is read, which evicts the 256 MB Infinity Cache and the L2s, so
    every trial starts from HBM (median of event-timed trials with the caches
    flushed, the timing method of the Scaling DoRA page, "reproduction and
    evaluation").  The flush reads rather than writes: a written buffer would
    leave up to 256 MB of dirty lines whose write-back lands inside the next
    trial (it doubled a 30 us DoRA call and added about 38 us to the 70B
    batch's first kernel), while reading also writes the previous trial's dirty
    outputs back before the events start."""

    FLUSH_BYTES = 512 << 20

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self.scratch = torch.ones(self.FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = None

    def flush(self):
        self.sink = self.scratch.sum()

    def trials(self, fn, steps, warmup, flush=True):
        torch = self.torch
        for _ in range(warmup):
            if flush:
                self.flush()
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in ev:
            if flush:
                self.flush()
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in ev]

    def median(self, fn, steps, warmup, flush=True):
        t = sorted(self.trials(fn, steps, warmup, flush))
        return t[len(t) // 2]


def mixed_case(lf, torch, w, stream):
    """Device tensors, the adapter table and preallocated outputs of a
    mixed-adapter workload; returns (fused step, frozen steps, per-row ranks)."""
    from synth import make_tensors_device
    import numpy as np

    t = make_tensors_device(w, "cuda")
    X, W, dY, As, Bs = t["X"], t["W"], t["dY"], t["A"], t["B"]
    dAs = [torch.empty_like(a) for a in As]
    dBs = [torch.empty_like(b) for b in Bs]
    alphas = [a.alpha for a in w.adapters]
    ps = [a.p for a in w.adapters]
    table = lf.adapter_table(As, Bs, alphas, ps, dAs, dBs)
    so = torch.as_tensor(w.seg_off).cuda()
    sa = torch.as_tensor(w.seg_adapter).cuda()
    m, k, n, rm, na, ns = w.m, w.k, w.n, w.r_max, len(As), len(w.seg_adapter)
    Y = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    S = torch.empty(m, rm, dtype=torch.float32, device="cuda")
    keep = torch.empty(m, (k + 31) // 32, dtype=torch.int32, device="cuda")
    dX = torch.empty(m, k, dtype=torch.bfloat16, device="cuda")
    wsf = torch.empty(max(1, lf.multi_lora_fwd_workspace_size(m, k, n, rm, na, ns)), dtype=torch.uint8,
                      device="cuda")
    wsb = torch.empty(max(1, lf.multi_lora_bwd_workspace_size(m, k, n, rm, na, ns)), dtype=torch.uint8,
                      device="cuda")

    def step():
        lf.multi_lora_linear_fwd(X, W, table, na, so, sa, rm, w.seed, w.offset, Y=Y, S=S, keep_bits=keep,
                                 workspace=wsf, stream=stream)
        lf.multi_lora_linear_bwd(dY, X, W, table, na, so, sa, S, keep, rm, dX=dX, workspace=wsb, stream=stream)

    def frozen_ours():
        lf.lora_frozen_fwd(X, W, Y=Y, stream=stream)
        lf.lora_frozen_bwd(dY, W, dX=dX, stream=stream)

    Wt = W.t().contiguous()

    # torch.matmul with W^T as a view and as a contiguous copy (the caller takes the faster)
    def frozen_torch_view():
        torch.matmul(X, W, out=Y)
        torch.matmul(dY, W.t(), out=dX)

    def frozen_torch_copy():
        torch.matmul(X, W, out=Y)
        torch.matmul(dY, Wt, out=dX)

    frozen_torch = (frozen_torch_view, frozen_torch_copy)
    row_r = np.zeros(m, dtype=np.int64)
    for s in range(ns):
        row_r[w.seg_off[s]:w.seg_off[s + 1]] = w.adapters[int(w.seg_adapter[s])].r
    return step, frozen_ours, frozen_torch, row_r, t


def single_case(lf, torch, m, k, n, r, alpha, p, variant, stream, cid=1):
    from synth import AdapterSpec, Workload, make_tensors_device
    w = Workload(f"m{m} k{k} n{n}", cid, variant, m, k, n, [AdapterSpec(r, alpha, p)])
    t = make_tensors_device(w, "cuda")
    X, W, A, B, dY = t["X"], t["W"], t["A"][0], t["B"][0], t["dY"]
    Y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((m, r), dtype=torch.float32, device="cuda")
    keep = torch.empty((m, (k + 31) // 32), dtype=torch.int32, device="cuda")
    dX = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((k, r), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((r, n), dtype=torch.bfloat16, device="cuda")
    wsf = torch.empty(max(1, lf.lora_linear_fwd_workspace_size(m, k, n, r)), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(1, lf.lora_linear_bwd_workspace_size(m, k, n, r)), dtype=torch.uint8, device="cuda")

    def step():
        lf.lora_linear_fwd(X, W, A, B, alpha, p, 0, 0, Y=Y, S=S, keep_bits=keep, workspace=wsf, stream=stream)
        lf.lora_linear_bwd(dY, X, W, A, B, S, keep, alpha, p, dX=dX, dA=dA, dB=dB, workspace=wsb, stream=stream)

    def frozen_ours():
        lf.lora_frozen_fwd(X, W, Y=Y, stream=stream)
        lf.lora_frozen_bwd(dY, W, dX=dX, stream=stream)

    Wt = W.t().contiguous()

    # torch.matmul with W^T as a view and as a contiguous copy (the caller takes the faster)
    def frozen_torch_view():
        torch.matmul(X, W, out=Y)
        torch.matmul(dY, W.t(), out=dX)

    def frozen_torch_copy():
        torch.matmul(X, W, out=Y)
        torch.matmul(dY, Wt, out=dX)

    frozen_torch = (frozen_torch_view, frozen_torch_copy)

    ua = A.detach().clone().requires_grad_(True)
    ub = B.detach().clone().requires_grad_(True)

    def unfused():
        # the eager PyTorch LoRA layer (dropout, three matmuls, scale, add;
        # backward by autograd); its mask comes from torch's own generator
        ua.grad = None
        ub.grad = None
        xg = X.detach().requires_grad_(True)
        xd = torch.nn.functional.dropout(xg, p=p, training=True)
        y = xg @ W + alpha * ((xd @ ua) @ ub)
        y.backward(dY)

    return step, frozen_ours, frozen_torch, unfused


KERNEL_NAMES = ("router", "f1_mask_down", "sum_s_partials", "gemm_f2_fwd_lora", "b1_ds_db", "reduce_ds_db",
                "b2_da", "reduce_da", "gemm_b3_bwd_dx")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding over several GPUs is described, not implemented", file=sys.stderr)
        sys.exit(2)
    if args.pack:
        pack_report(args)
        return

    import numpy as np
    import torch

    import lora_fine_tuning_amd as lf
    from synth import workload

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.configs:
        config_report(args)
        return
    if args.dora:
        dora_report(args)
        copy_calibration(torch, args)
        return
    if args.hbm:
        hbm_report(args)
        return
    if args.concat:
        concat_report(args)
        return
    lf.load()
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    K, Wm = args.steps, args.warmup

    # ---- the headline: 70B MLP down_proj, 8 adapters of ranks 8..128
    w = workload(4)
    m, k, n = w.m, w.k, w.n
    step, frozen_ours, frozen_torch, row_r, tens = mixed_case(lf, torch, w, stream)
    print(f"[bench] {w.name}: warmup {Wm}, {K} flushed trials", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_all = timer.trials(step, K, Wm)
    ts = sorted(t_all)
    ms = ts[len(ts) // 2]
    print(f"[bench] fused fwd+bwd median {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # per-kernel HIP events on the launch stream over a second, identical timed region
    lf.lora_profiling_enable(True, capacity=64 * K + 64)
    lf.lora_profiling_reset()
    timer.trials(step, K, 0)
    kernels = {}
    for name in KERNEL_NAMES:
        cnt, tot = lf.lora_profiling_query(name)
        kernels[name] = {"launches": cnt, "total_ms": round(tot, 4),
                         "avg_us": round(tot / cnt * 1e3, 2) if cnt else None}
    lf.lora_profiling_enable(False)

    ms_fo = timer.median(frozen_ours, K, Wm)
    ms_ft = min(timer.median(f, K, Wm) for f in frozen_torch)
    ms_b2b = sum(timer.trials(step, K, 0, flush=False)) / K
    print(f"[bench] frozen ours {ms_fo:.3f} ms, torch {ms_ft:.3f} ms", file=sys.stderr, flush=True)

    # algorithmic FLOPs per launch: F2 2mkn + 2n sum_i r_i; B3 2mnk + 2k sum_i r_i
    sr = float(row_r.sum())
    flops = {"gemm_f2_fwd_lora": 2.0 * m * k * n + 2.0 * n * sr,
             "gemm_b3_bwd_dx": 2.0 * m * n * k + 2.0 * k * sr}
    dom = max(flops, key=lambda nm: kernels[nm]["total_ms"])
    achieved = flops[dom] / (kernels[dom]["avg_us"] * 1e-6) / 1e12
    traffic = committed_traffic(dom)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else round(traffic)}
    # HBM-bound kernels: algorithmic bytes per launch (per token 2k + k/8 + 4 r_i for
    # F1 and B2, 2n + 8 r_i for B1; plus each adapter's A, B, dA, dB once) / event time
    kw = (k + 31) // 32
    ra = sum(a.r for a in w.adapters)
    hbm_bytes = {"f1_mask_down": 2.0 * m * k + 4.0 * m * kw + 4.0 * sr + 2.0 * k * ra,
                 "b1_ds_db": 2.0 * m * n + 8.0 * sr + 4.0 * n * ra,
                 "b2_da": 2.0 * m * k + 4.0 * m * kw + 4.0 * sr + 2.0 * k * ra}
    hbm = {}
    for nm, b in hbm_bytes.items():
        if kernels[nm]["avg_us"]:
            gbs = b / (kernels[nm]["avg_us"] * 1e-6) / 1e9
            hbm[nm] = {"GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}

    copy_calibration(torch, args)

    # ---- the LLaMA-8B projections (r 16), each alone and both as one step
    extra = {}
    if not args.headline_only:
        c1 = {}
        for vi, nn in enumerate((4096, 14336)):
            s1, fo1, ft1, un1 = single_case(lf, torch, 8192, 4096, nn, 16, 2.0, 0.1, vi, stream)
            f1 = timer.median(s1, K, Wm)
            o1 = timer.median(fo1, K, Wm)
            t1 = min(timer.median(f, K, Wm) for f in ft1)
            u1 = timer.median(un1, max(K // 4, 5), 2)
            c1[f"k4096_n{nn}"] = {"fused_ms": round(f1, 4), "frozen_ours_ms": round(o1, 4),
                                  "frozen_torch_ms": round(t1, 4), "fused_over_frozen": round(f1 / min(o1, t1), 4),
                                  "unfused_torch_ms": round(u1, 4), "tokens_per_s": round(8192 / (f1 * 1e-3), 1)}
            del s1, fo1, ft1, un1
            torch.cuda.empty_cache()
        both = sum(v["fused_ms"] for v in c1.values())
        both_frozen = sum(min(v["frozen_ours_ms"], v["frozen_torch_ms"]) for v in c1.values())
        c1["both_shapes"] = {"fused_ms": round(both, 4), "fused_over_frozen": round(both / both_frozen, 4),
                             "tokens_per_s": round(8192 / (both * 1e-3), 1)}
        extra["llama8b_projections_m8192_r16"] = c1
        # ---- the small workload (m 512, k = n 1024, r 16): launch- and cache-bound
        s0, fo0, ft0, _ = single_case(lf, torch, 512, 1024, 1024, 16, 2.0, 0.1, 0, stream, cid=0)
        f0, o0 = timer.median(s0, K, Wm), timer.median(fo0, K, Wm)
        t0 = min(timer.median(f, K, Wm) for f in ft0)
        extra["small_m512_k1024_n1024_r16"] = {"fused_ms": round(f0, 4), "tokens_per_s": round(512 / (f0 * 1e-3), 1),
                                               "frozen_ours_ms": round(o0, 4), "frozen_torch_ms": round(t0, 4),
                                               "fused_over_frozen": round(f0 / min(o0, t0), 4)}
    print(f"[bench] other workloads done", file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": round(m / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"70B MLP down_proj LoRA linear fwd+bwd: m={m} tokens, k={k} -> n={n}, "
                               f"8 adapters r={[a.r for a in w.adapters]} in 8 Dirichlet(1) segments "
                               f"{np.diff(w.seg_off).tolist()}, alpha=2, p=0.1",
                   "m": m, "k": k, "n": n, "ranks": [a.r for a in w.adapters],
                   "segments": w.seg_off.tolist(), "timing": "median of per-step HIP-event trials, "
                   "512 MiB read between trials (cache flush)"},
        "ms_per_step_mean": round(sum(t_all) / K, 4),
        "ms_per_step_min": round(ts[0], 4),
        "ms_per_step_back_to_back": round(ms_b2b, 4),
        "roofline": roofline,
        "frozen": {"ours_ms": round(ms_fo, 4), "torch_matmul_ms": round(ms_ft, 4),
                   "fused_over_frozen": round(ms / min(ms_fo, ms_ft), 4)},
        "kernels": kernels,
        "hbm_kernels": hbm,
        "other_workloads": extra,
        "gemm_source_digest": source_digest(),
    }
    del step, frozen_ours, frozen_torch
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, tens, args.cpu_rows)
    print(json.dumps(result), flush=True)


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, tens, rows):
    """The oracle (double-precision C, OpenMP over rows, built as it stands)
    timed on a row sample of the same workload: the first rows/8 rows of each
    of the 8 segments, forward and backward of their adapters (mask, S, Y; dS,
    dB, dA, dX), on up to one host thread per sampled row of a segment, then
    on one thread for a smaller sample."""
    import ctypes

    import numpy as np
    import torch

    import oracle

    oracle.build(force=False)
    per = max(1, rows // len(w.seg_adapter))
    idx, so, sa = [], [0], []
    for s in range(len(w.seg_adapter)):
        lo, hi = int(w.seg_off[s]), int(w.seg_off[s + 1])
        take = list(range(lo, min(hi, lo + per)))
        idx += take
        so.append(so[-1] + len(take))
        sa.append(int(w.seg_adapter[s]))
    ii = torch.as_tensor(idx, device="cuda")
    to64 = lambda t: np.ascontiguousarray(t.to("cpu", torch.float64).numpy())  # noqa: E731
    X, dY, W = to64(tens["X"][ii]), to64(tens["dY"][ii]), to64(tens["W"])
    ads = [{"A": to64(a), "B": to64(b), "alpha": ad.alpha, "p": np.float32(ad.p)}
           for a, b, ad in zip(tens["A"], tens["B"], w.adapters)]

    def run(nrows_per_seg):
        so2, sa2, sel = [0], [], []
        for s in range(len(sa)):
            take = list(range(so[s], min(so[s + 1], so[s] + nrows_per_seg)))
            sel += take
            so2.append(so2[-1] + len(take))
            sa2.append(sa[s])
        Xs, dYs = np.ascontiguousarray(X[sel]), np.ascontiguousarray(dY[sel])
        t0 = time.perf_counter()
        oracle.multi_lora_fwd(Xs, W, ads, so2, sa2, w.r_max, 0, 0)
        oracle.multi_lora_bwd(dYs, Xs, W, ads, so2, sa2, w.r_max, 0, 0)
        return len(sel), time.perf_counter() - t0

    n_all, t_all = run(per)
    threads = oracle.num_threads()
    one = None
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        n1, t1 = run(max(1, per // 32))
        gomp.omp_set_num_threads(threads)
        one = {"value": round(n1 / t1, 3), "rows": n1, "seconds": round(t1, 2)}
    except OSError:
        pass
    # the oracle parallelises over the rows of one segment at a time
    return {"value": round(n_all / t_all, 3), "unit": "tokens/s", "cores": min(threads, per), "kind": "oracle",
            "sample": f"{n_all} of {w.m} tokens ({per} from each of the 8 segments), forward and backward, "
                      f"double-precision C oracle, {t_all:.1f} s",
            "cpu_model": cpu_model(), "single_thread": one}


if __name__ == "__main__":
    main()
