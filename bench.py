#!/usr/bin/env python3
"""Benchmark of the sketch hot path on one MI355X.

Headline step (the largest single-GPU workload, mlp_70b_prefill): sketch-
encode the 28672x8192 bfloat16 weight (Student-t(4), std 0.015, importance
U(0.5, 1.5), 0.5 bits per weight, row blocks of 16) and run the 2048-token
prefill product Y = X W_hat^T (bf16 matrix cores, float32 accumulation).  The
weight (470 MB) is larger than the 256 MB last-level cache, so every encode
streams it from HBM.  `value` = weights per second of whole steps (M*N / step
time); the roofline object is the dominant kernel of the step, the prefill
GEMM, against the 2.5 PFLOP/s dense bf16 peak.

Breakdown (every workload the benchmark specification names):
  encode      Mw/s and %HBM on the attention, MLP-up (0.5 and 0.75 bpw),
              decoder-layer and 70B MLP weights;
  gemv        decode products: attention batch 1, MLP-up at 0.5/0.75 bpw and
              batches 1/4/16 (single calls: latency-bound), the 7-linear
              decoder layer over 256 fresh-x token steps (tables cache-
              resident), and the same layer as 32 distinct copies (405 MB of
              tables, beyond the last-level cache: the HBM-bound figure);
  gemm        the prefill GEMM alone;
  decode, multi_row_2, allocated, q4: materialised W_hat and the sketch
              variants on the attention weight.
Parity of the headline tables and outputs against the CPU oracle, and the
oracle's own time on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-breakdown] [--no-ext] [--no-cpu-baseline]
    python bench.py --profile-kernels     # short eager run of every hot kernel, for rocprofv3
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "decode-GEMV eff. weights/s & % HBM roofline; GEMM % MFMA peak; encode Mw/s"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-breakdown", action="store_true", help="headline step only")
    ap.add_argument("--no-ext", action="store_true", help="skip the multi-row, allocation and 4-bit figures")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline sample budget")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="short eager run of every hot kernel plus a 256 MiB copy, for rocprofv3 "
                         "(kernel trace or counters); prints no JSON")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {"encode_kernel": ("encode.hip", "common.h"), "gemv_mfma_kernel": ("gemv.hip", "common.h"),
                  "gemm_tile_kernel": ("gemm.hip", "common.h"), "decode_map_kernel": ("decode.hip", "common.h"),
                  "rows_gemm_kernel": ("rows.hip", "common.h"), "rows_gemv_kernel": ("rows.hip", "common.h"),
                  "alloc_gemm_kernel": ("alloc.hip", "common.h"), "alloc_gemv_kernel": ("alloc.hip", "common.h"),
                  "block_importance_kernel": ("alloc.hip", "common.h"),
                  "alloc_decode_kernel": ("alloc.hip", "common.h"),
                  "q4_gemm_kernel": ("q4.hip", "common.h"), "q4_gemv_kernel": ("q4.hip", "common.h"),
                  "q4_decode_kernel": ("q4.hip", "common.h")}


def kernel_source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sub_bit_weight_sketch_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch (reads + writes, counter-calibrated) from the
    committed rocprofv3 counter summary, or None when it is missing or was
    taken on other kernel sources."""
    try:
        with open(os.path.join(PROFILES, "traffic.json")) as fh:
            rec = json.load(fh).get("%s@%s" % (kernel, workload))
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != kernel_source_digest(kernel):
        return None
    return rec["bytes_per_launch"]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gpu_student_t_bf16(torch, M, N, std, gen, device, rows_per_chunk=2048):
    """Student-t(4) via normal / sqrt(chi2_4 / 4), scaled to std, rounded to bf16 (on the GPU)."""
    out = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    scale = std / math.sqrt(2.0)
    for r0 in range(0, M, rows_per_chunk):
        r1 = min(M, r0 + rows_per_chunk)
        z = torch.randn((r1 - r0, N), generator=gen, device=device)
        c = torch.zeros_like(z)
        for _ in range(4):
            c.add_(torch.randn((r1 - r0, N), generator=gen, device=device).square_())
        out[r0:r1] = (z * torch.rsqrt(c * 0.25) * scale).to(torch.bfloat16)
    return out


class Timer:
    """Average duration of launches on the library's stream: HIP events
    around graph replays of back-to-back launches (host gaps and other
    kernels stay out of the average)."""

    def __init__(self, torch, sk, dev):
        self.torch, self.sk, self.dev = torch, sk, dev
        self.stream = torch.cuda.current_stream(dev)

    def capture(self, fns):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            hs = self.sk._stream_handle(self.dev)
            for fn in fns:
                fn(hs)
        return g

    def graph_avg(self, fns, reps):
        """Average seconds per launch of the list `fns` replayed `reps` times."""
        torch = self.torch
        g = self.capture(fns)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(reps):
            g.replay()
        e1.record(self.stream)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e-3 / (reps * len(fns))

    def eager_avg(self, fn, reps):
        torch = self.torch
        fn(None)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(reps):
            fn(None)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps


def hbm(bytes_, seconds):
    gbs = bytes_ / seconds / 1e9
    return {"algorithmic_bytes": int(bytes_), "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}


def enc_bytes(M, N, tb, es=2):
    """Encode algorithmic bytes: read W and importance, write the tables."""
    return M * N * es + 4 * N + tb


def gemv_bytes(tb, b, N, M):
    """Decode-product algorithmic bytes: read the tables and x, write y (float32)."""
    return tb + b * N * 2 + b * M * 4


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def setup_headline(torch, sk, dev, np):
    import synth
    log("bench: generating mlp_70b_prefill (28672x8192 weight, 2048x8192 activations)")
    lin, X = synth.mlp_70b_prefill()
    W = torch.from_numpy(lin.W.view(np.int16)).to(dev).view(torch.bfloat16)
    imp = torch.from_numpy(lin.imp).to(dev)
    Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
    p = sk.params(lin.M, lin.N, lin.R, lin.bpw, lin.seed, sk.ABSMIN, sk.BF16)
    nb, Bg, tb = sk.sketch_layout(p)
    proj = sk.projection(p, dev)
    T = torch.empty((nb, Bg), dtype=torch.int16, device=dev)
    Y = torch.empty((X.shape[0], lin.M), dtype=torch.float32, device=dev)
    return lin, X, W, imp, Xd, p, proj, T, Y, tb


def encode_copies(torch, sk, dev, gen, M, N, R, bpw, copies, std=0.02):
    """`copies` GPU-generated weights of one shape with their importance,
    params (AbsMin, bf16), projection and table buffers."""
    p = sk.params(M, N, R, bpw, 1, sk.ABSMIN, sk.BF16)
    nb, Bg, tb = sk.sketch_layout(p)
    proj = sk.projection(p, dev)
    Ws = [gpu_student_t_bf16(torch, M, N, std, gen, dev) for _ in range(copies)]
    imps = [torch.rand(N, generator=gen, device=dev) + 0.5 for _ in range(copies)]
    tabs = [torch.empty((nb, Bg), dtype=torch.int16, device=dev) for _ in range(copies)]
    return p, proj, Ws, imps, tabs, tb


def bench_encodes(torch, sk, dev, gen, tm, status, headline):
    """Encode throughput on every weight shape of the specification: enough
    distinct copies rotate that the weights stream from HBM."""
    out = {}
    shapes = [("attn_4096x4096", 4096, 4096, 8, 0.5, 16), ("mlp_up_11008x4096@0.5bpw", 11008, 4096, 8, 0.5, 4),
              ("mlp_up_11008x4096@0.75bpw", 11008, 4096, 8, 0.75, 4)]
    for name, M, N, R, bpw, copies in shapes:
        p, proj, Ws, imps, tabs, tb = encode_copies(torch, sk, dev, gen, M, N, R, bpw, copies)
        fns = [lambda hs, c=c: sk.sketch_encode(p, proj, Ws[c], imps[c], tabs[c], status, hs) for c in range(copies)]
        t = tm.graph_avg(fns, max(2, 32 // copies))
        out[name] = dict({"kernel": "encode_kernel", "avg_us": t * 1e6, "Mw_per_s": M * N / t / 1e6,
                          "weights": M * N, "copies": copies}, **hbm(enc_bytes(M, N, tb), t))
        del Ws, tabs
    # the 7 linears of one decoder layer, encoded back to back (405 MB of weights)
    import synth
    ps, projs, Ws, imps, tabs, tot_w, tot_b = [], [], [], [], [], 0, 0
    for name, M, N in synth.LAYER_7B_SHAPES:
        p, proj, W1, i1, t1, tb = encode_copies(torch, sk, dev, gen, M, N, 8, 0.5, 1)
        ps.append(p), projs.append(proj), Ws.append(W1[0]), imps.append(i1[0]), tabs.append(t1[0])
        tot_w += M * N
        tot_b += enc_bytes(M, N, tb)
    fns = [lambda hs, c=c: sk.sketch_encode(ps[c], projs[c], Ws[c], imps[c], tabs[c], status, hs) for c in range(7)]
    t = tm.graph_avg(fns, 4) * 7
    out["layer_7b"] = dict({"kernel": "encode_kernel", "layer_us": t * 1e6, "Mw_per_s": tot_w / t / 1e6,
                            "weights": tot_w, "note": "the 7 linears of the layer encoded back to back"},
                           **hbm(tot_b, t))
    del Ws, tabs
    lin, W, imp, p, proj, T, tb = headline
    t = tm.graph_avg([lambda hs: sk.sketch_encode(p, proj, W, imp, T, status, hs)], 8)
    out["mlp_70b_prefill"] = dict({"kernel": "encode_kernel", "avg_us": t * 1e6, "Mw_per_s": lin.M * lin.N / t / 1e6,
                                   "weights": lin.M * lin.N,
                                   "traffic": measured_traffic("encode_kernel", "mlp_70b_prefill")},
                                  **hbm(enc_bytes(lin.M, lin.N, tb), t))
    pmax = sk.params(lin.M, lin.N, lin.R, lin.bpw, lin.seed, sk.ABSMAX, sk.BF16)
    T2 = torch.empty_like(T)
    t = tm.graph_avg([lambda hs: sk.sketch_encode(pmax, proj, W, imp, T2, status, hs)], 8)
    out["mlp_70b_prefill_absmax"] = dict({"kernel": "encode_kernel", "avg_us": t * 1e6,
                                          "Mw_per_s": lin.M * lin.N / t / 1e6}, **hbm(enc_bytes(lin.M, lin.N, tb), t))
    torch.cuda.synchronize()
    if int(status.item()):
        raise SystemExit("encode reported flags 0x%x" % int(status.item()))
    return out


def bench_gemvs(torch, sk, dev, gen, tm, status):
    """Decode products of the specification's workloads."""
    import synth
    out = {}
    # attention batch 1 and MLP-up at both bpw and batches 1/4/16: single
    # calls over tables that sit in the cache (1-4 MiB): latency-bound
    for name, M, N, bpw, batches in (("attn_4096x4096", 4096, 4096, 0.5, (1,)),
                                     ("mlp_up_11008x4096@0.5bpw", 11008, 4096, 0.5, (1, 4, 16)),
                                     ("mlp_up_11008x4096@0.75bpw", 11008, 4096, 0.75, (1, 4, 16))):
        p, proj, Ws, imps, tabs, tb = encode_copies(torch, sk, dev, gen, M, N, 8, bpw, 1)
        sk.sketch_encode(p, proj, Ws[0], imps[0], tabs[0], status)
        del Ws
        for b in batches:
            X = torch.randn((b, N), generator=gen, device=dev).to(torch.bfloat16)
            Y = torch.empty((b, M), dtype=torch.float32, device=dev)
            wsb = sk.sketch_workspace_bytes(p, b, sk.BF16)
            ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
            t = tm.graph_avg([lambda hs: sk.sketch_matmul(p, proj, tabs[0], X, Y, ws, hs)] * 16, 8)
            out["%s_b%d" % (name, b)] = dict({"avg_us": t * 1e6, "eff_weights_per_s": M * N / t, "batch": b},
                                             **hbm(gemv_bytes(tb, b, N, M), t))
    # decoder layer: 7 linears, 256 token steps with fresh x per linear
    layer = []
    for name, M, N in synth.LAYER_7B_SHAPES:
        p, proj, Ws, imps, tabs, tb = encode_copies(torch, sk, dev, gen, M, N, 8, 0.5, 1)
        sk.sketch_encode(p, proj, Ws[0], imps[0], tabs[0], status)
        del Ws
        xs = torch.randn((256, N), generator=gen, device=dev).to(torch.bfloat16)
        ys = torch.empty((256, M), dtype=torch.float32, device=dev)
        wsb = sk.sketch_workspace_bytes(p, 1, sk.BF16)
        layer.append((name, M, N, p, proj, tabs[0], xs, ys, torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev),
                      tb))
    step_w = sum(M * N for _, M, N, *_ in layer)
    step_b = sum(gemv_bytes(tb, 1, N, M) for _, M, N, _, _, _, _, _, _, tb in layer)
    fns = []
    for s in range(256):
        for (name, M, N, p, proj, T, xs, ys, ws, tb) in layer:
            fns.append(lambda hs, p=p, proj=proj, T=T, x=xs[s:s + 1], y=ys[s:s + 1], ws=ws:
                       sk.sketch_matmul(p, proj, T, x, y, ws, hs))
    t = tm.graph_avg(fns, 3) * 7
    out["layer_7b_256_steps"] = dict({"step_us": t * 1e6, "total_us": t * 256e6, "eff_weights_per_s": step_w / t,
                                      "launches_per_step": 7,
                                      "note": "12 MiB of tables: cache-resident, launch-bound"}, **hbm(step_b, t))
    # the same 256 steps, each step's 7 products as one grouped call
    # (sketch_matmul_group: a Z launch and one tile stream over all 7)
    del fns
    groups = [sk.Group([sk.Tables(p, T, proj) for (_, _, _, p, proj, T, _, _, _, _) in layer],
                       [xs[s] for (_, _, _, _, _, _, xs, _, _, _) in layer],
                       [ys[s] for (_, _, _, _, _, _, _, ys, _, _) in layer]) for s in range(256)]
    t = tm.graph_avg([lambda hs, g=g: g.run(hs) for g in groups], 3)
    out["layer_7b_256_steps_grouped"] = dict({"step_us": t * 1e6, "total_us": t * 256e6,
                                              "eff_weights_per_s": step_w / t, "launches_per_step": 2,
                                              "kernels": "group_z_kernel + group_stream_kernel"}, **hbm(step_b, t))
    del groups, layer
    torch.cuda.empty_cache()
    # 32 copies of the layer as one group: 224 products with their own x,
    # 405 MB of tables (beyond the 256 MB last-level cache), one token step
    # of a 32-layer model's linears taken together
    tabs, xs, ys, w32, b32 = [], [], [], 0, 0
    for name, M, N in synth.LAYER_7B_SHAPES:
        for c in range(32):
            p, proj, Ws, imps, tl, tb = encode_copies(torch, sk, dev, gen, M, N, 8, 0.5, 1)
            sk.sketch_encode(p, proj, Ws[0], imps[0], tl[0], status)
            del Ws
            tabs.append(sk.Tables(p, tl[0], proj))
            xs.append(torch.randn(N, generator=gen, device=dev).to(torch.bfloat16))
            ys.append(torch.empty(M, dtype=torch.float32, device=dev))
            w32 += M * N
            b32 += gemv_bytes(tb, 1, N, M)
    torch.cuda.synchronize()
    g32 = sk.Group(tabs, xs, ys)
    t = tm.graph_avg([lambda hs: g32.run(hs)] * 4, 5)
    out["layers32_7b_grouped"] = dict({"avg_us": t * 1e6, "linears": len(tabs), "eff_weights_per_s": w32 / t,
                                       "kernels": "group_z_kernel + group_stream_kernel"}, **hbm(b32, t))
    return out


def cpu_baseline(args, np, lin, X):
    """The oracle on the headline workload: the whole encode, then products
    of token batches until the time budget is spent; the step time is
    extrapolated to the 2048-token batch."""
    import oracle
    c0 = time.perf_counter()
    S = oracle.encode(lin.W, lin.imp, lin.R, lin.bpw, lin.seed, oracle.ABSMIN, w_dtype=oracle.BF16)
    t_enc = time.perf_counter() - c0
    ntok, c1 = 0, time.perf_counter()
    while True:
        oracle.matmul(S, X[ntok:ntok + 4], lin.M, lin.N, lin.R, lin.bpw, lin.seed, x_dtype=oracle.BF16)
        ntok += 4
        if time.perf_counter() - c0 >= args.cpu_seconds or ntok >= X.shape[0]:
            break
    t_prod = time.perf_counter() - c1
    t_step = t_enc + t_prod * X.shape[0] / ntok
    return {"value": lin.M * lin.N / t_step, "unit": "weights/s", "cores": oracle.max_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "mlp_70b_prefill: full encode of the 28672x8192 weight (%.2f s) + float64 products of %d of "
                      "the 2048 tokens (%.2f s), step time extrapolated to 2048 tokens (%.1f s)"
                      % (t_enc, ntok, t_prod, t_step)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the sketch path here is built and timed on a single MI355X; "
              "multi-GPU runs (--gpus %d) are not part of this build." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sub_bit_weight_sketch_amd as sk

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    sk.lib()  # fail loudly if the HIP library is missing
    gen = torch.Generator(device=dev)
    gen.manual_seed(20240601)
    tm = Timer(torch, sk, dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    lin, X, W, imp, Xd, p, proj, T, Y, tb = setup_headline(torch, sk, dev, np)
    M, N, TOK = lin.M, lin.N, X.shape[0]
    sh = sk._stream_handle(dev)

    def step():
        sk.sketch_encode(p, proj, W, imp, T, status, sh)
        sk.sketch_matmul(p, proj, T, Xd, Y, None, sh)

    if args.profile_kernels:
        profile_kernels(torch, sk, dev, gen, tm, status, step)
        return

    # ------------------------------------------------------------ headline
    log("bench: %d warmup + %d timed steps (encode 28672x8192 + 2048-token prefill)" % (args.warmup, args.steps))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    flags = int(status.item())
    if flags:
        raise SystemExit("encode reported flags 0x%x" % flags)
    ms_per_step = elapsed / args.steps * 1e3
    value = M * N / (elapsed / args.steps)

    flops = 2.0 * TOK * M * N
    t_gemm = tm.eager_avg(lambda hs: sk.sketch_matmul(p, proj, T, Xd, Y, None, sh), 10)
    t_enc = tm.graph_avg([lambda hs: sk.sketch_encode(p, proj, W, imp, T, status, hs)], 8)
    gemm_tf = flops / t_gemm / 1e12
    breakdown = {
        "step": {"encode_us": t_enc * 1e6, "gemm_us": t_gemm * 1e6},
        "gemm": {"workload": "mlp_70b_prefill: X 2048x8192 bf16, W 28672x8192 at 0.5 bpw (R=16)",
                 "kernel": "gemm_tile_kernel", "avg_ms": t_gemm * 1e3, "TFLOP_per_s": gemm_tf,
                 "mfma_frac": gemm_tf / BF16_PEAK_TFLOPS,
                 "traffic": measured_traffic("gemm_tile_kernel", "mlp_70b_prefill")},
    }

    # ------------------------------------------------------------ parity
    log("bench: parity of the headline against the oracle")
    import oracle
    S_ref = oracle.encode(lin.W, lin.imp, lin.R, lin.bpw, lin.seed, oracle.ABSMIN, w_dtype=oracle.BF16)
    S_gpu = T.cpu().numpy().view(np.uint16)
    rows = [0, 1023, 2047]
    Yr = oracle.matmul(S_ref, X[rows], M, N, lin.R, lin.bpw, lin.seed, x_dtype=oracle.BF16)
    Yg = Y[rows].cpu().numpy().astype(np.float64)
    rms = np.sqrt((Yr ** 2).mean(axis=1, keepdims=True))
    parity = {"workload": "mlp_70b_prefill", "tables_mismatch": int((S_gpu != S_ref).sum()),
              "y_rows_checked": rows, "y_max_rel": float((np.abs(Yg - Yr) / np.maximum(np.abs(Yr), rms)).max()),
              "y_tol": 1e-3}
    del S_ref

    # ------------------------------------------------------------ breakdown
    if not args.no_breakdown:
        log("bench: encode on every weight shape")
        breakdown["encode"] = bench_encodes(torch, sk, dev, gen, tm, status, (lin, W, imp, p, proj, T, tb))
        log("bench: decode products")
        breakdown["gemv"] = bench_gemvs(torch, sk, dev, gen, tm, status)
        torch.cuda.empty_cache()
        if not args.no_ext:
            breakdown.update(bench_extensions(torch, sk, dev, gen, tm, status, np))

    # ------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline (~%.0f s)" % args.cpu_seconds)
        cpu = cpu_baseline(args, np, lin, X)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Student-t(4) weights, U(0.5,1.5) importance, N(0,1) activations)",
        "config": {"workload": "mlp_70b_prefill: encode 28672x8192 bf16 at 0.5 bpw (R=16) + 2048-token prefill "
                               "product", "global_batch": TOK, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "gemm_tile_kernel", "achieved": gemm_tf, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": gemm_tf / BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("gemm_tile_kernel", "mlp_70b_prefill"),
                     "algorithmic_flops_per_launch": flops},
        "cpu_baseline": cpu,
        "breakdown": breakdown,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------------------
# sketch variants on the attention weight
# ----------------------------------------------------------------------------

EXT_TOKENS = 2048


def bench_extensions(torch, sk, dev, gen, tm, status, np):
    """Materialised W_hat (forward map vs per-weight hash) and the multi-row,
    importance-aware and 4-bit sketches on attention-shaped weights: encode,
    decode, batch-1 and 2048-token products."""
    M, N, R, bpw = 4096, 4096, 8, 0.5
    copies = 4
    p, proj, Ws, imps, tabs, tb = encode_copies(torch, sk, dev, gen, M, N, R, bpw, copies)
    for c in range(copies):
        sk.sketch_encode(p, proj, Ws[c], imps[c], tabs[c], status)
    xs = [torch.randn((1, N), generator=gen, device=dev).to(torch.bfloat16) for _ in range(copies)]
    X = torch.randn((EXT_TOKENS, N), generator=gen, device=dev).to(torch.bfloat16)
    Yb = torch.empty((EXT_TOKENS, M), dtype=torch.float32, device=dev)
    y = torch.empty((1, M), dtype=torch.float32, device=dev)
    w_hat = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    flops = 2.0 * EXT_TOKENS * M * N
    eb = enc_bytes(M, N, tb)
    out = {}

    def avg(fn):
        return tm.graph_avg([lambda hs, c=c: fn(c, hs) for c in range(copies)] * 2, 4)

    log("bench: decode (forward map vs per-weight hash)")
    t_map = avg(lambda c, hs: sk.sketch_decode(p, proj, tabs[c], w_hat, hs))
    t_hash = avg(lambda c, hs: sk.sketch_decode_hashed(p, tabs[c], w_hat, hs))
    sk.sketch_decode(p, proj, tabs[0], w_hat)
    w_map = w_hat.clone()
    sk.sketch_decode_hashed(p, tabs[0], w_hat)
    torch.cuda.synchronize()
    out["decode"] = dict({"kernel": "decode_map_kernel", "avg_us": t_map * 1e6,
                          "hashed_kernel": "decode_hashed_kernel", "hashed_avg_us": t_hash * 1e6,
                          "hashed_over_map": t_hash / t_map, "same_bits": bool(torch.equal(w_map, w_hat)),
                          "note": "W_hat 4096x4096 as bfloat16 from the forward map vs hashing every weight; the "
                                  "pages report 14.9x for their matrix form over a naive hash-based sketch "
                                  "(hardware not named)"},
                         **hbm(tb + R * N * 2 + M * N * 2, t_map))

    def variant(name, pv, projv, tabsv, tbv, dec_bytes):
        for c in range(copies):
            sk.sketch_encode(pv[c] if isinstance(pv, list) else pv, projv, Ws[c], imps[c], tabsv[c], status)
        P = (lambda c: pv[c]) if isinstance(pv, list) else (lambda c: pv)
        r = {}
        t = avg(lambda c, hs: sk.sketch_encode(P(c), projv, Ws[c], imps[c], tabsv[c], status, hs))
        r["encode"] = dict({"avg_us": t * 1e6}, **hbm(eb - tb + tbv, t))
        t = avg(lambda c, hs: sk.sketch_decode(P(c), projv, tabsv[c], w_hat, hs))
        r["decode"] = dict({"avg_us": t * 1e6}, **hbm(dec_bytes, t))
        t = avg(lambda c, hs: sk.sketch_matmul(P(c), projv, tabsv[c], xs[c], y, None, hs))
        r["gemv_b1"] = {"avg_us": t * 1e6, "eff_weights_per_s": M * N / t}
        t = tm.graph_avg([lambda hs, c=c: sk.sketch_matmul(P(c), projv, tabsv[c], X, Yb, None, hs)
                          for c in range(copies)], 2)
        r["gemm_2048"] = {"avg_us": t * 1e6, "TFLOP_per_s": flops / t / 1e12,
                          "mfma_frac": flops / t / 1e12 / BF16_PEAK_TFLOPS}
        torch.cuda.synchronize()
        if int(status.item()):
            raise SystemExit("%s encode reported flags 0x%x" % (name, int(status.item())))
        return r

    log("bench: multi-row sketch (2 rows)")
    p2 = sk.params(M, N, R, bpw, 1, sk.ABSMIN, sk.BF16, rows=2)
    proj2 = sk.projection(p2, dev)
    tabs2 = [torch.empty_like(tabs[0]) for _ in range(copies)]
    out["multi_row_2"] = variant("multi-row", p2, proj2, tabs2, tb, tb + 2 * R * N * 2 + M * N * 2)
    out["multi_row_2"]["workload"] = "attn 4096x4096 sketched with 2 rows of 512 buckets per row block (0.5 bpw)"

    log("bench: importance-aware allocation")
    allocs = [sk.allocate(Ws[c], imps[c], R=R, bpw=bpw) for c in range(copies)]
    pa = [sk.params(M, N, R, bpw, 1, sk.ABSMIN, sk.BF16, alloc=a) for a in allocs]
    proja = sk.projection(pa[0], dev)
    tabsa = [torch.empty(tabs[0].numel(), dtype=torch.int16, device=dev) for _ in range(copies)]
    out["allocated"] = variant("allocated", pa, proja, tabsa, tb, tb + R * N * 4 + M * N * 2)
    out["allocated"]["counts"] = {"min": int(allocs[0].counts.min()), "max": int(allocs[0].counts.max())}

    log("bench: 4-bit buckets")
    p4 = sk.params(M, N, R, bpw, 1, sk.ABSMIN, sk.BF16, bits=4)
    proj4 = sk.projection(p4, dev)
    _, _, tb4 = sk.sketch_layout(p4)
    tabs4 = [torch.zeros(tb4, dtype=torch.uint8, device=dev) for _ in range(copies)]
    out["q4"] = variant("4-bit", p4, proj4, tabs4, tb4, tb4 + R * N * 2 + M * N * 2)
    out["q4"]["workload"] = "attn 4096x4096 at 0.5 bpw with 4-bit buckets (8 weights per bucket, block scales)"
    return out


def profile_kernels(torch, sk, dev, gen, tm, status, step):
    """Eager launches of every hot kernel for rocprofv3 (kernel trace or
    counters): 3 headline steps (encode + prefill GEMM), encodes and decode
    products of the other workloads, and 3 copies of 256 MiB (a kernel of
    known traffic that calibrates the byte counters)."""
    log("bench: profile run")
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    log("bench: profile run: headline done")
    p, proj, Ws, imps, tabs, tb = encode_copies(torch, sk, dev, gen, 4096, 4096, 8, 0.5, 4)
    for c in range(4):
        sk.sketch_encode(p, proj, Ws[c], imps[c], tabs[c], status)
    x = torch.randn((1, 4096), generator=gen, device=dev).to(torch.bfloat16)
    y = torch.empty((1, 4096), dtype=torch.float32, device=dev)
    for c in range(4):
        sk.sketch_matmul(p, proj, tabs[c], x, y, None)
    torch.cuda.synchronize()
    a = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("bench: profile run done")


if __name__ == "__main__":
    main()
