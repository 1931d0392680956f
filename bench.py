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
    ap.add_argument("--profile-kernels", metavar="WORKLOAD", choices=sorted(PROFILE_WORKLOADS),
                    help="eager launches of one workload's hot kernels plus copies of 256 MiB, for a "
                         "rocprofv3 pass (kernel trace or counters); prints no JSON. WORKLOAD: "
                         + ", ".join(sorted(PROFILE_WORKLOADS)))
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/*.md and profiles/traffic.json from the rocprofv3 databases under "
                         "DIR/<workload>/<pass> (passes: kt, fetch, write, mfma)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {"encode_kernel": ("encode.hip", "common.h"), "gemv_mfma_kernel": ("gemv.hip", "common.h"),
                  "group_z_kernel": ("group.hip", "common.h"), "group_stream_kernel": ("group.hip", "common.h"),
                  "group_reduce_kernel": ("group.hip", "common.h"),
                  "gemm_tile_kernel": ("gemm.hip", "common.h"), "decode_map_kernel": ("decode.hip", "common.h"),
                  "decode_hashed_kernel": ("decode.hip", "common.h"),
                  "dgemm_kernel": ("dgemm.h", "rows.hip", "alloc.hip", "q4.hip", "common.h"),
                  "dgemm_add_kernel": ("dgemm.h", "common.h"),
                  "rows_gemv_kernel": ("rows.hip", "common.h"),
                  "alloc_gemv_kernel": ("alloc.hip", "common.h"),
                  "block_importance_kernel": ("alloc.hip", "common.h"),
                  "alloc_decode_kernel": ("alloc.hip", "common.h"),
                  "q4_gemv_kernel": ("q4.hip", "common.h"),
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
    return rec.get("bytes_per_call", rec.get("bytes_per_launch"))


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


def group_kernels(g, q4=False):
    """The kernels one run of a planned Group launches and their count: the Z
    launch, the tile stream and, when the plan splits tiles into pieces,
    the launch that adds the pieces (read from the plan's header)."""
    import struct
    pieces = struct.unpack_from("<11I", bytes(g.plan[:44].cpu().numpy()))[9]
    tag = "<4-bit>" if q4 else ""
    names = ["group_z_kernel" + tag, "group_stream_kernel" + tag]
    if pieces > 1:
        names.append("group_reduce_kernel" + tag)
    return {"kernels": " + ".join(names), "launches_per_step": len(names), "tile_pieces": pieces}


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
                                              "eff_weights_per_s": step_w / t}, **group_kernels(groups[0]),
                                             **hbm(step_b, t))
    del groups, layer
    torch.cuda.empty_cache()
    # 32 copies of the layer as one group: 224 products with their own x,
    # 405 MB of tables (beyond the 256 MB last-level cache), one token step
    # of a 32-layer model's linears taken together
    # The same weights are also sketched with 4-bit codes at 0.5 bpw (R*N/8
    # codes per block, one binary16 scale per block): the same table bytes,
    # four times the buckets, on the 4-bit group kernels.
    tabs, tabs4, xs, ys, w32, b32, b32q = [], [], [], [], 0, 0, 0
    for name, M, N in synth.LAYER_7B_SHAPES:
        p4 = sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.BF16, bits=4)
        nb4, bg4, tb4 = sk.sketch_layout(p4)
        proj4 = sk.projection(p4, dev)
        for c in range(32):
            p, proj, Ws, imps, tl, tb = encode_copies(torch, sk, dev, gen, M, N, 8, 0.5, 1)
            sk.sketch_encode(p, proj, Ws[0], imps[0], tl[0], status)
            t4 = torch.zeros(tb4, dtype=torch.uint8, device=dev)
            sk.sketch_encode(p4, proj4, Ws[0], imps[0], t4, status)
            del Ws
            tabs.append(sk.Tables(p, tl[0], proj))
            tabs4.append(sk.Tables(p4, t4, proj4))
            xs.append(torch.randn(N, generator=gen, device=dev).to(torch.bfloat16))
            ys.append(torch.empty(M, dtype=torch.float32, device=dev))
            w32 += M * N
            b32 += gemv_bytes(tb, 1, N, M)
            b32q += gemv_bytes(nb4 * bg4 // 2 + 2 * nb4, 1, N, M)   # codes + block scales
    torch.cuda.synchronize()
    g32 = sk.Group(tabs, xs, ys)
    t = tm.graph_avg([lambda hs: g32.run(hs)] * 4, 5)
    out["layers32_7b_grouped"] = dict({"avg_us": t * 1e6, "linears": len(tabs), "eff_weights_per_s": w32 / t},
                                      **group_kernels(g32), **hbm(b32, t))
    del g32, tabs
    g32q = sk.Group(tabs4, xs, ys)
    t = tm.graph_avg([lambda hs: g32q.run(hs)] * 4, 5)
    out["layers32_7b_q4_grouped"] = dict({"avg_us": t * 1e6, "linears": len(tabs4), "eff_weights_per_s": w32 / t,
                                          "note": "4-bit codes at 0.5 bpw, one binary16 scale per block"},
                                         **group_kernels(g32q, True), **hbm(b32q, t))
    del g32q, tabs4, xs, ys
    torch.cuda.empty_cache()
    # One tall linear (2,097,152 x 4096 at 0.5 bpw, R = 8: 512 MiB of tables)
    # and one token, in both bucket formats: the tile stream with nothing
    # between its tiles (no linear boundaries, one Z slice set).  The tables
    # are random (finite binary16 buckets; any 4-bit codes with finite block
    # scales): time and traffic do not depend on their values.
    for bits in (16, 4):
        p = sk.params(2097152, 4096, 8, 0.5, 1, sk.ABSMIN, sk.BF16, bits=bits)
        nb, bg, tb = sk.sketch_layout(p)
        if bits == 16:
            tt = torch.randint(0, 0x3C00, (nb, bg), generator=gen, device=dev, dtype=torch.int16)
            tbytes = nb * bg * 2
        else:
            tt = torch.randint(0, 0x3C, (tb,), generator=gen, device=dev, dtype=torch.uint8)
            tbytes = nb * bg // 2 + 2 * nb
        x = torch.randn(4096, generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty(2097152, dtype=torch.float32, device=dev)
        g = sk.Group([sk.Tables(p, tt, sk.projection(p, dev))], [x], [y])
        t = tm.graph_avg([lambda hs: g.run(hs)] * 4, 5)
        out["stack_2097152x4096_%s_grouped" % ("q4" if bits == 4 else "b16")] = dict(
            {"avg_us": t * 1e6, "eff_weights_per_s": 2097152 * 4096 / t,
             "note": "one 2,097,152 x 4096 linear (512 MiB of tables), one token; random tables"},
            **group_kernels(g, bits == 4), **hbm(gemv_bytes(tbytes, 1, 4096, 2097152), t))
        del g, tt, x, y
        torch.cuda.empty_cache()
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
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
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

    if args.profile_kernels:
        profile_kernels(torch, sk, dev, gen, status, args.profile_kernels)
        return

    lin, X, W, imp, Xd, p, proj, T, Y, tb = setup_headline(torch, sk, dev, np)
    M, N, TOK = lin.M, lin.N, X.shape[0]
    sh = sk._stream_handle(dev)

    def step(ev=None):
        # ev: three HIP events recorded on the library's stream around the
        # encode and the product, so both kernels are timed inside the
        # timed region itself
        if ev:
            ev[0].record(tm.stream)
        sk.sketch_encode(p, proj, W, imp, T, status, sh)
        if ev:
            ev[1].record(tm.stream)
        sk.sketch_matmul(p, proj, T, Xd, Y, None, sh)
        if ev:
            ev[2].record(tm.stream)

    # ------------------------------------------------------------ headline
    # each kernel alone first (breakdown figures: the product back to back,
    # the encode from a graph); this also lets the clocks settle, which takes
    # a few dozen launches of the product (0.91 ms in the first ones, 0.76 ms
    # after)
    log("bench: the product and the encode alone")
    # the tables the product reads (the product's speed depends on them: with
    # all-zero tables it draws less power and runs at a higher clock)
    sk.sketch_encode(p, proj, W, imp, T, status, sh)
    t_gemm_alone = tm.eager_avg(lambda hs: sk.sketch_matmul(p, proj, T, Xd, Y, None, sh), 40)
    t_enc_alone = tm.graph_avg([lambda hs: sk.sketch_encode(p, proj, W, imp, T, status, hs)], 8)
    log("bench: %d warmup + %d timed steps (encode 28672x8192 + 2048-token prefill)" % (args.warmup, args.steps))
    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    flags = int(status.item())
    if flags:
        raise SystemExit("encode reported flags 0x%x" % flags)
    ms_per_step = elapsed / args.steps * 1e3
    value = M * N / (elapsed / args.steps)
    t_enc = sum(e[0].elapsed_time(e[1]) for e in evs) * 1e-3 / args.steps
    t_gemm = sum(e[1].elapsed_time(e[2]) for e in evs) * 1e-3 / args.steps

    flops = 2.0 * TOK * M * N
    gemm_tf = flops / t_gemm / 1e12
    breakdown = {
        "step": {"encode_us": t_enc * 1e6, "gemm_us": t_gemm * 1e6,
                 "note": "HIP events around each launch of the timed steps"},
        "encode_alone_us": t_enc_alone * 1e6,
        "gemm": {"workload": "mlp_70b_prefill: X 2048x8192 bf16, W 28672x8192 at 0.5 bpw (R=16)",
                 "kernel": "gemm_tile_kernel", "avg_ms": t_gemm * 1e3, "TFLOP_per_s": gemm_tf,
                 "mfma_frac": gemm_tf / BF16_PEAK_TFLOPS,
                 "avg_ms_back_to_back": t_gemm_alone * 1e3,
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
        # with the workspace the call reports (the multi-row product splits K with it)
        wsb = sk.sketch_workspace_bytes(P(0), X.shape[0], sk.BF16)
        wsv = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev) if wsb else None
        t = tm.graph_avg([lambda hs, c=c: sk.sketch_matmul(P(c), projv, tabsv[c], X, Yb, wsv, hs)
                          for c in range(copies)], 2)
        r["gemm_2048"] = {"avg_us": t * 1e6, "TFLOP_per_s": flops / t / 1e12,
                          "mfma_frac": flops / t / 1e12 / BF16_PEAK_TFLOPS, "workspace_bytes": wsb}
        del wsv
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


PROFILE_REPS = 5       # repetitions the summaries average
PROFILE_WARMUP = 20    # repetitions before them, while the clocks settle


def _last_reps(items):
    """The last PROFILE_REPS repetitions' share of a kernel's dispatches (in
    launch order): each repetition launches it the same number of times."""
    k = max(1, round(len(items) / (PROFILE_WARMUP + PROFILE_REPS)))
    return items[-PROFILE_REPS * k:]


def _tables_bytes(M, N, R, bpw):
    return (M // R) * int(R * N * bpw / 16) * 2


def _profile_workloads():
    """Per workload: what one repetition launches, and the algorithmic
    bytes (or flops) of each profiled kernel per repetition."""
    c5_tb = _tables_bytes(28672, 8192, 16, 0.5)
    at_tb = _tables_bytes(4096, 4096, 8, 0.5)
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    l32_tb = 32 * sum(_tables_bytes(M, N, 8, 0.5) for M, N in shapes)
    l32_io = 32 * sum(N * 2 + M * 4 for M, N in shapes)
    l32_sc = 32 * sum(M // 8 * 2 for M, N in shapes)   # one binary16 scale per block of 8 rows
    l1_tb, l1_io, l1_sc = l32_tb // 32, l32_io // 32, l32_sc // 32
    at_w = 4096 * 4096 * 2                     # W or W_hat as bfloat16
    at_wi = at_w + 4096 * 4                    # W + importance
    at_map = 8 * 4096 * 2                      # one 16-bit forward map (R*N entries)
    at_q4 = 512 * 4096 // 2 + 512 * 2          # 4-bit codes + block scales
    at_x, at_y = 2048 * 4096 * 2, 2048 * 4096 * 4
    at_fl = 2 * 2048 * 4096 * 4096
    st_tb = _tables_bytes(2097152, 4096, 8, 0.5)
    st_io = 4096 * 2 + 2097152 * 4
    return {
        "mlp_70b_prefill": {
            "describe": "sketch_encode of the 28672x8192 bfloat16 weight at 0.5 bpw (R=16), then sketch_matmul "
                        "of the 2048-token prefill (X 2048x8192 bfloat16 -> Y 2048x28672 float32)",
            "kernels": {
                "encode_kernel": {"bytes": 28672 * 8192 * 2 + 8192 * 4 + c5_tb,
                                  "bytes_note": "W 469,762,048 + importance 32,768 read, tables %s written"
                                                % format(c5_tb, ",")},
                "gemm_tile_kernel": {"bytes": 2048 * 8192 * 2 + c5_tb + 2048 * 28672 * 4,
                                     "flops": 2 * 2048 * 28672 * 8192, "mfma": True,
                                     "bytes_note": "X 33,554,432 + tables %s read, Y 234,881,024 written"
                                                   % format(c5_tb, ",")}}},
        "attn_4096x4096": {
            "describe": "sketch_encode of one 4096x4096 bfloat16 weight at 0.5 bpw (R=8), a batch-1 "
                        "sketch_matmul (Z summed in place), and W_hat materialised as bfloat16 twice: "
                        "sketch_decode (forward map) and sketch_decode_hashed (every index hashed)",
            "kernels": {
                "encode_kernel": {"bytes": 4096 * 4096 * 2 + 4096 * 4 + at_tb,
                                  "bytes_note": "W 33,554,432 + importance 16,384 read, tables %s written"
                                                % format(at_tb, ",")},
                "gemv_mfma_kernel": {"bytes": at_tb + 4096 * 2 + 4096 * 4,
                                     "bytes_note": "tables %s + x 8,192 read, y 16,384 written"
                                                   % format(at_tb, ",")},
                "decode_map_kernel": {"bytes": at_tb + at_map + at_w,
                                      "bytes_note": "tables %s + forward map %s read, W_hat %s written"
                                                    % (format(at_tb, ","), format(at_map, ","), format(at_w, ","))},
                "decode_hashed_kernel": {"bytes": at_tb + at_w,
                                         "bytes_note": "tables %s read, W_hat %s written"
                                                       % (format(at_tb, ","), format(at_w, ","))}}},
        "attn_4096x4096_rows2": {
            "describe": "the 4096x4096 weight sketched with 2 rows (two segments of 512 buckets per row "
                        "block, 0.5 bpw, R=8): sketch_encode, sketch_decode to bfloat16, a batch-1 and a "
                        "2048-token sketch_matmul (with the workspace it reports: K split in two)",
            "kernels": {
                "encode_kernel": {"bytes": at_wi + at_tb,
                                  "bytes_note": "W + importance %s read, tables %s written"
                                                % (format(at_wi, ","), format(at_tb, ","))},
                "decode_map_kernel": {"bytes": at_tb + 2 * at_map + at_w,
                                      "bytes_note": "tables %s + two forward maps %s read, W_hat %s written"
                                                    % (format(at_tb, ","), format(2 * at_map, ","),
                                                       format(at_w, ","))},
                "rows_gemv_kernel": {"bytes": at_tb + 4096 * 2 + 4096 * 4,
                                     "bytes_note": "tables + x read, y written (every weight decoded)"},
                "dgemm_kernel": {"bytes": at_x + at_tb + at_y, "flops": at_fl, "mfma": True,
                                     "bytes_note": "X %s + tables read, Y %s written (K split in two: "
                                                   "the second half's part goes to the workspace)"
                                                   % (format(at_x, ","), format(at_y, ","))},
                "dgemm_add_kernel": {"bytes": 3 * at_y,
                                     "bytes_note": "Y and the part read, Y written (%s each)" % format(at_y, ",")}}},
        "attn_4096x4096_allocated": {
            "describe": "the 4096x4096 weight with importance-aware bucket counts (block scores from "
                        "W^2 E[x^2], the same total budget, 0.5 bpw, R=8): sketch_block_importance, "
                        "sketch_encode, sketch_decode to bfloat16, a batch-1 and a 2048-token sketch_matmul",
            "kernels": {
                "block_importance_kernel": {"bytes": 4096 * 4096 * 2 + 4096 * 4 + 512 * 4,
                                            "bytes_note": "W + E[x^2] read, 512 block scores written"},
                "encode_kernel": {"bytes": at_wi + at_tb,
                                  "bytes_note": "W + importance %s read, tables %s written"
                                                % (format(at_wi, ","), format(at_tb, ","))},
                "alloc_decode_kernel": {"bytes": at_tb + 2 * at_map + at_w,
                                        "bytes_note": "tables + 32-bit hash map %s read, W_hat %s written"
                                                      % (format(2 * at_map, ","), format(at_w, ","))},
                "alloc_gemv_kernel": {"bytes": at_tb + 4096 * 2 + 4096 * 4,
                                      "bytes_note": "tables + x read, y written (every weight decoded)"},
                "dgemm_kernel": {"bytes": at_x + at_tb + at_y, "flops": at_fl, "mfma": True,
                                      "bytes_note": "X %s + tables read, Y %s written"
                                                    % (format(at_x, ","), format(at_y, ","))}}},
        "attn_4096x4096_q4": {
            "describe": "the 4096x4096 weight with 4-bit codes at 0.5 bpw (4096 codes per row block of 8 rows, "
                        "one binary16 scale per block): sketch_encode, sketch_decode to bfloat16, a batch-1 "
                        "and a 2048-token sketch_matmul",
            "kernels": {
                "encode_kernel": {"bytes": at_wi + at_q4,
                                  "bytes_note": "W + importance %s read, codes + scales %s written"
                                                % (format(at_wi, ","), format(at_q4, ","))},
                "q4_decode_kernel": {"bytes": at_q4 + at_map + at_w,
                                     "bytes_note": "codes + scales + forward map read, W_hat %s written"
                                                   % format(at_w, ",")},
                "q4_gemv_kernel": {"bytes": at_q4 + 4096 * 2 + 4096 * 4,
                                   "bytes_note": "codes + scales + x read, y written (every weight decoded)"},
                "gemm_tile_kernel": {"bytes": at_x + at_q4 + at_y, "flops": at_fl, "mfma": True,
                                     "bytes_note": "X %s + codes + scales read, Y %s written"
                                                   % (format(at_x, ","), format(at_y, ","))}}},
        "layers32_7b": {
            "describe": "one sketch_matmul_group over 32 copies of a 7B decoder layer's seven linears "
                        "(4096x4096 x4, 11008x4096 x2, 4096x11008; R=8, 0.5 bpw; 224 linears, one "
                        "bfloat16 token each; tables of random finite binary16 bits, on which time and "
                        "traffic do not depend)",
            "kernels": {
                "group_stream_kernel": {"bytes": l32_tb + l32_io,
                                        "bytes_note": "tables %s read, x + y %s (algorithmic bytes of the "
                                                      "whole product)" % (format(l32_tb, ","), format(l32_io, ","))},
                "group_z_kernel": {"bytes": None}}},
        "layers32_7b_q4": {
            "describe": "one sketch_matmul_group over the same 224 linears sketched with 4-bit codes at 0.5 bpw "
                        "(R*N/8 codes per block, one binary16 scale per block; codes and scales random, on "
                        "which time and traffic do not depend)",
            "kernels": {
                "group_stream_kernel": {"bytes": l32_tb + l32_sc + l32_io,
                                        "bytes_note": "codes %s + block scales %s read, x + y %s (algorithmic "
                                                      "bytes of the whole product)"
                                                      % (format(l32_tb, ","), format(l32_sc, ","),
                                                         format(l32_io, ","))},
                "group_z_kernel": {"bytes": None}}},
        "layer_7b": {
            "describe": "one sketch_matmul_group over one 7B decoder layer's seven linears (4096x4096 x4, "
                        "11008x4096 x2, 4096x11008; R=8, 0.5 bpw; one bfloat16 token each; random finite "
                        "binary16 tables): 12 MiB of tables, cache-resident across repetitions; tiles split "
                        "into pieces, so three launches",
            "kernels": {
                "group_stream_kernel": {"bytes": l1_tb + l1_io,
                                        "bytes_note": "tables %s read, x + y %s (algorithmic bytes of the "
                                                      "whole product)" % (format(l1_tb, ","), format(l1_io, ","))},
                "group_z_kernel": {"bytes": None},
                "group_reduce_kernel": {"bytes": None}}},
        "layer_7b_q4": {
            "describe": "one sketch_matmul_group over the same seven linears with 4-bit codes at 0.5 bpw (one "
                        "binary16 scale per block; random codes and scales); three launches",
            "kernels": {
                "group_stream_kernel": {"bytes": l1_tb + l1_sc + l1_io,
                                        "bytes_note": "codes %s + block scales %s read, x + y %s"
                                                      % (format(l1_tb, ","), format(l1_sc, ","),
                                                         format(l1_io, ","))},
                "group_z_kernel": {"bytes": None},
                "group_reduce_kernel": {"bytes": None}}},
        "stack_2097152x4096": {
            "describe": "one sketch_matmul_group of a single 2,097,152x4096 linear at 0.5 bpw (R=8: 512 MiB of "
                        "binary16 tables, random finite bits) and one bfloat16 token",
            "kernels": {
                "group_stream_kernel": {"bytes": st_tb + st_io,
                                        "bytes_note": "tables %s read, x + y %s" % (format(st_tb, ","),
                                                                                 format(st_io, ","))},
                "group_z_kernel": {"bytes": None}}},
        "stack_2097152x4096_q4": {
            "describe": "the same 2,097,152x4096 linear with 4-bit codes at 0.5 bpw (512 MiB of random codes, "
                        "random finite block scales) and one bfloat16 token",
            "kernels": {
                "group_stream_kernel": {"bytes": st_tb + 262144 * 2 + st_io,
                                        "bytes_note": "codes %s + block scales 524,288 read, x + y %s"
                                                      % (format(st_tb, ","), format(st_io, ","))},
                "group_z_kernel": {"bytes": None}}},
    }


PROFILE_WORKLOADS = ("mlp_70b_prefill", "attn_4096x4096", "attn_4096x4096_rows2", "attn_4096x4096_allocated",
                     "attn_4096x4096_q4", "layers32_7b", "layers32_7b_q4", "layer_7b", "layer_7b_q4",
                     "stack_2097152x4096", "stack_2097152x4096_q4")


def profile_kernels(torch, sk, dev, gen, status, workload):
    """Eager launches of one workload's hot kernels for a rocprofv3 pass:
    setup, then PROFILE_WARMUP + PROFILE_REPS repetitions of the workload, then 3 copies of
    256 MiB (a kernel of known traffic that calibrates the byte counters)."""
    import numpy as np
    import synth
    log("bench: profile run of %s" % workload)
    if workload == "mlp_70b_prefill":
        lin, X, W, imp, Xd, p, proj, T, Y, tb = setup_headline(torch, sk, dev, np)
        torch.cuda.synchronize()
        for _ in range(PROFILE_WARMUP + PROFILE_REPS):
            sk.sketch_encode(p, proj, W, imp, T, status)
            sk.sketch_matmul(p, proj, T, Xd, Y, None)
    elif workload == "attn_4096x4096":
        p, proj, Ws, imps, tabs, tb = encode_copies(torch, sk, dev, gen, 4096, 4096, 8, 0.5, 1)
        x = torch.randn((1, 4096), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((1, 4096), dtype=torch.float32, device=dev)
        w_hat = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for _ in range(PROFILE_WARMUP + PROFILE_REPS):
            sk.sketch_encode(p, proj, Ws[0], imps[0], tabs[0], status)
            sk.sketch_matmul(p, proj, tabs[0], x, y, None)
            sk.sketch_decode(p, proj, tabs[0], w_hat)
            sk.sketch_decode_hashed(p, tabs[0], w_hat)
    elif workload.startswith("attn_4096x4096_"):
        M = N = 4096
        p, proj, Ws, imps, tabs, tb = encode_copies(torch, sk, dev, gen, M, N, 8, 0.5, 1)
        x = torch.randn((1, N), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((1, M), dtype=torch.float32, device=dev)
        X = torch.randn((2048, N), generator=gen, device=dev).to(torch.bfloat16)
        Y = torch.empty((2048, M), dtype=torch.float32, device=dev)
        w_hat = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        kind = workload[len("attn_4096x4096_"):]
        if kind == "rows2":
            pv = sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.BF16, rows=2)
            tv = torch.empty_like(tabs[0])
        elif kind == "q4":
            pv = sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.BF16, bits=4)
            tv = torch.zeros(sk.sketch_layout(pv)[2], dtype=torch.uint8, device=dev)
        else:
            tv = torch.empty(tabs[0].numel(), dtype=torch.int16, device=dev)
        wsb = sk.sketch_workspace_bytes(pv, 2048, sk.BF16) if kind != "allocated" else 0
        wsv = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev) if wsb else None
        torch.cuda.synchronize()
        for _ in range(PROFILE_WARMUP + PROFILE_REPS):
            if kind == "allocated":   # the block importances and counts are part of each repetition
                a = sk.allocate(Ws[0], imps[0], R=8, bpw=0.5)
                pv = sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.BF16, alloc=a)
            pj = sk.projection(pv, dev)
            sk.sketch_encode(pv, pj, Ws[0], imps[0], tv, status)
            sk.sketch_decode(pv, pj, tv, w_hat)
            sk.sketch_matmul(pv, pj, tv, x, y, None)
            sk.sketch_matmul(pv, pj, tv, X, Y, wsv)   # with the reported workspace (multi-row: K split)
    elif workload.startswith("stack_2097152x4096"):
        q4 = workload.endswith("_q4")
        p = sk.params(2097152, 4096, 8, 0.5, 1, sk.ABSMIN, sk.BF16, bits=4 if q4 else 16)
        nb, bg, tb = sk.sketch_layout(p)
        if q4:   # bytes below 0x3C make every binary16 scale finite
            tt = torch.randint(0, 0x3C, (tb,), generator=gen, device=dev, dtype=torch.uint8)
        else:
            tt = torch.randint(0, 0x3C00, (nb, bg), generator=gen, device=dev, dtype=torch.int16)
        x = torch.randn(4096, generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty(2097152, dtype=torch.float32, device=dev)
        g = sk.Group([sk.Tables(p, tt, sk.projection(p, dev))], [x], [y])
        torch.cuda.synchronize()
        for _ in range(PROFILE_WARMUP + PROFILE_REPS):
            g.run()
    else:
        # one buffer of random tables (the product's time and traffic do not
        # depend on the values: finite binary16 buckets, or any 4-bit codes
        # with finite block scales), sliced per linear: a few setup
        # dispatches instead of hundreds under the counters
        q4 = workload.endswith("_q4")
        shapes = [(M, N) for _, M, N in synth.LAYER_7B_SHAPES] * (32 if workload.startswith("layers32") else 1)
        ps = [sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.BF16, bits=4 if q4 else 16) for M, N in shapes]
        lay = [sk.sketch_layout(p) for p in ps]
        if q4:
            # each linear's buffer at a 256-byte boundary: codes, then scales;
            # bytes below 0x3C make every binary16 scale finite
            sizes = [(tb + 255) // 256 * 256 for _, _, tb in lay]
            tall = torch.randint(0, 0x3C, (sum(sizes),), generator=gen, device=dev, dtype=torch.int32).to(torch.uint8)
        else:
            tall = torch.randint(0, 0x3C00, (sum(nb * bg for nb, bg, _ in lay),), generator=gen, device=dev,
                                 dtype=torch.int32).to(torch.int16)
        xall = torch.randn(sum(N for _, N in shapes), generator=gen, device=dev).to(torch.bfloat16)
        yall = torch.empty(sum(M for M, _ in shapes), dtype=torch.float32, device=dev)
        tabs, xs, ys, at, ax, ay = [], [], [], 0, 0, 0
        for i, ((M, N), p, (nb, bg, tb)) in enumerate(zip(shapes, ps, lay)):
            if q4:
                tabs.append(sk.Tables(p, tall[at:at + tb], sk.projection(p, dev)))
                at += sizes[i]
            else:
                tabs.append(sk.Tables(p, tall[at:at + nb * bg].view(nb, bg), sk.projection(p, dev)))
                at += nb * bg
            xs.append(xall[ax:ax + N])
            ys.append(yall[ay:ay + M])
            ax, ay = ax + N, ay + M
        g = sk.Group(tabs, xs, ys)
        torch.cuda.synchronize()
        for _ in range(PROFILE_WARMUP + PROFILE_REPS):
            g.run()
    torch.cuda.synchronize()
    if int(status.item()):
        raise SystemExit("encode reported flags 0x%x" % int(status.item()))
    a = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("bench: profile run done")


COPY_KERNEL = "copyBuffer"
COPY_KIB = 256 * 1024


def _db_rows(path, query):
    import glob
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(path, "**", "*results.db"), recursive=True))
    if not dbs:
        return None
    con = sqlite3.connect(dbs[-1])
    try:
        return list(con.execute(query))
    finally:
        con.close()


def _short_name(name):
    if name.startswith("_Z"):   # a name the trace left mangled
        import subprocess
        try:
            name = subprocess.run(["c++filt", name], capture_output=True, text=True, check=True).stdout.strip()
        except (OSError, subprocess.CalledProcessError):
            pass
    if name.startswith("_ZN"):   # still mangled: the last nested name, plus <n> for one integer argument
        import re
        parts, rest = [], name[3:]
        while rest and rest[0].isdigit():
            m = re.match(r"(\d+)", rest)
            k = int(m.group(1))
            parts.append(rest[len(m.group(1)):len(m.group(1)) + k])
            rest = rest[len(m.group(1)) + k:]
        arg = re.match(r"ILi(\d+)E", rest)
        return (parts[-1] if parts else name) + ("<%s>" % arg.group(1) if arg else "")
    n = name.replace("(anonymous namespace)::", "").replace("sketch::", "").replace("void ", "")
    return n.split("(")[0].strip()


def summarize_profiles(top):
    """profiles/<kernel>_<workload>.md and profiles/traffic.json from the
    rocprofv3 databases of the --profile-kernels passes under
    top/<workload>/{kt,fetch,write,mfma}."""
    cmds = {
        "kt": "rocprofv3 --kernel-trace --stats -d {d}/{w}/kt -o run -- python3 -u bench.py --profile-kernels {w}",
        "fetch": "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -d {d}/{w}/fetch -o run -- python3 -u bench.py "
                 "--profile-kernels {w}",
        "write": "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -d {d}/{w}/write -o run -- python3 -u bench.py "
                 "--profile-kernels {w}",
        "mfma": "timeout -s KILL 120 rocprofv3 --pmc MfmaUtil SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS "
                "SQ_BUSY_CYCLES SQ_WAVES -d {d}/{w}/mfma -o run -- python3 -u bench.py --profile-kernels {w}",
    }
    try:
        with open(os.path.join(PROFILES, "traffic.json")) as fh:
            traffic = json.load(fh)
    except (OSError, ValueError):
        traffic = {}
    written = []
    for w, spec in _profile_workloads().items():
        wd = os.path.join(top, w)
        if not os.path.isdir(wd):
            continue
        kt = _db_rows(os.path.join(wd, "kt"), "select name, start, end from kernels order by start") or []
        counters = {}
        for ps in ("fetch", "write", "mfma"):
            rows = _db_rows(os.path.join(wd, ps), "select dispatch_id, kernel_name, counter_name, value "
                                                  "from counters_collection")
            if rows is None:
                continue
            per = {}
            for did, kname, cname, val in rows:
                per.setdefault((kname, cname), {}).setdefault(did, 0.0)
                per[(kname, cname)][did] += val
            counters[ps] = per
        def counter_sum(ps, pattern, cname):
            """Sum over the dispatches of kernels named like pattern, and the
            number of dispatches."""
            tot, n = 0.0, 0
            for (kname, cn), d in counters.get(ps, {}).items():
                if pattern in kname and cn == cname:
                    vals = _last_reps([d[i] for i in sorted(d)])
                    tot += sum(vals)
                    n += len(vals)
            return tot, n
        # calibration: the three 256 MiB copies (the largest copy dispatches;
        # small copies, e.g. of a status word, use the same kernel)
        cal = {}
        for ps, cname in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
            vals = sorted((v for (kname, cn), d in counters.get(ps, {}).items()
                           if COPY_KERNEL in kname and cn == cname for v in d.values()), reverse=True)[:3]
            cal[cname] = (COPY_KIB / (sum(vals) / len(vals)), sum(vals) / len(vals)) if len(vals) == 3 else (None, None)
        for kern, ks in spec["kernels"].items():
            disp = []
            for name in sorted({n for n, _, _ in kt if kern in n}):
                disp += [(name, d) for d in _last_reps([(e - st) / 1e3 for n, st, e in kt if n == name])]
            lines = ["# %s on %s" % (kern, w), "", spec["describe"] + ". One MI355X (gfx950); one "
                     "repetition of the workload is one call; the profile run makes %d, of which the "
                     "figures below take the last %d (the first ones let the clocks settle)."
                     % (PROFILE_WARMUP + PROFILE_REPS, PROFILE_REPS), ""]
            lines += ["## Kernel duration (rocprofv3 kernel trace)", "",
                      "Command (from the repository root, any scratch directory `<d>`):", "",
                      "    " + cmds["kt"].format(d="<d>", w=w), "",
                      "| kernel | dispatches | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
            names = sorted({n for n, _ in disp})
            per_call_us = 0.0
            for n in names:
                ds = [t for m, t in disp if m == n]
                lines.append("| `%s` | %d | %.2f | %.2f | %.2f |" % (_short_name(n), len(ds), sum(ds) / len(ds),
                                                                   min(ds), max(ds)))
                per_call_us += sum(ds) / PROFILE_REPS
            lines += ["", "Per call: **%.2f us**." % per_call_us, ""]
            rec = {"kernels": [_short_name(n) for n in names], "us_per_call": per_call_us,
                   "source_digest": kernel_source_digest(kern)}
            if ks.get("bytes"):
                rec["algorithmic_bytes"] = ks["bytes"]
                lines.append("Algorithmic bytes per call: %s (%s): %.1f%% of 8 TB/s at that duration."
                             % (format(ks["bytes"], ","), ks["bytes_note"],
                                100.0 * ks["bytes"] / (per_call_us * 1e-6) / 8e12 if per_call_us else 0.0))
                lines.append("")
            if ks.get("flops"):
                rec["algorithmic_flops"] = ks["flops"]
                lines.append("Algorithmic flops per call: %s: %.1f%% of the 2.5 PFLOP/s dense bf16 peak at that "
                             "duration." % (format(ks["flops"], ","),
                                           100.0 * ks["flops"] / (per_call_us * 1e-6) / 2.5e15 if per_call_us else 0))
                lines.append("")
            fz, nf = counter_sum("fetch", kern, "FETCH_SIZE")
            wz, nw = counter_sum("write", kern, "WRITE_SIZE")
            if nf and nw and cal["FETCH_SIZE"][0] and cal["WRITE_SIZE"][0]:
                fs, ws = cal["FETCH_SIZE"][0], cal["WRITE_SIZE"][0]
                fb = fz / PROFILE_REPS * fs * 1024
                wb = wz / PROFILE_REPS * ws * 1024
                lines += ["## HBM traffic (rocprofv3 counters, one counter per pass)", "",
                          "    " + cmds["fetch"].format(d="<d>", w=w), "    " + cmds["write"].format(d="<d>", w=w), "",
                          "The same run copies 256 MiB three times (`%s`): per copy FETCH_SIZE reads %.1f KiB and "
                          "WRITE_SIZE %.1f KiB against 262,144 KiB moved each way, so FETCH_SIZE is scaled by %.3f "
                          "and WRITE_SIZE by %.3f." % (COPY_KERNEL, cal["FETCH_SIZE"][1], cal["WRITE_SIZE"][1], fs, ws),
                          "", "| counter | dispatches | raw KiB per call | scaled bytes per call |", "|---|---|---|---|",
                          "| FETCH_SIZE | %d | %.1f | %d |" % (nf, fz / PROFILE_REPS, fb),
                          "| WRITE_SIZE | %d | %.1f | %d |" % (nw, wz / PROFILE_REPS, wb), ""]
                line = "Measured traffic per call: **%d bytes**" % (fb + wb)
                if ks.get("bytes"):
                    line += "; algorithmic %s; ratio %.3f" % (format(ks["bytes"], ","), (fb + wb) / ks["bytes"])
                lines += [line + ".", ""]
                rec["bytes_per_call"] = fb + wb
                rec["fetch_bytes_per_call"], rec["write_bytes_per_call"] = fb, wb
            if ks.get("mfma") and "mfma" in counters:
                util, nu = counter_sum("mfma", kern, "MfmaUtil")
                lines += ["## Matrix-core and instruction counters", "", "    " + cmds["mfma"].format(d="<d>", w=w), "",
                          "| counter | per call |", "|---|---|"]
                if nu:
                    lines.append("| MfmaUtil (%% of SIMD cycles the MFMA unit is busy; dispatch mean) | %.1f |"
                                 % (util / nu))
                    rec["mfma_util_pct"] = util / nu
                ins = {}
                for cn in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_BUSY_CYCLES", "SQ_WAVES"):
                    v, n = counter_sum("mfma", kern, cn)
                    if n:
                        ins[cn] = v / PROFILE_REPS
                        lines.append("| %s | %.4g |" % (cn, v / PROFILE_REPS))
                if ins.get("SQ_INSTS_MFMA"):
                    lines += ["", "VALU instructions per MFMA instruction: %.2f; LDS instructions per MFMA: %.2f."
                              % (ins.get("SQ_INSTS_VALU", 0) / ins["SQ_INSTS_MFMA"],
                                 ins.get("SQ_INSTS_LDS", 0) / ins["SQ_INSTS_MFMA"])]
                    rec["valu_per_mfma"] = ins.get("SQ_INSTS_VALU", 0) / ins["SQ_INSTS_MFMA"]
                lines.append("")
            lines.append("Kernel sources digest (sha256 of %s, first 16 hex): `%s`."
                         % (" + ".join(KERNEL_SOURCES[kern]), rec["source_digest"]))
            out = os.path.join(PROFILES, "%s_%s.md" % (kern, w))
            with open(out, "w") as fh:
                fh.write("\n".join(lines) + "\n")
            traffic["%s@%s" % (kern, w)] = rec
            written.append(out)
    # the default bench run under the kernel trace: its own per-kernel
    # averages beside the figures bench.py measured with HIP events
    bt = _db_rows(os.path.join(top, "bench", "kt"), "select name, start, end from kernels")
    if bt:
        agg = {}
        for n, st, e in bt:
            agg.setdefault(_short_name(n), []).append((e - st) / 1e3)
        lines = ["# Kernel trace of the default bench run", "",
                 "Every kernel of `bench.py` with no options but `--no-cpu-baseline` (the headline steps on "
                 "mlp_70b_prefill, then the encode, decode-product and extension breakdowns), one MI355X "
                 "(gfx950), ordered by total time.", "",
                 "    rocprofv3 --kernel-trace --stats -d <d>/bench/kt -o run -- python3 -u bench.py "
                 "--no-cpu-baseline > <d>/bench/bench.json", "",
                 "| kernel | calls | average (us) | median (us) | min (us) | max (us) | total (ms) |",
                 "|---|---|---|---|---|---|---|"]
        for n, ds in sorted(agg.items(), key=lambda kv: -sum(kv[1]))[:40]:
            lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %.2f | %.2f |"
                         % (n, len(ds), sum(ds) / len(ds), sorted(ds)[len(ds) // 2], min(ds), max(ds),
                            sum(ds) / 1e3))
        try:
            with open(os.path.join(top, "bench", "bench.json")) as fh:
                line = json.loads(fh.read().strip().splitlines()[-1])
            g = line["breakdown"]["gemm"]
            lines += ["", "The same run's own figures (HIP events): `gemm_tile_kernel` %.2f us per prefill product "
                      "(%.1f%% of the bf16 peak); headline step %.3f ms."
                      % (g["avg_ms"] * 1e3, 100 * g["mfma_frac"], line["ms_per_step"])]
        except (OSError, ValueError, KeyError, IndexError):
            pass
        out = os.path.join(PROFILES, "bench_kernel_trace.md")
        with open(out, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        written.append(out)
    with open(os.path.join(PROFILES, "traffic.json"), "w") as fh:
        json.dump(traffic, fh, indent=1, sort_keys=True)
        fh.write("\n")
    for o in written:
        log("wrote", os.path.relpath(o, ROOT))


if __name__ == "__main__":
    main()
