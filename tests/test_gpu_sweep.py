"""Seeded sweep of random configurations through the C ABI against the oracle.

Every case draws a sketch kind (binary16 buckets, multi-row, importance-aware
allocation, 4-bit buckets), a shape (ragged row blocks and column counts, N
not always a multiple of 8), a bucket count, a weight dtype, a rule, an
importance vector or none, and a batch (decode passes and the matrix-core
path); tables must match bit for bit and the product must meet the 1e-3
tolerance.  The case is printed before it runs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y_close, dev, oracle_dtype, to_dev

import sub_bit_weight_sketch_amd as sk

pytestmark = pytest.mark.gpu

KINDS = ("uniform", "rows", "alloc", "q4")


def _draw(seed):
    g = np.random.default_rng(1000 + seed)
    kind = KINDS[seed % len(KINDS)]
    for _ in range(200):
        R = int(g.choice([1, 2, 3, 4, 8, 16]))
        nb = int(g.integers(1, 24))
        N = int(g.choice([int(g.integers(8, 129)) * 8, int(g.integers(9, 700))]))
        per_bucket = int(g.choice([8, 16, 32, 64]))                 # weights per bucket
        div = 4 if kind == "q4" else 16
        buckets = (R * N) // per_bucket
        if buckets < 2:
            continue
        if kind == "q4":
            buckets -= buckets % 2
        rows = int(g.choice([2, 3, 4])) if kind == "rows" else 1
        buckets -= buckets % rows
        if buckets < max(2, rows):
            continue
        bpw = div * buckets / (R * N)
        try:
            sk.sketch_layout(sk.params(nb * R, N, R, bpw, bits=4 if kind == "q4" else 16, rows=rows))
        except sk.SketchError:
            continue
        wk = str(g.choice(["f32", "bf16", "f16"]))
        rule = int(g.integers(0, 2))
        use_imp = bool(g.random() < 0.7)
        batch = int(g.choice([1, 3, 16, 17, 40, 300]))
        xk = "bf16" if batch > 16 and N % 8 == 0 else str(g.choice(["f32", "bf16", "f16"]))
        return dict(kind=kind, M=nb * R, N=N, R=R, bpw=bpw, rows=rows, wk=wk, rule=rule, imp=use_imp, batch=batch,
                    xk=xk, seed=int(g.integers(0, 2 ** 32)))
    raise RuntimeError("no valid configuration drawn")


def _weights(c):
    Wf = synth.normal_f32((c["M"], c["N"]), 0.05, c["seed"] % 100000)
    if c["wk"] == "f32":
        return Wf
    if c["wk"] == "bf16":
        return synth.bf16_bits(Wf)
    return Wf.astype(np.float16).view(np.uint16)


def _x(c):
    b, N = c["batch"], c["N"]
    if c["xk"] == "f32":
        return synth.normal_f32((b, N), 1.0, 7 + b)
    X = synth.normal_bf16((b, N), 7 + b)
    if c["xk"] == "f16":
        X = synth.bf16_to_f32(X).reshape(b, N).astype(np.float16).view(np.uint16)
    return X


@pytest.mark.parametrize("case_id", range(40))
def test_random_configuration(case_id):
    c = _draw(case_id)
    print("sweep case", case_id, c, flush=True)
    M, N, R, bpw, seed, rule = c["M"], c["N"], c["R"], c["bpw"], c["seed"], c["rule"]
    W = _weights(c)
    Wd = to_dev(W, c["wk"])
    imp = synth.uniform_f32(N, 0.5, 1.5, case_id) if c["imp"] else None
    impd = torch.from_numpy(imp).to(dev()) if imp is not None else None
    code = oracle_dtype(c["wk"])
    X = _x(c)
    xcode = oracle_dtype(c["xk"])
    rname = "absmin" if rule == 0 else "absmax"
    if c["kind"] == "uniform":
        t = sk.encode(Wd, impd, bpw=bpw, seed=seed, R=R, rule=rname)
        S = oracle.encode(W, imp, R, bpw, seed, rule, w_dtype=code)
        got = t.tables.cpu().numpy().view(np.uint16)
        Yr = oracle.matmul(S, X, M, N, R, bpw, seed, x_dtype=xcode)
    elif c["kind"] == "rows":
        t = sk.encode(Wd, impd, bpw=bpw, seed=seed, R=R, rule=rname, rows=c["rows"])
        S = oracle.encode(W, imp, R, bpw, seed, rule, w_dtype=code, rows=c["rows"])
        got = t.tables.cpu().numpy().view(np.uint16)
        Yr = oracle.matmul(S, X, M, N, R, bpw, seed, x_dtype=xcode, rows=c["rows"], rule=rule)
    elif c["kind"] == "alloc":
        a2 = synth.uniform_f32(N, 0.25, 4.0, case_id + 1)
        scores = sk.block_importance(Wd, torch.from_numpy(a2).to(dev()), R)
        alloc = sk.allocate(Wd, None, R=R, bpw=bpw, scores=scores)
        t = sk.encode(Wd, impd, bpw=bpw, seed=seed, R=R, rule=rname, alloc=alloc)
        bg = alloc.counts.numpy()
        S = oracle.encode_alloc(W, imp, R, bg, seed, rule, w_dtype=code)
        got = t.tables.cpu().numpy().view(np.uint16)
        Yr = oracle.matmul_alloc(S, X, M, N, R, bg, seed, x_dtype=xcode)
    else:
        t = sk.encode(Wd, impd, bpw=bpw, seed=seed, R=R, rule=rname, bits=4)
        T, sc = oracle.encode_q4(W, imp, R, bpw, seed, rule, w_dtype=code)
        nb, bg4, _ = sk.sketch_layout(t.params)
        raw = t.tables.cpu().numpy()
        off = ((nb * bg4 // 2 + 255) // 256) * 256
        assert np.array_equal(raw[off:off + 2 * nb].view(np.uint16), sc), "scales"
        got, S = raw[:nb * bg4 // 2], T.reshape(-1)
        Yr = oracle.matmul_q4(T, sc, X, M, N, R, bpw, seed, x_dtype=xcode)
    bad = int((got.reshape(-1) != S.reshape(-1)).sum())
    assert bad == 0, "%d of %d table entries differ" % (bad, S.size)
    Y = sk.matmul(t, to_dev(X, c["xk"])).cpu().numpy()
    assert_y_close(Y, Yr, what="sweep case %d" % case_id)


@pytest.mark.parametrize("kind", ["rows", "alloc", "q4"])
def test_graph_replay_of_the_other_sketch_kinds(kind):
    """encode + decode + batch-1 and 300-token products of a multi-row,
    allocated or 4-bit sketch captured in one HIP graph (the multi-row one
    with its K split and the launch that adds the parts): every replay (with
    eager work and synchronisations in between) reproduces the eager results
    bit for bit."""
    M, N, R = 1024, 2048, 8
    W = to_dev(synth.bf16_bits(synth.normal_f32((M, N), 0.02, 111)), "bf16")
    imp = torch.from_numpy(synth.uniform_f32(N, 0.5, 1.5, 112)).to(dev())
    kw = {"rows": {"rows": 2}, "q4": {"bits": 4},
          "alloc": {"alloc": sk.allocate(W, imp, R=R, bpw=0.5)}}[kind]
    ref = sk.encode(W, imp, bpw=0.5, R=R, **kw)
    x1 = to_dev(synth.normal_bf16((1, N), 113), "bf16")
    xT = to_dev(synth.normal_bf16((300, N), 114), "bf16")
    # the 300-token product with the workspace the call reports (the
    # multi-row product splits K with it), eager and captured alike
    wsb = sk.sketch_workspace_bytes(ref.params, 300, sk.BF16)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev()) if wsb else None
    assert (wsb > 0) == (kind == "rows")
    y1_ref, yT_ref = sk.matmul(ref, x1), sk.matmul(ref, xT, workspace=ws)
    d_ref = sk.decode(ref, torch.bfloat16)
    p = ref.params
    tables = torch.zeros_like(ref.tables)
    y1, yT, d = torch.zeros_like(y1_ref), torch.zeros_like(yT_ref), torch.zeros_like(d_ref)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sh = sk._stream_handle(dev())
        sk.sketch_encode(p, ref.proj, W, imp, tables, status, sh)
        sk.sketch_decode(p, ref.proj, tables, d, sh)
        sk.sketch_matmul(p, ref.proj, tables, x1, y1, None, sh)
        sk.sketch_matmul(p, ref.proj, tables, xT, yT, ws, sh)
    other = to_dev(synth.bf16_bits(synth.normal_f32((M, N), 0.02, 115)), "bf16")
    for rep in range(3):
        tables.zero_()
        y1.zero_()
        yT.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(tables, ref.tables), rep
        assert torch.equal(d, d_ref), rep
        assert torch.equal(y1, y1_ref), rep
        assert torch.equal(yT, yT_ref), rep
        sk.encode(other, None, bpw=0.5, R=R, **kw)    # eager work between replays
    assert int(status.item()) == 0
