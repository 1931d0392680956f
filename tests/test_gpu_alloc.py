"""GPU parity of the importance-aware space allocation ("Resumen Técnico" ›
Metodología §2) against the oracle: block importances within float32
summation error, bucket counts identical (the plan is one host computation
on the same scores), tables and decoded weights bit-exact, products within
the 1e-3 relative tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y_close, dev, oracle_dtype, to_dev

import sub_bit_weight_sketch_amd as sk

pytestmark = pytest.mark.gpu


def _w(shape, kind, seed, std=0.05):
    Wf = synth.normal_f32(shape, std, seed)
    if kind == "f32":
        return Wf
    if kind == "bf16":
        return synth.bf16_bits(Wf)
    return Wf.astype(np.float16).view(np.uint16)


def _tables(t):
    torch.cuda.synchronize()
    return t.tables.cpu().numpy().view(np.uint16)


def _bf16_rne_bits(f32):
    u = np.asarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _allocated(M, N, R, bpw, kind, seed, rule="absmin", lo=None, imp=True):
    """Encode on the GPU with counts planned from the GPU's block importances,
    and the oracle's tables for the same counts."""
    W = _w((M, N), kind, seed)
    a2 = synth.uniform_f32(N, 0.25, 4.0, seed + 1)
    Wd = to_dev(W, kind)
    scores = sk.block_importance(Wd, torch.from_numpy(a2).to(dev()), R)
    ref_scores = oracle.block_importance(W, a2, R, w_dtype=oracle_dtype(kind))
    np.testing.assert_allclose(scores.cpu().numpy().astype(np.float64), ref_scores, rtol=2e-5)
    alloc = sk.allocate(Wd, None, R=R, bpw=bpw, lo=lo, scores=scores)
    nb, Bg = oracle.layout(M, N, R, bpw)
    bg = oracle.alloc_plan(scores.cpu().numpy().astype(np.float64), nb * Bg, max(1, Bg // 4) if lo is None else lo)
    assert np.array_equal(alloc.counts.numpy(), bg)
    impv = synth.uniform_f32(N, 0.5, 1.5, seed + 2) if imp else None
    t = sk.encode(Wd, torch.from_numpy(impv).to(dev()) if imp else None, bpw=bpw, seed=seed, R=R, rule=rule,
                  alloc=alloc)
    orule = oracle.ABSMIN if rule == "absmin" else oracle.ABSMAX
    S = oracle.encode_alloc(W, impv, R, bg, seed, orule, w_dtype=oracle_dtype(kind))
    return W, t, S, bg


CASES = [
    # M, N, R, bpw, w kind
    (256, 512, 8, 0.5, "f32"),
    (272, 1024, 16, 0.5, "bf16"),
    (48, 100, 3, 16 * 25 / 300, "f32"),   # Bg = 25, N % 8 != 0: the scalar paths
    (96, 256, 32, 0.5, "f16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%d_R%d_%s" % (c[0], c[1], c[2], c[4]))
@pytest.mark.parametrize("rule", ["absmin", "absmax"])
def test_allocated_encode_decode_product(case, rule):
    M, N, R, bpw, kind = case
    W, t, S, bg = _allocated(M, N, R, bpw, kind, 11 + M, rule)
    assert len(set(bg.tolist())) > 1
    got = _tables(t)
    bad = int((got != S).sum())
    assert bad == 0, "%d of %d buckets differ" % (bad, S.size)
    ref = oracle.decode_alloc(S, M, N, R, bg, 11 + M)
    want = {torch.float16: ref.astype(np.float16).view(np.uint16),
            torch.float32: ref.astype(np.float32).view(np.uint32),
            torch.bfloat16: _bf16_rne_bits(ref.astype(np.float32))}
    for dt, bits in want.items():
        for hashed in (False, True):
            out = sk.decode(t, dt, hashed=hashed)
            torch.cuda.synchronize()
            g = out.view(torch.int32 if dt == torch.float32 else torch.int16).cpu().numpy()
            g = g.view(np.uint32 if dt == torch.float32 else np.uint16)
            assert int((g != bits).sum()) == 0, (dt, hashed)
    batches = [(1, "f32"), (5, "bf16"), (16, "f16")]
    if kind == "bf16" and N % 8 == 0:
        batches += [(17, "bf16"), (300, "bf16")]
    for b, xk in batches:
        X = synth.normal_f32((b, N), 1.0, b) if xk == "f32" else synth.normal_bf16((b, N), b)
        if xk == "f16":
            X = synth.bf16_to_f32(X).reshape(b, N).astype(np.float16).view(np.uint16)
        Y = sk.matmul(t, to_dev(X, xk)).cpu().numpy()
        Yr = oracle.matmul_alloc(S, X, M, N, R, bg, 11 + M, x_dtype=oracle_dtype(xk))
        assert_y_close(Y, Yr, what="allocated %s batch %d %s" % (case, b, xk))


def test_uniform_counts_reproduce_the_uniform_sketch():
    """Every block at the uniform count: the allocated path's tables, decode
    and products equal the uniform sketch's (two independent GPU paths)."""
    M, N, R, bpw = 512, 1024, 8, 0.5
    W = to_dev(_w((M, N), "bf16", 5), "bf16")
    nb, Bg = oracle.layout(M, N, R, bpw)
    alloc = sk.Allocation(torch.arange(nb + 1, dtype=torch.int64) * Bg, Bg, dev())
    ta = sk.encode(W, None, bpw=bpw, R=R, alloc=alloc)
    tu = sk.encode(W, None, bpw=bpw, R=R)
    assert torch.equal(ta.tables.view(-1), tu.tables.view(-1))
    assert torch.equal(sk.decode(ta, torch.float32), sk.decode(tu, torch.float32))
    for b in (1, 64):
        X = to_dev(synth.normal_bf16((b, N), 3), "bf16")
        Ya, Yu = sk.matmul(ta, X), sk.matmul(tu, X)
        assert_y_close(Ya.cpu().numpy(), Yu.cpu().numpy().astype(np.float64), what="uniform counts batch %d" % b)


@pytest.mark.parametrize("T", [1, 2048])
def test_attention_shape_allocated(T):
    """attn_4096x4096 with counts from its block importances: tables
    bit-exact; the batch-1 product in full, the 2048-token product on 16
    tokens x 256 sampled outputs."""
    M = N = 4096
    W = synth.student_t_bf16((M, N), 0.02, 61)
    Wd = to_dev(W, "bf16")
    a2 = synth.uniform_f32(N, 0.25, 4.0, 62)
    scores = sk.block_importance(Wd, torch.from_numpy(a2).to(dev()), 8)
    alloc = sk.allocate(Wd, None, R=8, bpw=0.5, scores=scores)
    bg = alloc.counts.numpy()
    t = sk.encode(Wd, None, bpw=0.5, seed=1, R=8, alloc=alloc)
    S = oracle.encode_alloc(W, None, 8, bg, 1, w_dtype=oracle.BF16)
    assert int((_tables(t) != S).sum()) == 0
    X = synth.normal_bf16((T, N), 63)
    Y = sk.matmul(t, to_dev(X, "bf16")).cpu().numpy()
    if T == 1:
        assert_y_close(Y, oracle.matmul_alloc(S, X, M, N, 8, bg, 1, x_dtype=oracle.BF16), what="attention b1")
        return
    g = np.random.default_rng(64)
    toks = g.choice(T, size=16, replace=False)
    ti = np.repeat(toks, 256)
    ii = g.integers(0, M, size=ti.size)
    ys = oracle.matmul_sampled_alloc(S, X, M, N, 8, bg, ti, ii, 1, x_dtype=oracle.BF16)
    rms = np.sqrt((ys.reshape(16, 256) ** 2).mean(axis=1))
    assert_y_close(Y[ti, ii].reshape(16, 256), ys.reshape(16, 256), row_rms=rms[:, None], what="attention T2048")


def test_invalid_block_counts_are_flagged_and_give_nan_rows():
    """Offsets with an empty block (count 0) and one above bg_max: encode
    sets FLAG_ALLOCATION, decode and both product paths give NaN exactly for
    those blocks' rows and the oracle's values elsewhere."""
    M, N, R, bpw = 64, 512, 8, 0.5
    W = _w((M, N), "bf16", 71)
    Wd = to_dev(W, "bf16")
    nb, Bg = oracle.layout(M, N, R, bpw)
    counts = np.full(nb, Bg)
    counts[2], counts[3] = 0, 2 * Bg          # block 2 empty, block 3 over the stated maximum
    off = np.concatenate([[0], np.cumsum(counts)])
    alloc = sk.Allocation(torch.from_numpy(off), Bg + 8, dev())
    p = sk.params(M, N, R, bpw, 1, sk.ABSMIN, sk.BF16, alloc=alloc)
    proj = sk.projection(p, dev())
    tables = torch.zeros(nb * Bg, dtype=torch.int16, device=dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    sk.sketch_encode(p, proj, Wd, None, tables, status)
    torch.cuda.synchronize()
    assert int(status.item()) & sk.FLAG_ALLOCATION
    t = sk.Tables(p, tables, proj, alloc)
    bad_rows = np.zeros(M, bool)
    bad_rows[2 * R:4 * R] = True
    D = sk.decode(t, torch.float32).cpu().numpy()
    assert np.isnan(D[bad_rows]).all() and not np.isnan(D[~bad_rows]).any()
    # the other blocks against the oracle: its counts are the same with the
    # bad blocks at 1 bucket, so its table of block b sits at its own offset
    bg_or = counts.copy()
    bg_or[2], bg_or[3] = 1, 1
    off_or = np.concatenate([[0], np.cumsum(bg_or)])
    S_or = oracle.encode_alloc(W, None, R, bg_or, 1, w_dtype=oracle.BF16)
    S_gpu = tables.cpu().numpy().view(np.uint16)
    for b_ in range(nb):
        if b_ in (2, 3):
            continue
        assert np.array_equal(S_gpu[off[b_]:off[b_ + 1]], S_or[off_or[b_]:off_or[b_ + 1]]), b_
    for b in (1, 40):
        X = synth.normal_bf16((b, N), 72)
        Y = sk.matmul(t, to_dev(X, "bf16")).cpu().numpy()
        assert np.isnan(Y[:, bad_rows]).all(), b
        Yr = oracle.matmul_alloc(S_or, X, M, N, R, bg_or, 1, x_dtype=oracle.BF16)
        assert_y_close(Y[:, ~bad_rows], Yr[:, ~bad_rows], what="valid blocks, batch %d" % b)


def test_allocated_sketch_with_a_uniform_projection_is_nan():
    """A uniform projection (larger than the hash projection, so every read
    stays inside it) used for an allocated sketch: encode flags it, decode
    and products are NaN."""
    M, N, R = 64, 512, 8
    Wd = to_dev(_w((M, N), "bf16", 81), "bf16")
    alloc = sk.allocate(Wd, torch.ones(N, device=dev()), R=R, bpw=0.5)
    p = sk.params(M, N, R, 0.5, 1, sk.ABSMIN, sk.BF16, alloc=alloc)
    uniform = sk.projection(sk.params(M, N, R, 0.5, 1, sk.ABSMIN, sk.BF16), dev())
    assert uniform.numel() >= sk.sketch_projection_bytes(p)
    tables = torch.zeros(M // R * 128, dtype=torch.int16, device=dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    sk.sketch_encode(p, uniform, Wd, None, tables, status)
    torch.cuda.synchronize()
    assert int(status.item()) & sk.FLAG_PROJECTION
    t = sk.Tables(p, tables, uniform, alloc)
    assert bool(torch.isnan(sk.decode(t, torch.float32)).all())
    for b in (1, 40):
        Y = sk.matmul(t, to_dev(synth.normal_bf16((b, N), 82), "bf16"))
        torch.cuda.synchronize()
        assert bool(torch.isnan(Y).all()), b
