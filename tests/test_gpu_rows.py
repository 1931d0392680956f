"""GPU parity of the multi-row AbsMaxMin sketch ("Resumen Técnico" ›
Metodología §1, multi-row design) against the oracle: tables bit-exact,
decoded weights bit-exact, products within the 1e-3 relative tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_tables_equal, assert_y_close, dev, oracle_dtype, tables_np, to_dev

import sub_bit_weight_sketch_amd as sk

pytestmark = pytest.mark.gpu

RULES = [("absmin", oracle.ABSMIN), ("absmax", oracle.ABSMAX)]

CASES = [
    # M, N, R, bpw, rows, w_kind
    (256, 512, 8, 0.5, 2, "f32"),
    (4096, 4096, 8, 0.5, 4, "bf16"),       # the attention shape, 4 rows of 256 buckets
    (272, 1024, 16, 0.5, 2, "bf16"),
    (48, 100, 3, 16 * 25 / 300, 5, "f32"),  # Bg = 25 in 5 rows of 5, N % 8 != 0
    (96, 256, 32, 0.5, 4, "f16"),
]


def _w(shape, kind, seed):
    Wf = synth.normal_f32(shape, 0.05, seed)
    if kind == "f32":
        return Wf
    if kind == "bf16":
        return synth.bf16_bits(Wf)
    return Wf.astype(np.float16).view(np.uint16)


def _bf16_rne_bits(f32):
    u = np.asarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%d_R%d_rows%d_%s" % (c[0], c[1], c[2], c[4], c[5]))
@pytest.mark.parametrize("rule_name,rule", RULES)
def test_multi_row_encode_decode_product(case, rule_name, rule):
    M, N, R, bpw, rows, kind = case
    W = _w((M, N), kind, 100 + M + rows)
    imp = synth.uniform_f32(N, 0.5, 1.5, 200 + N)
    t = sk.encode(to_dev(W, kind), torch.from_numpy(imp).to(dev()), bpw=bpw, seed=4, R=R, rule=rule_name, rows=rows)
    S = oracle.encode(W, imp, R, bpw, 4, rule, w_dtype=oracle_dtype(kind), rows=rows)
    assert_tables_equal(tables_np(t), S, "multi-row %s %s" % (case, rule_name))
    # decoded weights, every output dtype, both methods
    ref = oracle.decode(S, M, N, R, bpw, 4, rows=rows, rule=rule)
    want = {torch.float16: ref.astype(np.float16).view(np.uint16),
            torch.float32: ref.astype(np.float32).view(np.uint32),
            torch.bfloat16: _bf16_rne_bits(ref.astype(np.float32))}
    for dt, bits in want.items():
        for hashed in (False, True):
            got = sk.decode(t, dt, hashed=hashed)
            torch.cuda.synchronize()
            g = got.view(torch.int32 if dt == torch.float32 else torch.int16).cpu().numpy()
            g = g.view(np.uint32 if dt == torch.float32 else np.uint16)
            bad = int((g != bits).sum())
            assert bad == 0, "%s %s hashed=%s: %d of %d differ" % (case, dt, hashed, bad, bits.size)
    # products: the decode-per-weight GEMV passes, and the bf16 matrix-core path
    batches = [(1, "f32"), (5, "bf16"), (16, "f16")]
    if kind == "bf16" and N % 8 == 0:
        batches += [(17, "bf16"), (130, "bf16")]
    for b, xk in batches:
        if xk == "f32":
            X = synth.normal_f32((b, N), 1.0, b)
        else:
            X = synth.normal_bf16((b, N), b)
            if xk == "f16":
                X = synth.bf16_to_f32(X).reshape(b, N).astype(np.float16).view(np.uint16)
        if M * N > 1 << 22 and b > 5:
            continue   # the full attention shape: batch 1 and 5 only (oracle time)
        Y = sk.matmul(t, to_dev(X, xk)).cpu().numpy()
        Yr = oracle.matmul(S, X, M, N, R, bpw, 4, x_dtype=oracle_dtype(xk), rows=rows, rule=rule)
        assert_y_close(Y, Yr, what="multi-row %s batch %d %s" % (case, b, xk))


def test_multi_row_projection_mismatch():
    """A single-row projection (larger than the multi-row one, so every read
    stays inside it) used for a multi-row sketch: encode flags it, products
    and decode are NaN."""
    M, N = 64, 512
    W = to_dev(_w((M, N), "bf16", 7), "bf16")
    p = sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.BF16, rows=2)
    single = sk.projection(sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.BF16), dev())
    assert single.numel() >= sk.sketch_projection_bytes(p)
    tables = torch.empty((M // 8, 128), dtype=torch.int16, device=dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    sk.sketch_encode(p, single, W, None, tables, status)
    assert int(status.item()) & sk.FLAG_PROJECTION
    good = sk.encode(W, None, bpw=0.5, R=8, rows=2)
    bad = sk.Tables(good.params, good.tables, single)
    for b in (1, 17):
        Y = sk.matmul(bad, to_dev(synth.normal_bf16((b, N), 3), "bf16"))
        torch.cuda.synchronize()
        assert bool(torch.isnan(Y).all()), b
    assert bool(torch.isnan(sk.decode(bad, torch.float32)).all())


GEMM_CASES = [
    # M, N, R, bpw, rows, T: several 256-token tiles with ragged tails, one or
    # several 32-column chunks with a ragged last chunk, ragged output tiles
    (200, 40, 8, 0.5, 2, 300),
    (136, 16, 8, 0.5, 2, 257),
    (384, 1000, 16, 0.5, 4, 520),
    (264, 96, 8, 0.5, 3, 270),
    (128, 512, 4, 0.75, 2, 768),
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "%dx%d_R%d_rows%d_T%d" % (c[0], c[1], c[2], c[4], c[5]))
@pytest.mark.parametrize("rule_name,rule", RULES)
def test_multi_row_gemm_tiles(case, rule_name, rule):
    """The bf16 matrix-core product of a multi-row sketch against the oracle,
    element by element."""
    M, N, R, bpw, rows, T = case
    W = _w((M, N), "bf16", 300 + M)
    t = sk.encode(to_dev(W, "bf16"), None, bpw=bpw, seed=6, R=R, rule=rule_name, rows=rows)
    S = oracle.encode(W, None, R, bpw, 6, rule, w_dtype=oracle.BF16, rows=rows)
    assert_tables_equal(tables_np(t), S, "multi-row %s" % (case,))
    X = synth.normal_bf16((T, N), 400 + T)
    Y = sk.matmul(t, to_dev(X, "bf16")).cpu().numpy()
    Yr = oracle.matmul(S, X, M, N, R, bpw, 6, x_dtype=oracle.BF16, rows=rows, rule=rule)
    assert_y_close(Y, Yr, what="multi-row gemm %s" % (case,))


@pytest.mark.parametrize("rows", [2, 4])
def test_multi_row_gemm_attention_2048_tokens_sampled(rows):
    """The attention projection 4096x4096 at 2048 tokens through the
    multi-row bf16 matrix-core product (the launch the micro-benchmark
    times), checked on 4096 sampled outputs against the oracle, both with the
    workspace sketch_workspace_bytes reports (K split in two, the parts added
    by a second launch) and without it (unsplit); the two agree to float32
    accumulation rounding."""
    M = N = 4096
    W = synth.student_t_bf16((M, N), 0.02, 71)
    t = sk.encode(to_dev(W, "bf16"), None, bpw=0.5, seed=1, R=8, rows=rows)
    S = oracle.encode(W, None, 8, 0.5, 1, oracle.ABSMIN, w_dtype=oracle.BF16, rows=rows)
    assert_tables_equal(tables_np(t), S, "attention rows %d" % rows)
    X = synth.normal_bf16((2048, N), 72)
    Y = sk.matmul(t, to_dev(X, "bf16")).cpu().numpy()
    g = np.random.default_rng(73)
    toks = g.choice(2048, size=16, replace=False)
    ti = np.repeat(toks, 256)
    ii = g.integers(0, M, size=ti.size)
    ys = oracle.matmul_sampled(S, X, M, N, 8, 0.5, ti, ii, 1, x_dtype=oracle.BF16, rows=rows)
    rms = np.sqrt((ys.reshape(16, 256) ** 2).mean(axis=1))
    assert_y_close(Y[ti, ii].reshape(16, 256), ys.reshape(16, 256), row_rms=rms[:, None],
                   what="attention rows %d sampled" % rows)
    assert sk.sketch_workspace_bytes(t.params, 2048, sk.BF16) == 2048 * M * 4
    Xd = to_dev(X, "bf16")
    Yu = torch.full((2048, M), float("nan"), dtype=torch.float32, device=dev())
    sk.sketch_matmul(t.params, t.proj, t.tables, Xd, Yu, None)   # no workspace: unsplit
    Yu = Yu.cpu().numpy()
    assert_y_close(Yu[ti, ii].reshape(16, 256), ys.reshape(16, 256), row_rms=rms[:, None],
                   what="attention rows %d sampled, unsplit" % rows)
    full_rms = np.sqrt((Yu.astype(np.float64) ** 2).mean(axis=1))
    assert np.all(np.abs(Y - Yu) <= 1e-5 * full_rms[:, None]), "split and unsplit differ beyond rounding"
    Y2 = sk.matmul(t, Xd).cpu().numpy()   # the split form gives the same bits on every call
    assert np.array_equal(Y, Y2)
