"""Pins of the oracle's multi-row AbsMaxMin sketch ("Resumen Técnico" ›
Metodología §1, multi-row design: several independent hash functions, each
with its own sketch row, and the Max over the rows at decompression).

Readings under test: row rho hashes with seed + rho into its own segment of
Bg/rows buckets of the block; each row keeps the single-row winner of its
segment; decode takes the candidate of largest magnitude (AbsMin; smallest
for AbsMax), the first row among equal magnitudes.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from oracle import oracle as orc


def _w(M, N, seed, kind="f32"):
    W = synth.normal_f32((M, N), 0.1, seed)
    if kind == "bf16":
        return synth.bf16_bits(W), oracle.BF16
    return W, oracle.F32


def test_rows_one_is_the_single_row_sketch():
    """rows = 1 through the multi-row functions gives the single-row results bit for bit."""
    L = orc._load()
    for (M, N, R, bpw, rule, seed) in [(32, 256, 8, 0.5, oracle.ABSMIN, 1), (30, 100, 3, 16 * 25 / 300, oracle.ABSMAX, 7),
                                       (64, 128, 16, 0.75, oracle.ABSMIN, 3)]:
        W, code = _w(M, N, M + N)
        imp = synth.uniform_f32(N, 0.5, 1.5, N)
        nb, Bg = oracle.layout(M, N, R, bpw)
        S_rows = np.zeros((nb, Bg), dtype=np.uint16)
        rc = L.oracle_encode_rows(M, N, R, bpw, seed, rule, 1, code, orc._ptr(W), orc._ptr(imp), orc._ptr(S_rows), 0)
        assert rc == 0
        S = oracle.encode(W, imp, R, bpw, seed, rule, w_dtype=code)
        assert np.array_equal(S_rows, S)
        D_rows = np.empty((M, N))
        assert L.oracle_decode_rows(M, N, R, bpw, seed, rule, 1, orc._ptr(S), orc._ptr(D_rows)) == 0
        assert np.array_equal(D_rows, oracle.decode(S, M, N, R, bpw, seed))
        X = synth.normal_f32((3, N), 1.0, 5)
        Y_rows = np.empty((3, M))
        assert L.oracle_matmul_rows(M, N, R, bpw, seed, rule, 1, orc._ptr(S), orc._ptr(X), oracle.F32, 3,
                                    orc._ptr(Y_rows), 0) == 0
        assert np.array_equal(Y_rows, oracle.matmul(S, X, M, N, R, bpw, seed))


@pytest.mark.parametrize("rows", [2, 4])
@pytest.mark.parametrize("rule", [oracle.ABSMIN, oracle.ABSMAX])
def test_each_row_is_an_independent_single_row_sketch(rows, rule):
    """Segment rho of a rows-row table is the single-row sketch of the same
    weights with Bg/rows buckets and seed + rho."""
    M, N, R, bpw, seed = 32, 256, 8, 0.5, 11
    W, code = _w(M, N, 21, "bf16")
    imp = synth.uniform_f32(N, 0.5, 1.5, 22)
    nb, Bg = oracle.layout(M, N, R, bpw)
    S = oracle.encode(W, imp, R, bpw, seed, rule, w_dtype=code, rows=rows)
    Bgr = Bg // rows
    for rho in range(rows):
        single = oracle.encode(W, imp, R, bpw / rows, seed + rho, rule, w_dtype=code)
        assert single.shape == (nb, Bgr)
        assert np.array_equal(S[:, rho * Bgr:(rho + 1) * Bgr], single), "row %d" % rho


def test_multi_row_decode_brute_force():
    """Decode of a tiny multi-row table against a direct NumPy pick of the
    largest-magnitude candidate (first row on ties)."""
    for rows, M, N, R, bpw in [(2, 8, 32, 4, 0.5), (3, 6, 48, 2, 1.0), (4, 16, 64, 8, 0.5)]:
        W, code = _w(M, N, 31 + rows)
        S = oracle.encode(W, None, R, bpw, 9, oracle.ABSMIN, w_dtype=code, rows=rows)
        nb, Bg = oracle.layout(M, N, R, bpw)
        Bgr = Bg // rows
        D = oracle.decode(S, M, N, R, bpw, 9, rows=rows)
        for i in range(M):
            for j in range(N):
                l = (i % R) * N + j
                cand = [oracle.f16_to_f64(int(S[i // R, rho * Bgr + oracle.bucket(l, 9 + rho, Bgr)]))
                        for rho in range(rows)]
                best = cand[0]
                for v in cand[1:]:
                    if abs(v) > abs(best):
                        best = v
                assert D[i, j] == best


def test_multi_row_bound_and_max_over_rows():
    """With all-ones importance every decoded weight is one of its rows'
    buckets, at most |binary16(w)| in magnitude (the underestimation bound),
    and at least as large in magnitude as each single row's bucket."""
    M, N, R, bpw, rows = 64, 512, 8, 0.5, 2
    W = synth.normal_f32((M, N), 0.1, 41)
    S = oracle.encode(W, None, R, bpw, 1, oracle.ABSMIN, rows=rows)
    D = oracle.decode(S, M, N, R, bpw, 1, rows=rows)
    w16 = oracle.f32_to_f16_array(W).view(np.float16).astype(np.float64)
    assert np.all(np.abs(D) <= np.abs(w16))
    nb, Bg = oracle.layout(M, N, R, bpw)
    Bgr = Bg // rows
    for rho in range(rows):
        seg = np.ascontiguousarray(S[:, rho * Bgr:(rho + 1) * Bgr])
        Drho = oracle.decode(seg, M, N, R, bpw / rows, 1 + rho)
        assert np.all(np.abs(D) >= np.abs(Drho))
    assert np.all(np.isin(D, np.concatenate([oracle.decode(np.ascontiguousarray(S[:, r * Bgr:(r + 1) * Bgr]), M, N,
                                                                      R, bpw / rows, 1 + r) for r in range(rows)])))


def test_multi_row_absmax_picks_the_smallest_magnitude():
    M, N, R, bpw, rows = 16, 128, 8, 0.5, 2
    W = synth.normal_f32((M, N), 0.1, 43)
    S = oracle.encode(W, None, R, bpw, 1, oracle.ABSMAX, rows=rows)
    D = oracle.decode(S, M, N, R, bpw, 1, rows=rows, rule=oracle.ABSMAX)
    w16 = oracle.f32_to_f16_array(W).view(np.float16).astype(np.float64)
    assert np.all(np.abs(D) >= np.abs(w16))   # each AbsMax bucket holds a collider of at least |w|


def test_multi_row_product_is_the_dense_product():
    """Y = X . W_hat^T from the multi-row oracle against np.matmul on its W_hat."""
    M, N, R, bpw, rows = 48, 256, 8, 0.75, 3
    W, code = _w(M, N, 51, "bf16")
    S = oracle.encode(W, None, R, bpw, 2, oracle.ABSMIN, w_dtype=code, rows=rows)
    D = oracle.decode(S, M, N, R, bpw, 2, rows=rows)
    X = synth.normal_f32((5, N), 1.0, 52)
    Y = oracle.matmul(S, X, M, N, R, bpw, 2, rows=rows)
    ref = np.matmul(X.astype(np.float64), D.T)
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    t = np.array([0, 4, 2]); i = np.array([0, 47, 13])
    ys = oracle.matmul_sampled(S, X, M, N, R, bpw, t, i, 2, rows=rows)
    assert np.array_equal(ys, Y[t, i])


def test_multi_row_rejections():
    W = synth.normal_f32((16, 64), 0.1, 61)
    with pytest.raises(oracle.OracleError):          # Bg = 32 does not split into 3 rows
        oracle.encode(W, None, 8, 0.5, rows=3)
    with pytest.raises(oracle.OracleError):
        oracle.encode(W, None, 8, 0.5, rows=0)
    with pytest.raises(oracle.OracleError):
        oracle.decode(np.zeros((2, 32), np.uint16), 16, 64, 8, 0.5, rows=3)


def test_multi_row_ties_go_to_the_first_row():
    """Weights of one magnitude and random signs: every bucket of every row
    holds +c or -c, all candidates tie in magnitude, and the decode is row
    0's bucket for every position."""
    M, N, R, bpw, rows = 16, 128, 8, 0.5, 4
    g = np.random.default_rng(71)
    W = np.where(g.random((M, N)) < 0.5, -0.25, 0.25).astype(np.float32)
    S = oracle.encode(W, None, R, bpw, 3, oracle.ABSMIN, rows=rows)
    D = oracle.decode(S, M, N, R, bpw, 3, rows=rows)
    nb, Bg = oracle.layout(M, N, R, bpw)
    row0 = oracle.decode(np.ascontiguousarray(S[:, :Bg // rows]), M, N, R, bpw / rows, 3)
    assert np.array_equal(D, row0)
    assert set(np.unique(np.abs(D))) == {0.25}
