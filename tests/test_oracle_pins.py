"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the bit
budget, published hash vectors, NumPy's binary16 conversion, an independent
set-based brute force on tiny matrices, invariants the method guarantees
(underestimation bound, membership), special cases with closed forms, and the
matrix identity W_hat = S * P^T with an explicit one-hot P.

Citations: "UltraSketchLLM: Sub-1-Bit LLM Compression via Sketch and
Hardware-Friendly Operators", gist.science explainer ("Resumen Técnico";
Dutch twin "Technische Samenvatting").
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, HealthCheck
from hypothesis import strategies as st

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# ---------------------------------------------------------------------------
# independent helpers (no oracle code): the hash written from its published
# description, and NumPy's own binary16 conversion
# ---------------------------------------------------------------------------
_M32 = 0xFFFFFFFF


def py_fmix32(h):
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & _M32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & _M32
    h ^= h >> 16
    return h


def py_bucket(l, seed, Bg):
    u = ((l * 0x9E3779B1) & _M32) ^ seed
    return (py_fmix32(u) * Bg) >> 32


def np_f16_bits(f32):
    return np.asarray(f32, dtype=np.float32).astype(np.float16).view(np.uint16)


def brute_encode(Wf, imp, R, Bg, seed, rule):
    """Set-based resolution: for every bucket, the collider set, then the
    extreme key (ties: smallest local index).  Keys are one float32 multiply."""
    M, N = Wf.shape
    kmap = [py_bucket(l, seed, Bg) for l in range(R * N)]
    S = np.zeros((M // R, Bg), dtype=np.uint16)
    for b in range(M // R):
        block = Wf[b * R:(b + 1) * R]
        keys = {}
        for l in range(R * N):
            r, j = divmod(l, N)
            keys[l] = np.float32(abs(block[r, j])) * np.float32(1.0 if imp is None else imp[j])
        for q in range(Bg):
            coll = [l for l in range(R * N) if kmap[l] == q]
            if not coll:
                continue
            if rule == oracle.ABSMIN:
                win = min(coll, key=lambda l: (keys[l], l))
            else:
                win = min(coll, key=lambda l: (-keys[l], l))
            r, j = divmod(win, N)
            S[b, q] = np_f16_bits(block[r, j])
    return S


# ---------------------------------------------------------------------------
# bit budget
# ---------------------------------------------------------------------------

def test_bpw_accounting_golden():
    cases = json.load(open(os.path.join(GOLDEN, "bpw_accounting.json")))["cases"]
    for c in cases:
        nb, Bg = oracle.layout(c["M"], c["N"], c["R"], c["bpw"])
        assert (nb, Bg) == (c["num_blocks"], c["Bg"]), c["name"]
        assert nb * Bg == c["total_buckets"], c["name"]
        # every bucket is 16 bits: table bits equal the budget exactly
        assert nb * Bg * 16 == c["bpw"] * c["M"] * c["N"], c["name"]
        if c["bpw"] == 0.5:
            assert c["R"] * c["N"] == 32 * Bg, c["name"]   # one bucket per 32 weights


@pytest.mark.parametrize("args", [(10, 64, 3, 0.5), (16, 64, 8, 0.3), (16, 0, 8, 0.5), (16, 64, 0, 0.5),
                                  (16, 64, 8, 0.0), (16, 64, 8, float("nan")), (16, 3, 1, 0.5)])
def test_layout_rejects(args):
    with pytest.raises(oracle.OracleError):
        oracle.layout(*args)


def test_layout_empty_rows_ok():
    assert oracle.layout(0, 64, 8, 0.5) == (0, 16)


# ---------------------------------------------------------------------------
# hash
# ---------------------------------------------------------------------------

def _murmur3_x86_32(data, seed):
    """MurmurHash3_x86_32 body; the finalizer is the oracle's hash32."""
    c1, c2 = 0xCC9E2D51, 0x1B873593

    def rotl(x, r):
        return ((x << r) | (x >> (32 - r))) & _M32

    h = seed
    nblocks = len(data) // 4
    for i in range(nblocks):
        k = int.from_bytes(data[4 * i:4 * i + 4], "little")
        k = (k * c1) & _M32
        k = rotl(k, 15)
        k = (k * c2) & _M32
        h ^= k
        h = rotl(h, 13)
        h = (h * 5 + 0xE6546B64) & _M32
    tail = data[4 * nblocks:]
    k = 0
    if len(tail) >= 3:
        k ^= tail[2] << 16
    if len(tail) >= 2:
        k ^= tail[1] << 8
    if len(tail) >= 1:
        k ^= tail[0]
        k = (k * c1) & _M32
        k = rotl(k, 15)
        k = (k * c2) & _M32
        h ^= k
    h ^= len(data)
    return oracle.hash32(h)


def test_hash32_published_murmur3_vectors():
    vecs = json.load(open(os.path.join(GOLDEN, "murmur3_vectors.json")))["vectors"]
    for v in vecs:
        data = bytes.fromhex(v["hex"]) if "hex" in v else v["text"].encode("utf-8")
        assert _murmur3_x86_32(data, v["seed"]) == int(v["hash"], 16), v


def test_hash32_is_a_bijection_on_a_sample():
    # every step of the finalizer is invertible, so distinct inputs never collide
    xs = np.random.default_rng(7).choice(2**32, size=200000, replace=False)
    hs = {oracle.hash32(int(x)) for x in xs[:20000]}
    assert len(hs) == 20000


def test_bucket_power_of_two_is_top_bits():
    # multiply-high range reduction with Bg = 2^m keeps the top m bits of the hash
    for m in (0, 1, 5, 10, 12):
        Bg = 1 << m
        for l in range(0, 5000, 7):
            h = oracle.hash32(((l * 0x9E3779B1) & _M32) ^ 1)
            assert oracle.bucket(l, 1, Bg) == h >> (32 - m)


def test_bucket_map_matches_independent_hash():
    for (R, N, seed, Bg) in [(8, 512, 1, 128), (16, 100, 3, 37), (1, 1000, 0xFFFFFFFF, 2752)]:
        km = oracle.bucket_map(R, N, seed, Bg)
        ref = np.array([py_bucket(l, seed, Bg) for l in range(R * N)], dtype=np.uint32)
        np.testing.assert_array_equal(km, ref)
        assert km.max() < Bg


def test_bucket_loads_are_poisson_like():
    # 32 weights per bucket at 0.5 bpw; chi-square of bucket loads vs uniform
    R, N, Bg = 8, 4096, 1024
    km = oracle.bucket_map(R, N, 1, Bg)
    counts = np.bincount(km, minlength=Bg)
    expect = R * N / Bg
    chi2 = ((counts - expect) ** 2 / expect).sum()
    # dof = 1023; mean 1023, sd ~45; generous 6-sigma window
    assert abs(chi2 - (Bg - 1)) < 6 * math.sqrt(2 * (Bg - 1))
    # a different seed gives a different map
    assert (oracle.bucket_map(R, N, 2, Bg) != km).mean() > 0.99


# ---------------------------------------------------------------------------
# binary16 conversions
# ---------------------------------------------------------------------------

def test_f32_to_f16_all_bf16_patterns():
    f = (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(over="ignore"):
        ref = np_f16_bits(f)
    got = oracle.f32_to_f16_array(f)
    nan = np.isnan(f)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_f32_to_f16_random_and_boundary_patterns():
    g = np.random.default_rng(11)
    u = g.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # dense sweeps: around the subnormal/normal seam, near halfway points, near overflow
    seam = np.arange(0x33000000 - 4096, 0x38800000 + 4096, 97, dtype=np.uint32)
    top = np.arange(0x477FE000, 0x47801000, 1, dtype=np.uint32)
    u = np.concatenate([u, seam, seam | 0x80000000, top, top | 0x80000000])
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    with np.errstate(over="ignore"):
        ref = np_f16_bits(f)
    np.testing.assert_array_equal(oracle.f32_to_f16_array(f), ref)


def test_f16_to_f64_all_patterns():
    h = np.arange(65536, dtype=np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(x)) for x in h])
    nan = np.isnan(ref)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(got[nan]))


def test_bf16_to_f16_to_bf16_is_lossless():
    """Every finite bfloat16 of magnitude below 65520, rounded to binary16, is
    again a bfloat16 value: buckets of bfloat16 weights can feed a bfloat16
    matrix core without further rounding."""
    f = (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(np.float32)
    ok = np.isfinite(f) & (np.abs(f) < 65520)
    h = oracle.f32_to_f16_array(f[ok])
    back = h.view(np.float16).astype(np.float32)
    assert np.all((back.view(np.uint32) & 0xFFFF) == 0)
    changed = back != f[ok]
    assert np.all(np.abs(f[ok][changed]) < 2.0 ** -17)


# ---------------------------------------------------------------------------
# encode: brute force, invariants, special cases
# ---------------------------------------------------------------------------

def _special_values(g, n):
    pool = np.array([0.0, -0.0, 1e-8, -1e-8, 6e-8, 0.5, -0.5, 0.25, 1.0, -1.0, 3.0, 65504.0, -65519.0,
                     2.0 ** -24, 2.0 ** -25, 1e-40], dtype=np.float32)
    return pool[g.integers(0, pool.size, size=n)]


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.integers(1, 4), st.integers(1, 4), st.integers(1, 24), st.sampled_from([1, 2, 3, 5, 8, 16]),
       st.integers(0, 2**32 - 1), st.sampled_from([oracle.ABSMIN, oracle.ABSMAX]),
       st.booleans(), st.integers(0, 2**31), st.sampled_from(["f32", "bf16", "f16", "special"]))
def test_encode_matches_brute_force(nblk, R, N, bpr, seed, rule, use_imp, dseed, kind):
    """Tiny matrices: the oracle's sequential scan equals the set-based brute force."""
    M = nblk * R
    Bg = bpr                                   # buckets per block; bpw = 16*Bg/(R*N)
    bpw = 16.0 * Bg / (R * N)
    g = np.random.default_rng(dseed)
    if kind == "special":
        Wf = _special_values(g, M * N).reshape(M, N)
    else:
        Wf = (g.standard_normal((M, N)) * g.choice([1e-3, 1.0, 100.0])).astype(np.float32)
        if g.random() < 0.3:                   # force exact ties
            Wf = np.round(Wf)
    imp = None
    if use_imp:
        imp = g.choice(np.array([0.0, 0.5, 1.0, 2.0, 1.25], dtype=np.float32), size=N)
    if kind == "bf16":
        Wb = synth.bf16_bits(Wf)
        Wf = synth.bf16_to_f32(Wb).reshape(M, N)
        S = oracle.encode(Wb, imp, R, bpw, seed, rule, w_dtype=oracle.BF16)
    elif kind == "f16":
        Wh = np.clip(Wf, -65504, 65504).astype(np.float16)
        Wf = Wh.astype(np.float32)
        S = oracle.encode(Wh.view(np.uint16), imp, R, bpw, seed, rule, w_dtype=oracle.F16)
    else:
        S = oracle.encode(Wf, imp, R, bpw, seed, rule)
    np.testing.assert_array_equal(S, brute_encode(Wf, imp, R, Bg, seed, rule))


def _members(Wf, R, Bg, seed):
    """For every (block, bucket), the set of binary16 patterns of its colliders."""
    M, N = Wf.shape
    km = oracle.bucket_map(R, N, seed, Bg)
    h = np_f16_bits(Wf).reshape(M // R, R * N)
    return km, h


@pytest.mark.parametrize("rule", [oracle.ABSMIN, oracle.ABSMAX])
def test_membership_and_bound_on_outlier_linear(rule):
    """Every bucket holds the binary16 value of one of its own colliders (or +0
    if nobody hashes there).  With unit importance the AbsMin sketch never
    increases a magnitude (underestimation bound); AbsMax never decreases it."""
    lin, _ = synth.linear_256x512()
    R, Bg = lin.R, 128
    S = oracle.encode(lin.W, None, R, lin.bpw, lin.seed, rule)
    km, h = _members(lin.W, R, Bg, lin.seed)
    nb = S.shape[0]
    for b in range(nb):
        for q in range(Bg):
            coll = h[b, km == q]
            if coll.size == 0:
                assert S[b, q] == 0
            else:
                assert S[b, q] in set(coll.tolist())
    What = oracle.decode(S, lin.M, lin.N, R, lin.bpw, lin.seed)
    ref = np_f16_bits(lin.W).view(np.float16).astype(np.float64)
    if rule == oracle.ABSMIN:
        assert np.all(np.abs(What) <= np.abs(ref))
    else:
        assert np.all(np.abs(What) >= np.abs(ref))


def test_outlier_linear_argmin_argmax_at_full_size():
    """The small linear (1% of entries x10) at its real size: each bucket holds
    the first-occurring arg-extreme key of its colliders (NumPy argmin/argmax
    return the first occurrence = smallest l).  AbsMin keeps few outliers,
    AbsMax many: the outliers are the large weights the rule is about."""
    lin, _ = synth.linear_256x512()
    base = synth.outlier_normal_f32((256, 512), 0.02, 0.0, 10.0, 1001)  # same draw, no outliers
    is_out = lin.W != base
    assert is_out.sum() == 1311
    R, Bg = 8, 128
    km = oracle.bucket_map(R, lin.N, 1, Bg)
    S_min = oracle.encode(lin.W, lin.imp, R, 0.5, 1, oracle.ABSMIN)
    S_max = oracle.encode(lin.W, lin.imp, R, 0.5, 1, oracle.ABSMAX)
    out_blk = is_out.reshape(32, R * lin.N)
    Wblk = lin.W.reshape(32, R * lin.N)
    keys = np.abs(Wblk) * np.tile(lin.imp, R)[None, :]
    kept_min = kept_max = 0
    for b in range(32):
        for q in range(Bg):
            pos = np.flatnonzero(km == q)
            lo = pos[np.argmin(keys[b, pos])]
            hi = pos[np.argmax(keys[b, pos])]
            assert S_min[b, q] == np_f16_bits(Wblk[b, lo])
            assert S_max[b, q] == np_f16_bits(Wblk[b, hi])
            kept_min += bool(out_blk[b, lo])
            kept_max += bool(out_blk[b, hi])
    # a bucket holds >= 1 outlier with probability 1 - 0.99^32 ~ 0.28
    assert kept_min < 0.01 * 32 * Bg < 0.15 * 32 * Bg < kept_max


def test_single_bucket_collapses_to_block_extreme():
    """Bg = 1: the whole block shares one bucket, which holds the block's
    first-occurring minimum |w| (AbsMin) or maximum |w| (AbsMax)."""
    g = np.random.default_rng(3)
    R, N = 4, 8
    W = g.standard_normal((12, N)).astype(np.float32)
    bpw = 16.0 / (R * N)
    for rule, pick in ((oracle.ABSMIN, np.argmin), (oracle.ABSMAX, np.argmax)):
        S = oracle.encode(W, None, R, bpw, 9, rule)
        for b in range(3):
            blk = W[b * R:(b + 1) * R].reshape(-1)
            assert S[b, 0] == np_f16_bits(blk[pick(np.abs(blk))])


def test_constant_magnitude_keeps_sign_of_smallest_index():
    """All |w| equal: every key ties, so each bucket holds its smallest-l
    collider; the signs reveal which one won, under both rules."""
    g = np.random.default_rng(5)
    R, N, Bg, seed = 8, 64, 16, 1
    sign = g.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(16, N))
    W = (0.75 * sign).astype(np.float32)
    km = oracle.bucket_map(R, N, seed, Bg)
    for rule in (oracle.ABSMIN, oracle.ABSMAX):
        S = oracle.encode(W, None, R, 16.0 * Bg / (R * N), seed, rule)
        for b in range(2):
            blk = W[b * R:(b + 1) * R].reshape(-1)
            for q in range(Bg):
                first = np.flatnonzero(km == q)[0]
                assert S[b, q] == np_f16_bits(blk[first])


def test_single_collider_buckets_are_exact():
    g = np.random.default_rng(8)
    R, N, Bg, seed = 2, 40, 64, 4     # 80 positions into 64 buckets: many singletons
    W = g.standard_normal((6, N)).astype(np.float32)
    km = oracle.bucket_map(R, N, seed, Bg)
    cnt = np.bincount(km, minlength=Bg)
    S = oracle.encode(W, None, R, 16.0 * Bg / (R * N), seed, oracle.ABSMIN)
    What = oracle.decode(S, 6, N, R, 16.0 * Bg / (R * N), seed)
    ref = np_f16_bits(W).view(np.float16).astype(np.float64)
    single = cnt[km] == 1
    for b in range(3):
        blk_ref = ref[b * R:(b + 1) * R].reshape(-1)
        blk_hat = What[b * R:(b + 1) * R].reshape(-1)
        assert single.sum() > 10
        np.testing.assert_array_equal(blk_hat[single], blk_ref[single])
    assert np.all(S[:, cnt == 0] == 0)


def test_importance_changes_the_winner():
    """A column of importance 0 has key 0, so AbsMin picks it whenever it collides."""
    R, N, Bg, seed = 1, 64, 8, 1
    g = np.random.default_rng(2)
    W = (g.random((1, N)).astype(np.float32) + 1.0)
    imp = np.ones(N, dtype=np.float32)
    imp[17] = 0.0
    S = oracle.encode(W, imp, R, 16.0 * Bg / N, seed, oracle.ABSMIN)
    q = oracle.bucket(17, seed, Bg)
    assert S[0, q] == np_f16_bits(W[0, 17])


@pytest.mark.parametrize("bad,code", [(float("nan"), -2), (float("inf"), -2), (65520.0, -2), (-70000.0, -2)])
def test_encode_rejects_out_of_range_weights(bad, code):
    W = np.ones((8, 32), dtype=np.float32)
    W[3, 5] = bad
    with pytest.raises(oracle.OracleError) as e:
        oracle.encode(W, None, 8, 0.5, 1)
    assert e.value.code == code


def test_encode_accepts_largest_finite_rounding():
    W = np.ones((8, 32), dtype=np.float32)
    W[3, 5] = 65519.0       # rounds to 65504
    S = oracle.encode(W, None, 8, 0.5, 1, oracle.ABSMAX)
    assert S.max() == 0x7BFF


@pytest.mark.parametrize("bad", [-1.0, float("nan"), float("inf")])
def test_encode_rejects_bad_importance(bad):
    W = np.ones((8, 32), dtype=np.float32)
    imp = np.ones(32, dtype=np.float32)
    imp[4] = bad
    with pytest.raises(oracle.OracleError) as e:
        oracle.encode(W, imp, 8, 0.5, 1)
    assert e.value.code == -1


# ---------------------------------------------------------------------------
# decode and product
# ---------------------------------------------------------------------------

def _one_hot_P(R, N, seed, Bg):
    km = oracle.bucket_map(R, N, seed, Bg)
    P = np.zeros((R * N, Bg))
    P[np.arange(R * N), km] = 1.0
    return P


def test_decode_is_S_times_P_transpose():
    """W_hat = S * P^T with the one-hot projection (Metodología §4): for block b,
    the R*N reconstructed weights are S[b] . P^T."""
    lin, _ = synth.linear_256x512()
    S = oracle.encode(lin.W, lin.imp, 8, 0.5, 1)
    P = _one_hot_P(8, lin.N, 1, 128)
    S_val = S.view(np.float16).astype(np.float64)
    What = oracle.decode(S, lin.M, lin.N, 8, 0.5, 1)
    mm = (S_val @ P.T).reshape(lin.M, lin.N)
    np.testing.assert_array_equal(What, mm)


def test_product_dense_identity_and_factorized_form():
    """Y = X . W_hat^T (NumPy float64 matmul on the oracle's W_hat) and the
    factorized Y[t, bR+r] = sum_k S[b,k] (P^T x)[r,k] (the matrix form the
    pages prove equal to the sequential one) both match the oracle's product."""
    lin, x = synth.linear_256x512()
    R, N, Bg = 8, lin.N, 128
    S = oracle.encode(lin.W, lin.imp, R, 0.5, 1)
    X = np.concatenate([x, synth.normal_f32((3, N), 1.0, 77)])
    Y = oracle.matmul(S, X, lin.M, N, R, 0.5, 1)
    What = oracle.decode(S, lin.M, N, R, 0.5, 1)
    Yd = X.astype(np.float64) @ What.T
    np.testing.assert_allclose(Y, Yd, rtol=1e-12, atol=1e-12)
    km = oracle.bucket_map(R, N, 1, Bg).reshape(R, N)
    Z = np.zeros((X.shape[0], R, Bg))
    for r in range(R):
        for j in range(N):
            Z[:, r, km[r, j]] += X[:, j]
    S_val = S.view(np.float16).astype(np.float64)         # [nb, Bg]
    Yf = np.einsum("bk,trk->tbr", S_val, Z).reshape(X.shape[0], lin.M)
    np.testing.assert_allclose(Y, Yf, rtol=1e-12, atol=1e-12)


def test_product_constant_weight_closed_form():
    """W = c everywhere: every bucket holds fp16(c), so Y[t,i] = fp16(c) * sum_j X[t,j]."""
    c = np.float32(0.1)
    W = np.full((32, 96), c, dtype=np.float32)
    X = synth.normal_f32((5, 96), 1.0, 12)
    S = oracle.encode(W, None, 4, 0.5, 3)
    c16 = float(np.float16(c))
    assert np.all(S == np_f16_bits(c))
    Y = oracle.matmul(S, X, 32, 96, 4, 0.5, 3)
    ref = c16 * X.astype(np.float64).sum(axis=1)
    np.testing.assert_allclose(Y, np.repeat(ref[:, None], 32, axis=1), rtol=1e-13)


def test_sampled_product_equals_full_product():
    lin, x = synth.linear_256x512()
    S = oracle.encode(lin.W, lin.imp, 8, 0.5, 1)
    X = synth.normal_f32((4, lin.N), 1.0, 5)
    Y = oracle.matmul(S, X, lin.M, lin.N, 8, 0.5, 1)
    g = np.random.default_rng(1)
    t = g.integers(0, 4, 300)
    i = g.integers(0, lin.M, 300)
    np.testing.assert_array_equal(oracle.matmul_sampled(S, X, lin.M, lin.N, 8, 0.5, t, i, 1), Y[t, i])


def test_bf16_product_inputs_widen_exactly():
    """bfloat16 inputs enter the product as their exact values."""
    lin, _ = synth.linear_256x512()
    S = oracle.encode(lin.W, lin.imp, 8, 0.5, 1)
    Xb = synth.normal_bf16((2, lin.N), 6)
    Y16 = oracle.matmul(S, Xb, lin.M, lin.N, 8, 0.5, 1, x_dtype=oracle.BF16)
    Y32 = oracle.matmul(S, synth.bf16_to_f32(Xb).reshape(2, lin.N), lin.M, lin.N, 8, 0.5, 1)
    np.testing.assert_array_equal(Y16, Y32)
