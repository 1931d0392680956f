"""Pins of the oracle's importance-aware space allocation ("Resumen Técnico" ›
Metodología §2: rows or layers of higher importance, measured by E[a^2], get
more sketch space, i.e. more buckets).

Readings under test: the unit is the row block, its importance is
s_b = sum_{i in b} sum_j W[i][j]^2 * E[x_j^2]; the bucket counts keep the bit
budget (they add up to the uniform total), each block gets a floor of lo and
the rest in proportion to s_b by largest remainder (ties to the lower block);
block b hashes with the sketch's hash reduced to its own count and its table
sits at the offset sum_{c<b} bg_c; everything else is the single-row sketch.
"""
import numpy as np
import pytest

import oracle
import synth
from test_oracle_pins import brute_encode


def test_plan_worked_example():
    """s = (1, 2, 3, 0), total 40, floor 2: the 32 shared buckets have quotas
    16/3, 32/3, 16, 0 -> floors 5, 10, 16, 0 (31), the leftover unit goes to
    the largest remainder (2/3, block 1): 2 + (5, 11, 16, 0)."""
    bg = oracle.alloc_plan(np.array([1.0, 2.0, 3.0, 0.0]), 40, 2)
    assert bg.tolist() == [7, 13, 18, 2]


def test_plan_ties_go_to_the_lower_block():
    """Equal importances, 10 shared units over 4 blocks: quotas 2.5 each,
    floors 8, two leftover units to blocks 0 and 1."""
    assert oracle.alloc_plan(np.ones(4), 14, 1).tolist() == [4, 4, 3, 3]
    assert oracle.alloc_plan(np.zeros(4), 14, 1).tolist() == [4, 4, 3, 3]   # all zero: equal shares


@pytest.mark.parametrize("seed", range(6))
def test_plan_properties(seed):
    """Budget kept, floor respected, every block within one unit of its quota
    (floor or ceiling), more importance never fewer buckets, exactly the
    leftover count of blocks rounded up."""
    g = np.random.default_rng(seed)
    nb = int(g.integers(1, 300))
    s = g.gamma(0.7, 1.0, nb) * (g.random(nb) < 0.9)
    lo = int(g.integers(1, 20))
    total = nb * lo + int(g.integers(0, 50 * nb))
    bg = oracle.alloc_plan(s, total, lo)
    assert bg.sum() == total and bg.min() >= lo
    E = total - nb * lo
    q = E * s / s.sum() if s.sum() > 0 else np.full(nb, E / nb)
    extra = bg - lo
    assert np.all(extra >= np.floor(q) - 1e-9) and np.all(extra <= np.floor(q) + 1)
    assert int((extra > np.floor(q)).sum()) == E - int(np.floor(q).sum())
    for a in range(min(nb, 40)):
        for c in range(min(nb, 40)):
            if s[a] > s[c]:
                assert bg[a] >= bg[c]


def test_plan_largest_remainder_brute_force():
    """Tiny cases: Hamilton's allocation is the integer allocation with the
    right total that is closest to the quotas in L1 distance (sum |a_b - q_b|);
    found here by enumerating every allocation (random real importances, so
    there are no ties)."""
    import itertools
    g = np.random.default_rng(11)
    for _ in range(40):
        nb = int(g.integers(1, 5))
        s = g.gamma(1.0, 1.0, nb)
        lo = int(g.integers(1, 3))
        E = int(g.integers(0, 10))
        q = E * s / s.sum()
        best = None
        for a in itertools.product(range(E + 1), repeat=nb):
            if sum(a) != E:
                continue
            d = float(np.abs(np.array(a) - q).sum())
            if best is None or d < best[0] - 1e-12:
                best = (d, a)
        assert oracle.alloc_plan(s, nb * lo + E, lo).tolist() == [lo + v for v in best[1]]


def test_plan_rejections():
    with pytest.raises(oracle.OracleError):
        oracle.alloc_plan(np.ones(4), 7, 2)            # below the floor
    with pytest.raises(oracle.OracleError):
        oracle.alloc_plan(np.array([1.0, -1.0]), 10, 1)
    with pytest.raises(oracle.OracleError):
        oracle.alloc_plan(np.array([1.0, np.nan]), 10, 1)
    with pytest.raises(oracle.OracleError):
        oracle.alloc_plan(np.ones(3), 10, 0)


def test_block_importance_is_expected_squared_output():
    """s_b against NumPy's float64 sum of W^2 * E[x^2] over the block, for
    float32 and bfloat16 weights; and against the mean square of X W^T over
    many independent zero-mean inputs with those second moments."""
    M, N, R = 48, 96, 8
    W = synth.normal_f32((M, N), 0.1, 3)
    a2 = synth.uniform_f32(N, 0.25, 2.0, 4)
    ref = (W.astype(np.float64) ** 2 * a2.astype(np.float64)).reshape(M // R, R, N).sum(axis=(1, 2))
    np.testing.assert_allclose(oracle.block_importance(W, a2, R), ref, rtol=1e-12)
    Wb = synth.bf16_bits(W)
    Wbf = synth.bf16_to_f32(Wb).reshape(M, N).astype(np.float64)
    refb = (Wbf ** 2 * a2).reshape(M // R, R, N).sum(axis=(1, 2))
    np.testing.assert_allclose(oracle.block_importance(Wb, a2, R, w_dtype=oracle.BF16), refb, rtol=1e-12)
    g = np.random.default_rng(5)
    X = g.standard_normal((200000, N)) * np.sqrt(a2.astype(np.float64))
    Ey2 = ((X @ W.astype(np.float64).T) ** 2).mean(axis=0).reshape(M // R, R).sum(axis=1)
    np.testing.assert_allclose(oracle.block_importance(W, a2, R), Ey2, rtol=0.02)


def test_uniform_allocation_is_the_uniform_sketch():
    """Every block at the uniform count: tables, decode and product equal the
    single-row sketch's bit for bit."""
    for (M, N, R, bpw, seed, rule) in [(64, 256, 8, 0.5, 1, oracle.ABSMIN), (30, 100, 3, 16 * 25 / 300, 7, oracle.ABSMAX)]:
        W = synth.normal_f32((M, N), 0.1, M + N)
        imp = synth.uniform_f32(N, 0.5, 1.5, N)
        nb, Bg = oracle.layout(M, N, R, bpw)
        bg = np.full(nb, Bg)
        S = oracle.encode(W, imp, R, bpw, seed, rule)
        Sa = oracle.encode_alloc(W, imp, R, bg, seed, rule)
        assert np.array_equal(Sa, S.reshape(-1))
        assert np.array_equal(oracle.decode_alloc(Sa, M, N, R, bg, seed), oracle.decode(S, M, N, R, bpw, seed))
        X = synth.normal_f32((3, N), 1.0, 9)
        assert np.array_equal(oracle.matmul_alloc(Sa, X, M, N, R, bg, seed), oracle.matmul(S, X, M, N, R, bpw, seed))


@pytest.mark.parametrize("rule", [oracle.ABSMIN, oracle.ABSMAX])
def test_each_block_is_a_brute_force_sketch_of_its_own_size(rule):
    """Block b's segment against the set-based brute force of that block alone
    with bg_b buckets (independent hash), on ragged counts."""
    g = np.random.default_rng(21)
    M, N, R = 24, 20, 4
    W = np.round(g.standard_normal((M, N)) * 4).astype(np.float32) / 4
    imp = g.choice(np.array([0.0, 0.5, 1.0, 2.0], dtype=np.float32), size=N)
    bg = np.array([1, 7, 3, 12, 5, 2])
    S = oracle.encode_alloc(W, imp, R, bg, 99, rule)
    off = np.concatenate([[0], np.cumsum(bg)])
    for b in range(M // R):
        ref = brute_encode(W[b * R:(b + 1) * R], imp, R, int(bg[b]), 99, rule)
        assert np.array_equal(S[off[b]:off[b + 1]], ref[0]), "block %d" % b


def test_decode_and_product_of_an_allocated_sketch():
    """decode: W_hat[i][j] = S[off_b + k_b(l)] against a direct NumPy index
    computation with the oracle's bucket function; product: the dense product
    of that W_hat; sampled outputs equal the full product's."""
    M, N, R = 40, 64, 8
    W = synth.normal_f32((M, N), 0.1, 31)
    a2 = synth.uniform_f32(N, 0.5, 1.5, 32)
    nb, Bg = oracle.layout(M, N, R, 0.5)
    bg = oracle.alloc_plan(oracle.block_importance(W, a2, R), nb * Bg, 4)
    assert len(set(bg.tolist())) > 1
    S = oracle.encode_alloc(W, None, R, bg, 5)
    D = oracle.decode_alloc(S, M, N, R, bg, 5)
    off = np.concatenate([[0], np.cumsum(bg)])
    for i in range(M):
        b = i // R
        for j in range(N):
            q = oracle.bucket((i % R) * N + j, 5, int(bg[b]))
            assert D[i, j] == oracle.f16_to_f64(int(S[off[b] + q]))
    X = synth.normal_f32((4, N), 1.0, 33)
    Y = oracle.matmul_alloc(S, X, M, N, R, bg, 5)
    ref = X.astype(np.float64) @ D.T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    t = np.array([0, 3, 2]); i = np.array([0, 39, 17])
    assert np.array_equal(oracle.matmul_sampled_alloc(S, X, M, N, R, bg, t, i, 5), Y[t, i])


def test_more_buckets_reconstruct_more_weights_exactly():
    """Every non-empty bucket reconstructs its winner exactly (AbsMin, unit
    importance), so a block reconstructs at least as many weights exactly as
    it has non-empty buckets -- and giving it more buckets gives it more of
    them (the reason the pages give more space to the important rows)."""
    M, N, R = 16, 256, 8
    W = synth.normal_f32((M, N), 0.1, 41)
    w16 = oracle.f32_to_f16_array(W).view(np.float16).astype(np.float64)
    nonempty = []
    for bg0 in (16, 64, 256, 1024):
        bg = np.array([bg0, 64])
        S = oracle.encode_alloc(W, None, R, bg, 3)
        D = oracle.decode_alloc(S, M, N, R, bg, 3)
        ne = int((S[:bg0] != 0).sum())
        exact = int((D[:R] == w16[:R]).sum())
        assert exact >= ne
        nonempty.append(ne)
    assert nonempty[0] < nonempty[1] < nonempty[2] < nonempty[3]


def test_alloc_rejections():
    W = synth.normal_f32((16, 32), 0.1, 51)
    with pytest.raises(oracle.OracleError):
        oracle.encode_alloc(W, None, 8, np.array([4, 0]))
    with pytest.raises(ValueError):
        oracle.encode_alloc(W, None, 8, np.array([4, 4, 4]))
    with pytest.raises(oracle.OracleError):
        oracle.block_importance(W, np.full(32, -1.0, np.float32), 8)
