"""Pins of the oracle's 4-bit buckets ("Resumen Técnico" › Resultados: 0.5
bits per weight combined with 4-bit quantization).

Readings under test: Bg4 = R*N*bpw/4 signed 4-bit buckets per block (8
weights per bucket at 0.5 bpw, the same table bytes as binary16 buckets); the
winner of a bucket is the binary16 sketch's winner; one binary16 scale per
block, s = f16(max |winner| / 7); q = clamp(rint(w / s), -7, 7) in float32;
empty buckets and s == 0 give 0; W_hat = q * s; two codes per byte, the even
bucket in the low nibble.
"""
import numpy as np
import pytest

import oracle
import synth
from test_oracle_pins import py_bucket


def _unpack(T, Bg4):
    """Codes int[nb, Bg4] from the packed bytes (two's complement nibbles)."""
    lo = (T & 0x0F).astype(np.int64)
    hi = (T >> 4).astype(np.int64)
    q = np.empty((T.shape[0], Bg4), dtype=np.int64)
    q[:, 0::2], q[:, 1::2] = lo, hi
    return np.where(q >= 8, q - 16, q)


def brute_q4(Wf, imp, R, Bg4, seed, rule):
    """Set-based winners (independent hash), then the scale and the codes with
    NumPy float32 arithmetic."""
    M, N = Wf.shape
    kmap = [py_bucket(l, seed, Bg4) for l in range(R * N)]
    codes = np.zeros((M // R, Bg4), dtype=np.int64)
    scales = np.zeros(M // R, dtype=np.uint16)
    for b in range(M // R):
        block = Wf[b * R:(b + 1) * R]
        keys = {l: np.float32(abs(block[l // N, l % N])) * np.float32(1.0 if imp is None else imp[l % N])
                for l in range(R * N)}
        win = {}
        for q in range(Bg4):
            coll = [l for l in range(R * N) if kmap[l] == q]
            if coll:
                win[q] = min(coll, key=(lambda l: (keys[l], l)) if rule == oracle.ABSMIN else (lambda l: (-keys[l], l)))
        amax = max((np.float32(abs(block[l // N, l % N])) for l in win.values()), default=np.float32(0))
        s16 = np.float16(np.float32(amax) / np.float32(7.0))
        scales[b] = s16.view(np.uint16)
        s = np.float32(s16)
        for q, l in win.items():
            if s > 0:
                v = np.rint(np.float32(block[l // N, l % N]) / s)
                codes[b, q] = int(min(7.0, max(-7.0, v)))
    return codes, scales


def test_layout_same_bytes_as_binary16_buckets():
    """8 weights per 4-bit bucket at 0.5 bpw: four times the buckets of the
    binary16 sketch and the same table bytes (plus one scale per block)."""
    for (M, N, R, bpw) in [(256, 512, 8, 0.5), (4096, 4096, 8, 0.5), (28672, 8192, 16, 0.5), (64, 96, 4, 0.75)]:
        nb, Bg4 = oracle.layout_q4(M, N, R, bpw)
        nb16, Bg = oracle.layout(M, N, R, bpw)
        assert nb == nb16 and Bg4 == 4 * Bg
        assert nb * Bg4 // 2 == nb16 * Bg * 2
        assert (R * N) // Bg4 == 8 or bpw != 0.5
    with pytest.raises(oracle.OracleError):
        oracle.layout_q4(8, 6, 1, 0.5)        # Bg4 = 0.75
    with pytest.raises(oracle.OracleError):
        oracle.layout_q4(8, 12, 1, 1.0)       # Bg4 = 3: odd


@pytest.mark.parametrize("rule", [oracle.ABSMIN, oracle.ABSMAX])
def test_brute_force(rule):
    g = np.random.default_rng(7)
    for _ in range(10):
        R = int(g.integers(1, 5))
        N = int(g.choice([8, 12, 16, 20]))
        M = R * int(g.integers(1, 4))
        bpw = float(g.choice([0.5, 1.0, 2.0]))
        Bg4 = R * N * bpw / 4
        if Bg4 != int(Bg4) or int(Bg4) % 2 or Bg4 < 2:
            continue
        Bg4 = int(Bg4)
        W = (g.standard_normal((M, N)) * 0.3).astype(np.float32)
        imp = g.choice(np.array([0.0, 0.5, 1.0, 2.0], dtype=np.float32), size=N)
        seed = int(g.integers(0, 2**32))
        T, sc = oracle.encode_q4(W, imp, R, bpw, seed, rule)
        codes, scales = brute_q4(W, imp, R, Bg4, seed, rule)
        assert np.array_equal(_unpack(T, Bg4), codes)
        assert np.array_equal(sc, scales)


def test_codes_follow_the_binary16_sketch():
    """With weights exact in binary16, every code is the rounding of the
    binary16 sketch's bucket (same bucket count) by the block scale, the
    block's largest winner gets |q| = 7 and the sign is the bucket's."""
    M, N, R = 64, 512, 8
    g = np.random.default_rng(3)
    W = (np.round(g.standard_normal((M, N)) * 256) / 2048).astype(np.float32)   # exact in binary16
    imp = synth.uniform_f32(N, 0.5, 1.5, 4)
    T, sc = oracle.encode_q4(W, imp, R, 0.5, 9)
    nb, Bg4 = oracle.layout_q4(M, N, R, 0.5)
    S16 = oracle.encode(W, imp, R, 2.0, 9)             # binary16 sketch with Bg = Bg4 buckets
    assert S16.shape == (nb, Bg4)
    vals = S16.view(np.float16).astype(np.float32)
    codes = _unpack(T, Bg4)
    for b in range(nb):
        s = np.float32(sc[b:b + 1].view(np.float16)[0])
        amax = np.abs(vals[b]).max()
        assert s == np.float32(np.float16(amax / np.float32(7)))
        want = np.clip(np.rint(vals[b] / s), -7, 7).astype(np.int64)
        assert np.array_equal(codes[b], want), b
        assert np.abs(codes[b]).max() == 7
        assert np.all(np.sign(codes[b]) * np.sign(vals[b]) >= 0)


def test_decode_and_product():
    M, N, R = 48, 256, 8
    W = synth.normal_f32((M, N), 0.1, 21)
    T, sc = oracle.encode_q4(W, None, R, 0.5, 2)
    nb, Bg4 = oracle.layout_q4(M, N, R, 0.5)
    codes = _unpack(T, Bg4)
    s = sc.view(np.float16).astype(np.float64)
    D = oracle.decode_q4(T, sc, M, N, R, 0.5, 2)
    for i in range(0, M, 5):
        for j in range(0, N, 7):
            k = oracle.bucket((i % R) * N + j, 2, Bg4)
            assert D[i, j] == codes[i // R, k] * s[i // R]
    X = synth.normal_f32((3, N), 1.0, 22)
    Y = oracle.matmul_q4(T, sc, X, M, N, R, 0.5, 2)
    ref = X.astype(np.float64) @ D.T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    t = np.array([0, 2]); i = np.array([47, 3])
    assert np.array_equal(oracle.matmul_sampled_q4(T, sc, X, M, N, R, 0.5, t, i, 2), Y[t, i])


def test_quantization_error_bound():
    """AbsMin with unit importance: |W_hat - winner| <= s/2 for every bucket
    (no clamping below the block maximum), so the 4-bit sketch differs from
    the binary16 sketch of the same bucket count by at most half a step."""
    M, N, R = 32, 512, 8
    W = synth.normal_f32((M, N), 0.1, 31)
    T, sc = oracle.encode_q4(W, None, R, 0.5, 5)
    D4 = oracle.decode_q4(T, sc, M, N, R, 0.5, 5)
    D16 = oracle.decode(oracle.encode(W, None, R, 2.0, 5), M, N, R, 2.0, 5)
    s = np.repeat(sc.view(np.float16).astype(np.float64), R)[:, None]
    assert np.all(np.abs(D4 - D16) <= s / 2 + np.abs(D16) * 2.0 ** -10)


def test_zero_and_underflowing_blocks_give_zero_codes():
    M, N, R = 16, 64, 8
    W = np.zeros((M, N), np.float32)
    W[8:] = 1e-9                                 # max / 7 underflows binary16 to 0
    T, sc = oracle.encode_q4(W, None, R, 0.5)
    assert np.all(T == 0) and np.all(sc == 0)
    assert np.all(oracle.decode_q4(T, sc, M, N, R, 0.5) == 0)


def test_q4_rejections():
    W = synth.normal_f32((16, 64), 0.1, 41)
    with pytest.raises(oracle.OracleError):
        oracle.encode_q4(W, None, 8, 0.1)       # Bg4 not an integer
    W[0, 0] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.encode_q4(W, None, 8, 0.5)
