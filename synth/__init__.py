"""Seeded synthetic inputs shared by the oracle side and the HIP side of the tests.

This module draws random numbers and rounds them to the storage formats of the
workloads; it holds none of the sketch method's arithmetic (no hashing, no
bucket selection, no decoding, no products).  Every array comes from NumPy's
PCG64 generator with an explicit seed, so both sides see identical bytes.

Storage conventions: float32 arrays are float32; bfloat16 data is returned as
uint16 bit patterns (NumPy has no bfloat16).

Workloads (LLM-shaped linears, W is [out, in] = [M, N]):
  linear_256x512      256x512 float32 W ~ N(0, 0.02^2) with 1% of the entries
                      (1,311 distinct positions) multiplied by 10; importance
                      ~ U(0.5, 1.5); one float32 x ~ N(0, 1); R=8, 0.5 bpw.
  attn_4096x4096      4096x4096 bfloat16 W from Student-t(4) scaled to std 0.02;
                      importance ~ U(0.5, 1.5); bfloat16 x ~ N(0, 1); R=8, 0.5 bpw.
  mlp_up_11008x4096   11008x4096 bfloat16 Student-t(4), std 0.02; 0.5 and 0.75 bpw;
                      R=8; batches 1, 4, 16.
  layer_7b            the seven linears of a 7B-style decoder layer (q, k, v, o
                      4096x4096; gate, up 11008x4096; down 4096x11008), Student-t(4)
                      std 0.02, 0.5 bpw, R=8; 256 steps of fresh batch-1 x per linear.
  mlp_70b_prefill     28672x8192 bfloat16 Student-t(4), std 0.015, 0.5 bpw, R=16;
                      X 2048x8192 bfloat16 ~ N(0, 1); importance ~ U(0.5, 1.5).
"""
import math

import numpy as np

# ----------------------------------------------------------------------------
# primitives
# ----------------------------------------------------------------------------


def rng(seed):
    return np.random.Generator(np.random.PCG64(int(seed)))


def bf16_bits(f32):
    """float32 array -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits):
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(shape, std, seed):
    return (rng(seed).standard_normal(shape) * std).astype(np.float32)


def normal_bf16(shape, seed):
    """bfloat16 N(0, 1) samples (float64 draw -> float32 -> bfloat16 RNE)."""
    return bf16_bits(rng(seed).standard_normal(shape).astype(np.float32))


def student_t_bf16(shape, std, seed, df=4, chunk_rows=1024):
    """bfloat16 Student-t(df) samples scaled to standard deviation ``std``.

    t(df) has variance df/(df-2), so the draw is multiplied by
    std / sqrt(df/(df-2)).  Rows are drawn in chunks from one generator to
    bound host memory; the sequence does not depend on the chunk size.
    """
    M, N = shape
    g = rng(seed)
    scale = std / math.sqrt(df / (df - 2.0))
    out = np.empty((M, N), dtype=np.uint16)
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        out[r0:r1] = bf16_bits((g.standard_t(df, size=(r1 - r0, N)) * scale).astype(np.float32))
    return out


def uniform_f32(n, lo, hi, seed):
    return rng(seed).uniform(lo, hi, size=n).astype(np.float32)


def outlier_normal_f32(shape, std, frac, factor, seed):
    """N(0, std^2) float32 with round(frac*size) distinct positions multiplied by ``factor``."""
    g = rng(seed)
    w = (g.standard_normal(shape) * std).astype(np.float32)
    n_out = int(round(frac * w.size))
    pos = g.choice(w.size, size=n_out, replace=False)
    flat = w.reshape(-1)
    flat[pos] *= np.float32(factor)
    return w


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

class Linear:
    """One sketched linear: weights, importance and sketch parameters."""

    def __init__(self, name, M, N, R, bpw, w_dtype, W, imp, seed=1):
        self.name, self.M, self.N, self.R, self.bpw = name, M, N, R, bpw
        self.w_dtype = w_dtype      # "f32" or "bf16"
        self.W, self.imp, self.seed = W, imp, seed

    def __repr__(self):
        return "Linear(%s %dx%d R=%d bpw=%g %s)" % (self.name, self.M, self.N, self.R, self.bpw, self.w_dtype)


def linear_256x512():
    base = 1000
    W = outlier_normal_f32((256, 512), 0.02, 0.01, 10.0, base + 1)
    imp = uniform_f32(512, 0.5, 1.5, base + 2)
    x = normal_f32((1, 512), 1.0, base + 3)
    return Linear("linear_256x512", 256, 512, 8, 0.5, "f32", W, imp), x


def attn_4096x4096():
    base = 2000
    W = student_t_bf16((4096, 4096), 0.02, base + 1)
    imp = uniform_f32(4096, 0.5, 1.5, base + 2)
    x = normal_bf16((1, 4096), base + 3)
    return Linear("attn_4096x4096", 4096, 4096, 8, 0.5, "bf16", W, imp), x


def mlp_up_11008x4096(bpw):
    base = 3000
    W = student_t_bf16((11008, 4096), 0.02, base + 1)
    imp = uniform_f32(4096, 0.5, 1.5, base + 2)
    xs = {b: normal_bf16((b, 4096), base + 10 + b) for b in (1, 4, 16)}
    return Linear("mlp_up_11008x4096", 11008, 4096, 8, bpw, "bf16", W, imp), xs


LAYER_7B_SHAPES = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                   ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008))


def layer_7b_linear(idx):
    base = 4000 + 100 * idx
    name, M, N = LAYER_7B_SHAPES[idx]
    W = student_t_bf16((M, N), 0.02, base + 1)
    imp = uniform_f32(N, 0.5, 1.5, base + 2)
    return Linear("layer_7b." + name, M, N, 8, 0.5, "bf16", W, imp)


def layer_7b_tokens(idx, steps=256):
    """Fresh batch-1 bfloat16 x for every step: array [steps, N]."""
    _, _, N = LAYER_7B_SHAPES[idx]
    return normal_bf16((steps, N), 4000 + 100 * idx + 3)


def mlp_70b_prefill(rows=28672, tokens=2048):
    base = 5000
    W = student_t_bf16((rows, 8192), 0.015, base + 1)
    imp = uniform_f32(8192, 0.5, 1.5, base + 2)
    X = normal_bf16((tokens, 8192), base + 3)
    return Linear("mlp_70b_prefill", rows, 8192, 16, 0.5, "bf16", W, imp), X
