"""ctypes front end of the C oracle (``sketch_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Arrays are NumPy: weights/activations are float32, or uint16 holding bfloat16
or binary16 bit patterns (``dtype`` says which); bucket tables are uint16
binary16 bit patterns of shape [M/R, Bg]; products are float64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, F16 = 0, 1, 2
ABSMIN, ABSMAX = 0, 1
_OK, _EINVAL, _ERANGE = 0, -1, -2


class OracleError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s: oracle status %d (%s)" % (
            what, code, {_EINVAL: "invalid argument", _ERANGE: "weight out of range"}.get(code, "?")))


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src_mtime = os.path.getmtime(_build.SRC)
    if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < src_mtime:
        _build.build()
    _lib = bind(ctypes.CDLL(_build.LIB))
    return _lib


def bind(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    i64, i32, u32, dbl, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = dbl
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_f32_to_f16_n.argtypes = [vp, i64, vp]
    lib.oracle_f32_to_f16_n.restype = None
    lib.oracle_layout.argtypes = [i64, i64, i32, dbl, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.oracle_layout.restype = ctypes.c_int
    lib.oracle_hash32.argtypes = [u32]
    lib.oracle_hash32.restype = u32
    lib.oracle_bucket.argtypes = [u32, u32, u32]
    lib.oracle_bucket.restype = u32
    lib.oracle_bucket_map.argtypes = [i64, i64, u32, u32, vp]
    lib.oracle_bucket_map.restype = None
    lib.oracle_encode.argtypes = [i64, i64, i32, dbl, u32, ctypes.c_int, ctypes.c_int, vp, vp, vp, ctypes.c_int]
    lib.oracle_encode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [i64, i64, i32, dbl, u32, vp, vp]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_matmul.argtypes = [i64, i64, i32, dbl, u32, vp, vp, ctypes.c_int, i64, vp, ctypes.c_int]
    lib.oracle_matmul.restype = ctypes.c_int
    lib.oracle_matmul_sampled.argtypes = [i64, i64, i32, dbl, u32, vp, vp, ctypes.c_int, i64, i64, vp, vp, vp,
                                          ctypes.c_int]
    lib.oracle_matmul_sampled.restype = ctypes.c_int
    lib.oracle_encode_rows.argtypes = [i64, i64, i32, dbl, u32, ctypes.c_int, i32, ctypes.c_int, vp, vp, vp,
                                       ctypes.c_int]
    lib.oracle_encode_rows.restype = ctypes.c_int
    lib.oracle_decode_rows.argtypes = [i64, i64, i32, dbl, u32, ctypes.c_int, i32, vp, vp]
    lib.oracle_decode_rows.restype = ctypes.c_int
    lib.oracle_matmul_rows.argtypes = [i64, i64, i32, dbl, u32, ctypes.c_int, i32, vp, vp, ctypes.c_int, i64, vp,
                                       ctypes.c_int]
    lib.oracle_matmul_rows.restype = ctypes.c_int
    lib.oracle_matmul_sampled_rows.argtypes = [i64, i64, i32, dbl, u32, ctypes.c_int, i32, vp, vp, ctypes.c_int, i64,
                                               i64, vp, vp, vp, ctypes.c_int]
    lib.oracle_matmul_sampled_rows.restype = ctypes.c_int
    lib.oracle_block_importance.argtypes = [i64, i64, i32, ctypes.c_int, vp, vp, vp]
    lib.oracle_block_importance.restype = ctypes.c_int
    lib.oracle_alloc_plan.argtypes = [i64, i64, i64, vp, vp]
    lib.oracle_alloc_plan.restype = ctypes.c_int
    lib.oracle_encode_alloc.argtypes = [i64, i64, i32, u32, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, ctypes.c_int]
    lib.oracle_encode_alloc.restype = ctypes.c_int
    lib.oracle_decode_alloc.argtypes = [i64, i64, i32, u32, vp, vp, vp]
    lib.oracle_decode_alloc.restype = ctypes.c_int
    lib.oracle_matmul_alloc.argtypes = [i64, i64, i32, u32, vp, vp, vp, ctypes.c_int, i64, vp, ctypes.c_int]
    lib.oracle_matmul_alloc.restype = ctypes.c_int
    lib.oracle_matmul_sampled_alloc.argtypes = [i64, i64, i32, u32, vp, vp, vp, ctypes.c_int, i64, i64, vp, vp, vp,
                                                ctypes.c_int]
    lib.oracle_matmul_sampled_alloc.restype = ctypes.c_int
    lib.oracle_layout_q4.argtypes = [i64, i64, i32, dbl, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.oracle_layout_q4.restype = ctypes.c_int
    lib.oracle_encode_q4.argtypes = [i64, i64, i32, dbl, u32, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, ctypes.c_int]
    lib.oracle_encode_q4.restype = ctypes.c_int
    lib.oracle_decode_q4.argtypes = [i64, i64, i32, dbl, u32, vp, vp, vp]
    lib.oracle_decode_q4.restype = ctypes.c_int
    lib.oracle_matmul_q4.argtypes = [i64, i64, i32, dbl, u32, vp, vp, vp, ctypes.c_int, i64, vp, ctypes.c_int]
    lib.oracle_matmul_q4.restype = ctypes.c_int
    lib.oracle_matmul_sampled_q4.argtypes = [i64, i64, i32, dbl, u32, vp, vp, vp, ctypes.c_int, i64, i64, vp, vp, vp,
                                             ctypes.c_int]
    lib.oracle_matmul_sampled_q4.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a, dtype):
    if a.dtype == np.float32:
        if dtype not in (None, F32):
            raise ValueError("float32 array passed with a 16-bit dtype code")
        return F32
    if a.dtype == np.uint16:
        if dtype not in (BF16, F16):
            raise ValueError("uint16 array needs dtype=BF16 or F16")
        return dtype
    raise TypeError("arrays must be float32 or uint16 bit patterns, got %s" % a.dtype)


def max_threads():
    return _load().oracle_max_threads()


def f16_to_f64(h):
    return _load().oracle_f16_to_f64(int(h))


def f32_to_f16(f):
    return _load().oracle_f32_to_f16(float(np.float32(f)))


def f32_to_f16_array(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_f32_to_f16_n(_ptr(a), a.size, _ptr(out))
    return out


def layout(M, N, R, bpw):
    """(num_blocks, Bg) for an M x N weight in row blocks of R rows at bpw bits/weight."""
    nb, bg = ctypes.c_int64(), ctypes.c_int64()
    rc = _load().oracle_layout(M, N, R, bpw, ctypes.byref(nb), ctypes.byref(bg))
    if rc != _OK:
        raise OracleError(rc, "layout")
    return nb.value, bg.value


def hash32(u):
    return _load().oracle_hash32(int(u) & 0xFFFFFFFF)


def bucket(l, seed, Bg):
    return _load().oracle_bucket(int(l), int(seed), int(Bg))


def bucket_map(R, N, seed, Bg):
    out = np.empty(R * N, dtype=np.uint32)
    _load().oracle_bucket_map(R, N, seed, Bg, _ptr(out))
    return out


def encode(W, imp, R, bpw, seed=1, rule=ABSMIN, w_dtype=None, nthreads=0, rows=1):
    """Bucket tables uint16[M/R, Bg] (binary16 bits).  imp may be None (all ones).
    rows > 1: the multi-row sketch (row rho owns buckets [rho*Bg/rows, (rho+1)*Bg/rows)
    and hashes with seed + rho)."""
    W = np.ascontiguousarray(W)
    M, N = W.shape
    code = _dtype_code(W, w_dtype)
    nb, Bg = layout(M, N, R, bpw)
    S = np.zeros((nb, Bg), dtype=np.uint16)
    ip = None
    if imp is not None:
        imp = np.ascontiguousarray(imp, dtype=np.float32)
        if imp.shape != (N,):
            raise ValueError("importance must have shape (N,)")
        ip = _ptr(imp)
    if rows == 1:
        rc = _load().oracle_encode(M, N, R, bpw, seed, rule, code, _ptr(W), ip, _ptr(S), nthreads)
    else:
        rc = _load().oracle_encode_rows(M, N, R, bpw, seed, rule, rows, code, _ptr(W), ip, _ptr(S), nthreads)
    if rc != _OK:
        raise OracleError(rc, "encode")
    return S


def decode(S, M, N, R, bpw, seed=1, rows=1, rule=ABSMIN):
    """W_hat float64[M, N] (rows > 1: the multi-row decode; rule picks the
    largest (AbsMin) or smallest (AbsMax) magnitude among the rows)."""
    S = np.ascontiguousarray(S, dtype=np.uint16)
    out = np.empty((M, N), dtype=np.float64)
    if rows == 1:
        rc = _load().oracle_decode(M, N, R, bpw, seed, _ptr(S), _ptr(out))
    else:
        rc = _load().oracle_decode_rows(M, N, R, bpw, seed, rule, rows, _ptr(S), _ptr(out))
    if rc != _OK:
        raise OracleError(rc, "decode")
    return out


def matmul(S, X, M, N, R, bpw, seed=1, x_dtype=None, nthreads=0, rows=1, rule=ABSMIN):
    """Y float64[batch, M] = X[batch, N] . W_hat^T."""
    S = np.ascontiguousarray(S, dtype=np.uint16)
    X = np.ascontiguousarray(X)
    if X.ndim == 1:
        X = X[None, :]
    code = _dtype_code(X, x_dtype)
    batch = X.shape[0]
    if X.shape[1] != N:
        raise ValueError("X must have N columns")
    Y = np.empty((batch, M), dtype=np.float64)
    if rows == 1:
        rc = _load().oracle_matmul(M, N, R, bpw, seed, _ptr(S), _ptr(X), code, batch, _ptr(Y), nthreads)
    else:
        rc = _load().oracle_matmul_rows(M, N, R, bpw, seed, rule, rows, _ptr(S), _ptr(X), code, batch, _ptr(Y),
                                        nthreads)
    if rc != _OK:
        raise OracleError(rc, "matmul")
    return Y


def matmul_sampled(S, X, M, N, R, bpw, t_idx, i_idx, seed=1, x_dtype=None, nthreads=0, rows=1, rule=ABSMIN):
    """y[s] = Y[t_idx[s], i_idx[s]] computed one output at a time (float64)."""
    S = np.ascontiguousarray(S, dtype=np.uint16)
    X = np.ascontiguousarray(X)
    if X.ndim == 1:
        X = X[None, :]
    code = _dtype_code(X, x_dtype)
    t_idx = np.ascontiguousarray(t_idx, dtype=np.int64)
    i_idx = np.ascontiguousarray(i_idx, dtype=np.int64)
    y = np.empty(t_idx.shape[0], dtype=np.float64)
    if rows == 1:
        rc = _load().oracle_matmul_sampled(M, N, R, bpw, seed, _ptr(S), _ptr(X), code, X.shape[0],
                                           t_idx.shape[0], _ptr(t_idx), _ptr(i_idx), _ptr(y), nthreads)
    else:
        rc = _load().oracle_matmul_sampled_rows(M, N, R, bpw, seed, rule, rows, _ptr(S), _ptr(X), code, X.shape[0],
                                                t_idx.shape[0], _ptr(t_idx), _ptr(i_idx), _ptr(y), nthreads)
    if rc != _OK:
        raise OracleError(rc, "matmul_sampled")
    return y


# ----------------------------------------------------------------------------
# Importance-aware space allocation (per-row-block bucket counts)

def block_importance(W, a2, R, w_dtype=None):
    """s[b] = sum over the rows i of block b of sum_j W[i][j]^2 * a2[j] (float64)."""
    W = np.ascontiguousarray(W)
    M, N = W.shape
    code = _dtype_code(W, w_dtype)
    a2 = np.ascontiguousarray(a2, dtype=np.float32)
    if a2.shape != (N,):
        raise ValueError("a2 must have shape (N,)")
    s = np.empty(M // R if R > 0 else 0, dtype=np.float64)
    rc = _load().oracle_block_importance(M, N, R, code, _ptr(W), _ptr(a2), _ptr(s))
    if rc != _OK:
        raise OracleError(rc, "block_importance")
    return s


def alloc_plan(s, total, lo=1):
    """Bucket counts int64[nb] from the block importances s (float64[nb]): lo
    each, the rest of the total in proportion to s by largest remainder."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    bg = np.empty(s.shape[0], dtype=np.int64)
    rc = _load().oracle_alloc_plan(s.shape[0], int(total), int(lo), _ptr(s), _ptr(bg))
    if rc != _OK:
        raise OracleError(rc, "alloc_plan")
    return bg


def _bg(bg):
    return np.ascontiguousarray(bg, dtype=np.int64)


def encode_alloc(W, imp, R, bg, seed=1, rule=ABSMIN, w_dtype=None, nthreads=0):
    """Concatenated tables uint16[sum(bg)]: block b's bg[b] buckets at offset sum(bg[:b])."""
    W = np.ascontiguousarray(W)
    M, N = W.shape
    code = _dtype_code(W, w_dtype)
    bg = _bg(bg)
    if bg.shape != (M // R,):
        raise ValueError("bg must have one entry per row block")
    S = np.zeros(int(bg.sum()), dtype=np.uint16)
    ip = None
    if imp is not None:
        imp = np.ascontiguousarray(imp, dtype=np.float32)
        if imp.shape != (N,):
            raise ValueError("importance must have shape (N,)")
        ip = _ptr(imp)
    rc = _load().oracle_encode_alloc(M, N, R, seed, rule, code, _ptr(W), ip, _ptr(bg), _ptr(S), nthreads)
    if rc != _OK:
        raise OracleError(rc, "encode_alloc")
    return S


def decode_alloc(S, M, N, R, bg, seed=1):
    S = np.ascontiguousarray(S, dtype=np.uint16)
    bg = _bg(bg)
    out = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_decode_alloc(M, N, R, seed, _ptr(bg), _ptr(S), _ptr(out))
    if rc != _OK:
        raise OracleError(rc, "decode_alloc")
    return out


def matmul_alloc(S, X, M, N, R, bg, seed=1, x_dtype=None, nthreads=0):
    S = np.ascontiguousarray(S, dtype=np.uint16)
    bg = _bg(bg)
    X = np.ascontiguousarray(X)
    if X.ndim == 1:
        X = X[None, :]
    code = _dtype_code(X, x_dtype)
    if X.shape[1] != N:
        raise ValueError("X must have N columns")
    Y = np.empty((X.shape[0], M), dtype=np.float64)
    rc = _load().oracle_matmul_alloc(M, N, R, seed, _ptr(bg), _ptr(S), _ptr(X), code, X.shape[0], _ptr(Y), nthreads)
    if rc != _OK:
        raise OracleError(rc, "matmul_alloc")
    return Y


def matmul_sampled_alloc(S, X, M, N, R, bg, t_idx, i_idx, seed=1, x_dtype=None, nthreads=0):
    S = np.ascontiguousarray(S, dtype=np.uint16)
    bg = _bg(bg)
    X = np.ascontiguousarray(X)
    if X.ndim == 1:
        X = X[None, :]
    code = _dtype_code(X, x_dtype)
    t_idx = np.ascontiguousarray(t_idx, dtype=np.int64)
    i_idx = np.ascontiguousarray(i_idx, dtype=np.int64)
    y = np.empty(t_idx.shape[0], dtype=np.float64)
    rc = _load().oracle_matmul_sampled_alloc(M, N, R, seed, _ptr(bg), _ptr(S), _ptr(X), code, X.shape[0],
                                             t_idx.shape[0], _ptr(t_idx), _ptr(i_idx), _ptr(y), nthreads)
    if rc != _OK:
        raise OracleError(rc, "matmul_sampled_alloc")
    return y


# ----------------------------------------------------------------------------
# 4-bit buckets (signed codes in [-7, 7], one binary16 scale per block)

def layout_q4(M, N, R, bpw):
    """(num_blocks, Bg4): Bg4 = R*N*bpw/4 four-bit buckets per block."""
    nb, bg = ctypes.c_int64(), ctypes.c_int64()
    rc = _load().oracle_layout_q4(M, N, R, bpw, ctypes.byref(nb), ctypes.byref(bg))
    if rc != _OK:
        raise OracleError(rc, "layout_q4")
    return nb.value, bg.value


def encode_q4(W, imp, R, bpw, seed=1, rule=ABSMIN, w_dtype=None, nthreads=0):
    """(codes uint8[nb, Bg4/2] two per byte, scales uint16[nb] binary16 bits)."""
    W = np.ascontiguousarray(W)
    M, N = W.shape
    code = _dtype_code(W, w_dtype)
    nb, Bg4 = layout_q4(M, N, R, bpw)
    T = np.zeros((nb, Bg4 // 2), dtype=np.uint8)
    sc = np.zeros(nb, dtype=np.uint16)
    ip = None
    if imp is not None:
        imp = np.ascontiguousarray(imp, dtype=np.float32)
        if imp.shape != (N,):
            raise ValueError("importance must have shape (N,)")
        ip = _ptr(imp)
    rc = _load().oracle_encode_q4(M, N, R, bpw, seed, rule, code, _ptr(W), ip, _ptr(T), _ptr(sc), nthreads)
    if rc != _OK:
        raise OracleError(rc, "encode_q4")
    return T, sc


def decode_q4(T, scales, M, N, R, bpw, seed=1):
    T = np.ascontiguousarray(T, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_decode_q4(M, N, R, bpw, seed, _ptr(T), _ptr(scales), _ptr(out))
    if rc != _OK:
        raise OracleError(rc, "decode_q4")
    return out


def matmul_q4(T, scales, X, M, N, R, bpw, seed=1, x_dtype=None, nthreads=0):
    T = np.ascontiguousarray(T, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    X = np.ascontiguousarray(X)
    if X.ndim == 1:
        X = X[None, :]
    code = _dtype_code(X, x_dtype)
    if X.shape[1] != N:
        raise ValueError("X must have N columns")
    Y = np.empty((X.shape[0], M), dtype=np.float64)
    rc = _load().oracle_matmul_q4(M, N, R, bpw, seed, _ptr(T), _ptr(scales), _ptr(X), code, X.shape[0], _ptr(Y),
                                  nthreads)
    if rc != _OK:
        raise OracleError(rc, "matmul_q4")
    return Y


def matmul_sampled_q4(T, scales, X, M, N, R, bpw, t_idx, i_idx, seed=1, x_dtype=None, nthreads=0):
    T = np.ascontiguousarray(T, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    X = np.ascontiguousarray(X)
    if X.ndim == 1:
        X = X[None, :]
    code = _dtype_code(X, x_dtype)
    t_idx = np.ascontiguousarray(t_idx, dtype=np.int64)
    i_idx = np.ascontiguousarray(i_idx, dtype=np.int64)
    y = np.empty(t_idx.shape[0], dtype=np.float64)
    rc = _load().oracle_matmul_sampled_q4(M, N, R, bpw, seed, _ptr(T), _ptr(scales), _ptr(X), code, X.shape[0],
                                          t_idx.shape[0], _ptr(t_idx), _ptr(i_idx), _ptr(y), nthreads)
    if rc != _OK:
        raise OracleError(rc, "matmul_sampled_q4")
    return y
