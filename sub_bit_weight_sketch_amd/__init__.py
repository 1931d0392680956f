"""Python binding of the MI355X sketch library (``_lib/libsketch.so``).

Argument marshalling only: every step of the encoder and of the product runs in
the library's HIP kernels.  PyTorch provides device memory and the stream.

The C ABI (``include/sketch.h``) has the same names:
``sketch_layout``, ``sketch_projection_bytes``, ``sketch_projection_build``,
``sketch_encode``, ``sketch_encode_status``, ``sketch_workspace_bytes``,
``sketch_matmul``, ``sketch_matmul_noalloc``, ``sketch_group_bytes``, ``sketch_group_plan``,
``sketch_matmul_group``, ``sketch_decode``, ``sketch_decode_hashed``,
``sketch_block_importance``, ``sketch_alloc_plan``, ``sketch_status_str``.

High-level use::

    import sub_bit_weight_sketch_amd as sk
    t = sk.encode(W, importance, bpw=0.5, seed=1, R=8)      # W on cuda, [M, N]
    Y = sk.matmul(t, X)                                       # X [batch, N] -> Y [batch, M] fp32
    W_hat = sk.decode(t, torch.bfloat16)                      # materialised [M, N]
    a = sk.allocate(W, a2, R=8, bpw=0.5)                      # importance-aware bucket counts
    t = sk.encode(W, importance, bpw=0.5, R=8, alloc=a)       # ragged tables, same budget
"""
import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libsketch.so")

OK, EINVAL, ERANGE, EDEVICE, ESMALL, ENOSPACE = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 8 << 20      # static scratch of sketch_matmul_noalloc (per GPU)
F32, BF16, F16 = 0, 1, 2
ABSMIN, ABSMAX = 0, 1
FLAG_WEIGHT_RANGE, FLAG_IMPORTANCE, FLAG_PROJECTION, FLAG_ALLOCATION = 1, 2, 4, 8

EXPORTS = ("sketch_layout", "sketch_projection_bytes", "sketch_projection_build", "sketch_encode",
           "sketch_encode_status", "sketch_workspace_bytes", "sketch_matmul", "sketch_matmul_noalloc",
           "sketch_group_bytes", "sketch_group_plan", "sketch_matmul_group",
           "sketch_decode", "sketch_decode_hashed", "sketch_block_importance", "sketch_alloc_plan",
           "sketch_status_str")
GROUP_MAX_ITEMS = 65536


class SketchParams(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("R", ctypes.c_int32), ("bpw", ctypes.c_double),
                ("seed", ctypes.c_uint32), ("rule", ctypes.c_int), ("w_dtype", ctypes.c_int), ("rows", ctypes.c_int32),
                ("block_offsets", ctypes.c_void_p), ("block_bg_max", ctypes.c_int32), ("bucket_bits", ctypes.c_int32)]


class GroupItem(ctypes.Structure):
    _fields_ = [("p", ctypes.POINTER(SketchParams)), ("proj", ctypes.c_void_p), ("tables", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class SketchError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (what, status_str(code), code))


_lib = None
_lib_lock = threading.Lock()


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError("libsketch.so is missing at %s: build it with "
                                  "`python -m sub_bit_weight_sketch_amd.build`" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            P = ctypes.POINTER(SketchParams)
            vp, i64, sz, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
            L.sketch_layout.argtypes = [P, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(sz)]
            L.sketch_projection_bytes.argtypes = [P, ctypes.POINTER(sz)]
            L.sketch_projection_build.argtypes = [P, vp, sz, vp]
            L.sketch_encode.argtypes = [P, vp, vp, vp, vp, vp, vp]
            L.sketch_encode_status.argtypes = [ctypes.c_int32]
            L.sketch_workspace_bytes.argtypes = [P, i64, ctypes.c_int, ctypes.POINTER(sz)]
            L.sketch_matmul.argtypes = [P, vp, vp, vp, ctypes.c_int, i64, vp, vp, sz, vp]
            L.sketch_matmul_noalloc.argtypes = [P, vp, vp, vp, ctypes.c_int, i64, vp, vp]
            G = ctypes.POINTER(GroupItem)
            L.sketch_group_bytes.argtypes = [G, ctypes.c_int32, ctypes.c_int, ctypes.POINTER(sz), ctypes.POINTER(sz)]
            L.sketch_group_plan.argtypes = [G, ctypes.c_int32, ctypes.c_int, vp, sz, vp]
            L.sketch_matmul_group.argtypes = [G, ctypes.c_int32, ctypes.c_int, vp, vp, sz, vp]
            L.sketch_decode.argtypes = [P, vp, vp, vp, ctypes.c_int, vp]
            L.sketch_decode_hashed.argtypes = [P, vp, vp, ctypes.c_int, vp]
            L.sketch_block_importance.argtypes = [P, vp, vp, vp, vp]
            L.sketch_alloc_plan.argtypes = [i64, i64, i64, vp, vp, ctypes.POINTER(ctypes.c_int32)]
            L.sketch_status_str.argtypes = [ctypes.c_int]
            L.sketch_status_str.restype = ctypes.c_char_p
            for name in EXPORTS[:-1]:
                getattr(L, name).restype = st
            _lib = L
    return _lib


def sketch_status_str(code):
    return lib().sketch_status_str(int(code)).decode()


status_str = sketch_status_str


def _check(code, what):
    if code != OK:
        raise SketchError(code, what)


def params(M, N, R=8, bpw=0.5, seed=1, rule=ABSMIN, w_dtype=BF16, rows=1, alloc=None, bits=16):
    """sketch_params; alloc: an Allocation (importance-aware bucket counts) or
    None; bits: 16 (binary16 buckets) or 4 (4-bit codes with block scales)."""
    if isinstance(rule, str):
        rule = {"absmin": ABSMIN, "absmax": ABSMAX}[rule.lower()]
    return SketchParams(int(M), int(N), int(R), float(bpw), int(seed) & 0xFFFFFFFF, int(rule), int(w_dtype),
                        int(rows), alloc.offsets.data_ptr() if alloc is not None else None,
                        int(alloc.bg_max) if alloc is not None else 0, int(bits))


_TORCH_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


def dtype_code(t):
    try:
        return _TORCH_DT[t.dtype]
    except KeyError:
        raise TypeError("unsupported dtype %s (float32, bfloat16 or float16)" % t.dtype) from None


def _stream_handle(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


# ---------------------------------------------------------------------------
# thin wrappers of the C ABI (same names)
# ---------------------------------------------------------------------------

def sketch_layout(p):
    nb, bg, tb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _check(lib().sketch_layout(ctypes.byref(p), ctypes.byref(nb), ctypes.byref(bg), ctypes.byref(tb)),
           "sketch_layout")
    return nb.value, bg.value, tb.value


def sketch_projection_bytes(p):
    n = ctypes.c_size_t()
    _check(lib().sketch_projection_bytes(ctypes.byref(p), ctypes.byref(n)), "sketch_projection_bytes")
    return n.value


def sketch_projection_build(p, proj, stream=None):
    stream = stream if stream is not None else _stream_handle(proj.device)
    _check(lib().sketch_projection_build(ctypes.byref(p), _ptr(proj), proj.numel() * proj.element_size(), stream),
           "sketch_projection_build")


def sketch_encode(p, proj, W, importance, tables, status, stream=None):
    """status: a zeroed int32 device tensor the kernel ORs flags into
    (asynchronous), or None: the call waits for the stream and raises
    SketchError for out-of-range weights or bad importance."""
    stream = stream if stream is not None else _stream_handle(W.device)
    _check(lib().sketch_encode(ctypes.byref(p), _ptr(proj), _ptr(W), _ptr(importance), _ptr(tables), _ptr(status),
                               stream), "sketch_encode")


def sketch_encode_status(flags):
    return lib().sketch_encode_status(int(flags))


def sketch_workspace_bytes(p, batch, x_dtype):
    n = ctypes.c_size_t()
    _check(lib().sketch_workspace_bytes(ctypes.byref(p), int(batch), int(x_dtype), ctypes.byref(n)),
           "sketch_workspace_bytes")
    return n.value


def sketch_matmul(p, proj, tables, X, Y, workspace, stream=None):
    stream = stream if stream is not None else _stream_handle(X.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sketch_matmul(ctypes.byref(p), _ptr(proj), _ptr(tables), _ptr(X), dtype_code(X), X.shape[0],
                               _ptr(Y), _ptr(workspace), wsb, stream), "sketch_matmul")


def sketch_matmul_noalloc(p, proj, tables, X, Y, stream=None):
    """sketch_matmul without a workspace: the library's static per-GPU
    scratch stands in for it (calls overlapping on one GPU race)."""
    stream = stream if stream is not None else _stream_handle(X.device)
    _check(lib().sketch_matmul_noalloc(ctypes.byref(p), _ptr(proj), _ptr(tables), _ptr(X), dtype_code(X), X.shape[0],
                                       _ptr(Y), stream), "sketch_matmul_noalloc")


def group_items(entries):
    """ctypes array of GroupItem from (params, proj, tables, x, y) tuples (x [N]
    or [1, N] and y [M] or [1, M] device tensors); keeps the params alive on
    the array."""
    arr = (GroupItem * len(entries))()
    keep = []
    for i, (p, proj, tables, x, y) in enumerate(entries):
        keep.append(p)
        arr[i].p = ctypes.pointer(p)
        arr[i].proj, arr[i].tables = proj.data_ptr(), tables.data_ptr()
        arr[i].x, arr[i].y = x.data_ptr(), y.data_ptr()
    arr._keep = keep
    return arr


def sketch_group_bytes(items, x_dtype):
    """(plan bytes, workspace bytes) of a group (host call)."""
    pb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().sketch_group_bytes(items, len(items), int(x_dtype), ctypes.byref(pb), ctypes.byref(wb)),
           "sketch_group_bytes")
    return pb.value, wb.value


def sketch_group_plan(items, x_dtype, plan, stream=None):
    stream = stream if stream is not None else _stream_handle(plan.device)
    _check(lib().sketch_group_plan(items, len(items), int(x_dtype), _ptr(plan), plan.numel() * plan.element_size(),
                                   stream), "sketch_group_plan")


def sketch_matmul_group(items, x_dtype, plan, workspace, stream=None):
    stream = stream if stream is not None else _stream_handle(plan.device)
    _check(lib().sketch_matmul_group(items, len(items), int(x_dtype), _ptr(plan), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), stream), "sketch_matmul_group")


def sketch_decode(p, proj, tables, out, stream=None):
    stream = stream if stream is not None else _stream_handle(out.device)
    _check(lib().sketch_decode(ctypes.byref(p), _ptr(proj), _ptr(tables), _ptr(out), dtype_code(out), stream),
           "sketch_decode")


def sketch_decode_hashed(p, tables, out, stream=None):
    stream = stream if stream is not None else _stream_handle(out.device)
    _check(lib().sketch_decode_hashed(ctypes.byref(p), _ptr(tables), _ptr(out), dtype_code(out), stream),
           "sketch_decode_hashed")


def sketch_block_importance(p, W, a2, scores, stream=None):
    stream = stream if stream is not None else _stream_handle(W.device)
    _check(lib().sketch_block_importance(ctypes.byref(p), _ptr(W), _ptr(a2), _ptr(scores), stream),
           "sketch_block_importance")


def sketch_alloc_plan(nb, total, lo, scores):
    """Host call: scores (CPU float64 tensor [nb]) -> (offsets CPU int64 tensor [nb + 1], bg_max)."""
    scores = scores.detach().to("cpu", torch.float64).contiguous()
    off = torch.empty(int(nb) + 1, dtype=torch.int32)
    mx = ctypes.c_int32()
    _check(lib().sketch_alloc_plan(int(nb), int(total), int(lo), _ptr(scores), _ptr(off), ctypes.byref(mx)),
           "sketch_alloc_plan")
    return off.to(torch.int64) & 0xFFFFFFFF, mx.value


# ---------------------------------------------------------------------------
# high-level API
# ---------------------------------------------------------------------------

_proj_cache = {}
_proj_lock = threading.Lock()


def projection(p, device):
    """Projection buffer for (R, N, Bg, seed) on `device`, built once and cached."""
    _, bg, _ = sketch_layout(p)
    dev = torch.device(device)
    key = (int(p.R), int(p.N), bg, int(p.seed), max(1, int(p.rows)), bool(p.block_offsets), dev.index)
    # (4-bit buckets share the binary16 projection of their bucket count: same key)
    with _proj_lock:
        t = _proj_cache.get(key)
        if t is None:
            t = torch.empty(sketch_projection_bytes(p), dtype=torch.uint8, device=dev)
            sketch_projection_build(p, t)
            # built once, then handed to callers on any stream: wait for it
            # here so that no later call can start on a half-built buffer
            torch.cuda.current_stream(dev).synchronize()
            _proj_cache[key] = t
    return t


class Tables:
    """Sketch state of one linear: parameters, bucket tables [M/R, Bg] (binary16
    bits in an int16 tensor) and the projection they were encoded with."""

    def __init__(self, p, tables, proj, alloc=None):
        self.params, self.tables, self.proj, self.alloc = p, tables, proj, alloc

    @property
    def shape(self):
        return (self.params.M, self.params.N)

    def half(self):
        """The buckets as a float16 tensor (a view, no copy)."""
        return self.tables.view(torch.float16)


class Allocation:
    """Importance-aware bucket counts of a weight's row blocks: offsets
    (uint32 [nb + 1] held in an int32 device tensor; block b owns buckets
    offsets[b] .. offsets[b+1]) and the largest count."""

    def __init__(self, offsets, bg_max, device):
        off = torch.as_tensor(offsets, dtype=torch.int64)
        self.counts = (off[1:] - off[:-1]).clone()
        self.offsets = off.to(torch.int32).to(device)   # bit pattern of the uint32 offsets
        self.bg_max = int(bg_max)


def block_importance(W, a2, R=8):
    """Float32 [M/R] on W's device: sum over each row block of W^2 * a2 (a2 = E[x^2] per input column)."""
    W = W.contiguous()
    M, N = W.shape
    p = params(M, N, R, 16.0, 1, ABSMIN, dtype_code(W))
    scores = torch.empty(M // R, dtype=torch.float32, device=W.device)
    a2 = a2.to(device=W.device, dtype=torch.float32).contiguous()
    sketch_block_importance(p, W, a2, scores)
    return scores


def allocate(W, a2, R=8, bpw=0.5, lo=None, scores=None):
    """Bucket counts for W [M, N] from the expected squared inputs a2 [N]:
    the uniform budget (M/R blocks x R*N*bpw/16 buckets), a floor of `lo`
    per block (default a quarter of the uniform count), the rest by block
    importance (largest remainder).  Synchronises to read the scores."""
    M, N = W.shape
    nb, bg, _ = sketch_layout(params(M, N, R, bpw))
    if scores is None:
        scores = block_importance(W, a2, R)
    lo = max(1, bg // 4) if lo is None else int(lo)
    off, mx = sketch_alloc_plan(nb, nb * bg, lo, scores.to(torch.float64).cpu())
    return Allocation(off, mx, W.device)


def encode(W, importance=None, bpw=0.5, seed=1, R=8, rule=ABSMIN, check=True, status=None, rows=1, alloc=None,
           bits=16):
    """Sketch-encode W [M, N] (float32, bfloat16 or float16 on a GPU).
    rows > 1: the multi-row sketch (rows hash functions sharing the Bg
    buckets of a block, Bg % rows == 0).  alloc: an Allocation (per-block
    bucket counts; the tables are then one flat [nb * Bg] tensor).  bits=4:
    4-bit buckets (the tables are a uint8 buffer of codes then block scales).

    importance: float32 [N] or None.  With check=True the call waits for the
    device and raises SketchError on out-of-range weights or bad importance;
    with check=False it stays asynchronous and ORs flags into `status`
    (a zeroed int32 device tensor of one element) when given.
    """
    if W.dim() != 2 or not W.is_cuda:
        raise ValueError("W must be a 2-D GPU tensor")
    W = W.contiguous()
    M, N = W.shape
    p = params(M, N, R, bpw, seed, rule, dtype_code(W), rows, alloc, bits)
    nb, bg, tb = sketch_layout(p)
    proj = projection(p, W.device)
    if bits == 4:
        tables = torch.zeros(tb, dtype=torch.uint8, device=W.device)
    else:
        tables = torch.empty((nb, bg) if alloc is None else (nb * bg,), dtype=torch.int16, device=W.device)
    if importance is not None:
        importance = importance.to(device=W.device, dtype=torch.float32).contiguous()
        if importance.shape != (N,):
            raise ValueError("importance must have shape (N,)")
    own_status = status is None
    if own_status:
        status = torch.zeros(1, dtype=torch.int32, device=W.device)
    sketch_encode(p, proj, W, importance, tables, status)
    if check:
        flags = int(status.item())
        rc = sketch_encode_status(flags)
        if rc != OK:
            raise SketchError(rc, "sketch_encode (device flags 0x%x)" % flags)
    return Tables(p, tables, proj, alloc)


def workspace_for(t, batch, x_dtype, device):
    """Workspace for products of `batch` tokens (None if not needed).  Reuse it
    across calls on one stream, never for two calls in flight at once."""
    n = sketch_workspace_bytes(t.params, batch, x_dtype)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n else None


def matmul(t, X, out=None, workspace=None):
    """Y = X . W_hat^T for X [batch, N] (or [N]) -> float32 [batch, M]."""
    squeeze = X.dim() == 1
    if squeeze:
        X = X[None, :]
    X = X.contiguous()
    if X.shape[1] != t.params.N:
        raise ValueError("X has %d columns, expected %d" % (X.shape[1], t.params.N))
    batch = X.shape[0]
    Y = out if out is not None else torch.empty((batch, t.params.M), dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = workspace_for(t, batch, dtype_code(X), X.device)
    sketch_matmul(t.params, t.proj, t.tables, X, Y, workspace)
    return Y[0] if squeeze else Y


class Group:
    """A planned grouped decode product: several Tables, each multiplied by its
    own token.  xs[i] is [N_i] (or [1, N_i]); ys[i] is [M_i] float32.  The plan
    names these exact buffers; call run() after refilling xs to multiply
    again.  The group holds a reference to every buffer its plan names
    (tables, projections, xs, ys), so none of them is freed (and, after
    torch.cuda.empty_cache(), unmapped) while the plan can still run."""

    def __init__(self, tables, xs, ys):
        if not (len(tables) == len(xs) == len(ys)) or not tables:
            raise ValueError("one x and one y per Tables")
        self._buffers = ([(t.tables, t.proj) for t in tables], list(xs), list(ys))
        self.x_dtype = dtype_code(xs[0])
        self.items = group_items([(t.params, t.proj, t.tables, x, y) for t, x, y in zip(tables, xs, ys)])
        pb, wb = sketch_group_bytes(self.items, self.x_dtype)
        dev = xs[0].device
        self.plan = torch.empty(pb, dtype=torch.uint8, device=dev)
        self.workspace = torch.empty(max(wb, 16), dtype=torch.uint8, device=dev)
        sketch_group_plan(self.items, self.x_dtype, self.plan)

    def run(self, stream=None):
        sketch_matmul_group(self.items, self.x_dtype, self.plan, self.workspace, stream)


def decode(t, dtype=torch.bfloat16, out=None, hashed=False):
    """W_hat [M, N] of dtype (float16: the bucket bits, float32: exact,
    bfloat16: rounded to nearest even).  hashed=True takes the per-weight
    hash path (the measurement baseline) instead of the forward map."""
    W = out if out is not None else torch.empty((t.params.M, t.params.N), dtype=dtype, device=t.tables.device)
    if hashed:
        sketch_decode_hashed(t.params, t.tables, W)
    else:
        sketch_decode(t.params, t.proj, t.tables, W)
    return W
