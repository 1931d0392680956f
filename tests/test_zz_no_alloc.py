"""sketch_matmul_noalloc (the product for callers that cannot allocate) against
sketch_matmul, both through the C ABI: identical outputs on two calls in a
row, the second smaller, on shapes whose product stages Z in the scratch;
calls beyond the scratch are refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y_close, dev, to_dev

sk = pytest.importorskip("sub_bit_weight_sketch_amd")

pytestmark = pytest.mark.gpu


def _noalloc(p, proj, tables, X, Y):
    L = sk.lib()
    fn = L.sketch_matmul_noalloc
    fn.argtypes = [ctypes.POINTER(sk.SketchParams), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn(ctypes.byref(p), ctypes.c_void_p(proj.data_ptr()), ctypes.c_void_p(tables.data_ptr()),
              ctypes.c_void_p(X.data_ptr()), sk.dtype_code(X), X.shape[0], ctypes.c_void_p(Y.data_ptr()),
              sk._stream_handle(X.device))


# M, N, R, batch, x kind: every case stages Z (a workspace > 0)
CASES = [
    (65536, 1024, 8, 5, "bf16"),     # stacked row blocks: Z once per call, the streaming loop
    (24, 4000, 3, 3, "f32"),         # R = 3: the float32 product after a Z pass
]


def test_noalloc_matches_sketch_matmul_twice_second_smaller():
    outs = []
    for M, N, R, b, xk in CASES:
        W = synth.normal_bf16((M, N), 700 + R)
        t = sk.encode(to_dev(W, "bf16"), None, bpw=0.5, seed=3, R=R)
        X = synth.normal_f32((b, N), 1.0, 710 + R) if xk == "f32" else synth.normal_bf16((b, N), 710 + R)
        Xd = to_dev(X, xk)
        wsb = sk.sketch_workspace_bytes(t.params, b, sk.dtype_code(Xd))
        assert wsb > 0
        Y_ref = torch.full((b, M), float("nan"), dtype=torch.float32, device=dev())
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev())
        sk.sketch_matmul(t.params, t.proj, t.tables, Xd, Y_ref, ws)
        Y = torch.full((b, M), float("nan"), dtype=torch.float32, device=dev())
        assert _noalloc(t.params, t.proj, t.tables, Xd, Y) == sk.OK
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ref), (M, N, R, b)
        S = t.tables.cpu().numpy().view(np.uint16)
        Yr = oracle.matmul(S, X, M, N, R, 0.5, 3, x_dtype=oracle.F32 if xk == "f32" else oracle.BF16)
        assert_y_close(Y.cpu().numpy(), Yr, what="noalloc %dx%d R=%d b=%d" % (M, N, R, b))
        outs.append(Y)
    assert CASES[1][0] * CASES[1][3] < CASES[0][0] * CASES[0][3]   # the second call is the smaller one


def test_noalloc_without_scratch_and_beyond_it():
    # batch 1 on a small weight sums Z in place (no scratch), and a GEMM-sized
    # bf16 batch needs none either: both give sketch_matmul's outputs
    M, N = 512, 2048
    W = synth.normal_bf16((M, N), 720)
    t = sk.encode(to_dev(W, "bf16"), None, bpw=0.5, R=8)
    for b in (1, 40):
        Xd = to_dev(synth.normal_bf16((b, N), 721 + b), "bf16")
        assert sk.sketch_workspace_bytes(t.params, b, sk.BF16) == 0
        Y_ref = sk.matmul(t, Xd)
        Y = torch.empty_like(Y_ref)
        assert _noalloc(t.params, t.proj, t.tables, Xd, Y) == sk.OK
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ref)
    # a product whose Z needs more than the scratch holds is refused (host check)
    big = sk.params(64 * 4096, 4096, 32, 2.0, 1, sk.ABSMIN, sk.BF16)     # R = 32, Bg = 16384: Z of 16 tokens is 32 MiB
    assert sk.sketch_workspace_bytes(big, 16, sk.F32) > sk.NOALLOC_SCRATCH_BYTES
    Xd = torch.zeros((16, 4096), dtype=torch.float32, device=dev())
    Y = torch.empty((16, 64 * 4096), dtype=torch.float32, device=dev())
    dummy = torch.empty(16, dtype=torch.uint8, device=dev())
    assert _noalloc(big, dummy, dummy, Xd, Y) == sk.ENOSPACE


def test_noalloc_multi_row_prefill_splits_k_only_when_the_scratch_holds_the_parts():
    """The multi-row prefill product's workspace is optional: at 128 tokens
    its K split (four parts, three of them in the workspace: 6 MiB) fits the
    scratch, and the call gives the bits of sketch_matmul with that
    workspace; at 300 tokens (14 MiB) it does not, and the call gives the
    bits of sketch_matmul without one (unsplit).  Random finite tables."""
    g = torch.Generator(device=dev())
    g.manual_seed(41)
    p = sk.params(4096, 4096, 8, 0.5, 1, sk.ABSMIN, sk.BF16, rows=2)
    nb, bg, _ = sk.sketch_layout(p)
    tables = torch.randint(0, 0x3C00, (nb, bg), generator=g, device=dev(), dtype=torch.int32).to(torch.int16)
    proj = sk.projection(p, dev())
    for tokens, fits in ((128, True), (300, False)):
        X = torch.randn((tokens, 4096), generator=g, device=dev()).to(torch.bfloat16)
        wsb = sk.sketch_workspace_bytes(p, tokens, sk.BF16)
        assert wsb == 3 * tokens * 4096 * 4 and (wsb <= (8 << 20)) == fits
        Y = torch.full((tokens, 4096), float("nan"), dtype=torch.float32, device=dev())
        assert _noalloc(p, proj, tables, X, Y) == sk.OK
        ref = torch.full_like(Y, float("nan"))
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev()) if fits else None
        sk.sketch_matmul(p, proj, tables, X, ref, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(Y).all() and torch.equal(Y, ref), tokens
