"""Host-side checks of the C-ABI library (no GPU needed).

The shared library must load and export every function ``include/sketch.h``
declares; the host-only calls (layout, buffer sizes, status names) and the
argument validation of the device calls are exercised without touching a GPU.
"""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sketch.h")

sk = pytest.importorskip("sub_bit_weight_sketch_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sketch_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 16, names
    L = sk.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(sk.EXPORTS)


def test_python_binding_has_the_same_names():
    for n in declared_functions():
        assert callable(getattr(sk, n)), n


def test_status_strings():
    for code in (sk.OK, sk.EINVAL, sk.ERANGE, sk.EDEVICE, sk.ESMALL, sk.ENOSPACE):
        assert sk.status_str(code) and sk.status_str(code) != "unknown status"
    assert sk.status_str(12345) == "unknown status"


@pytest.mark.parametrize("M,N,R,bpw", [(256, 512, 8, 0.5), (4096, 4096, 8, 0.5), (11008, 4096, 8, 0.75),
                                       (4096, 11008, 8, 0.5), (28672, 8192, 16, 0.5), (30, 100, 3, 0.32),
                                       (0, 64, 8, 0.5)])
def test_layout_matches_oracle(M, N, R, bpw):
    p = sk.params(M, N, R, bpw)
    nb, bg, tb = sk.sketch_layout(p)
    assert (nb, bg) == oracle.layout(M, N, R, bpw)
    assert tb == nb * bg * 2


@pytest.mark.parametrize("M,N,R,bpw", [(10, 64, 3, 0.5), (16, 64, 8, 0.3), (16, 0, 8, 0.5), (16, 64, 0, 0.5),
                                       (16, 64, 8, 0.0), (16, 64, 8, float("nan")), (16, 3, 1, 0.5),
                                       (8, 70000, 8, 0.5), (8, 65535, 8, 1.0)])
def test_layout_rejects(M, N, R, bpw):
    with pytest.raises(sk.SketchError) as e:
        sk.sketch_layout(sk.params(M, N, R, bpw))
    assert e.value.code == sk.EINVAL


def test_layout_block_byte_limit():
    """A block's weights (and its 2-byte forward map) must be addressable
    with 32-bit byte offsets: R*N*sizeof(w) < 2^32."""
    # R*N = 2^30, Bg = 16384: fine as bfloat16, too large as float32
    nb, bg, _ = sk.sketch_layout(sk.params(32768, 32768, 32768, 2.0 ** -12, w_dtype=sk.BF16))
    assert (nb, bg) == (1, 16384)
    with pytest.raises(sk.SketchError) as e:
        sk.sketch_layout(sk.params(32768, 32768, 32768, 2.0 ** -12, w_dtype=sk.F32))
    assert e.value.code == sk.EINVAL
    # R*N = 2^31: too large for 16-bit weights as well
    with pytest.raises(sk.SketchError) as e:
        sk.sketch_layout(sk.params(65536, 32768, 65536, 2.0 ** -13, w_dtype=sk.BF16))
    assert e.value.code == sk.EINVAL
    nb, bg, _ = sk.sketch_layout(sk.params(65536, 16384, 65536, 2.0 ** -12, w_dtype=sk.BF16))
    assert (nb, bg) == (1, 16384)


def test_bad_enums_rejected():
    p = sk.params(16, 64)
    p.rule = 7
    with pytest.raises(sk.SketchError):
        sk.sketch_layout(p)
    p = sk.params(16, 64)
    p.w_dtype = 9
    with pytest.raises(sk.SketchError):
        sk.sketch_layout(p)


def test_buffer_sizes():
    p = sk.params(4096, 4096, 8, 0.5)
    pb = sk.sketch_projection_bytes(p)
    # header + forward map + CSR offsets + columns + counters, 256-byte aligned sections
    assert pb >= 256 + 2 * 32768 + 4 * (8 * 1024 + 1) + 2 * 32768 + 4 * 8192
    assert pb % 256 == 0
    # a single token of a small product computes Z in place (no workspace);
    # several tokens, or a large stack of tables, compute Z once into the
    # workspace: [tokens of a pass][R][Bg] float32 + one maximum per 256
    # segments and token, each section 256-byte aligned
    assert sk.sketch_workspace_bytes(p, 1, sk.BF16) == 0
    assert sk.sketch_workspace_bytes(p, 2, sk.BF16) == 2 * 8 * 1024 * 4 + 2 * 32 * 4
    assert sk.sketch_workspace_bytes(p, 16, sk.BF16) == 16 * 8 * 1024 * 4 + 16 * 32 * 4
    big = sk.params(4096 * 512, 4096, 8, 0.5)
    assert sk.sketch_workspace_bytes(big, 1, sk.BF16) >= 4 * 8 * 1024
    assert sk.sketch_workspace_bytes(big, 16, sk.BF16) >= 4 * 8 * 1024
    # shapes outside the matrix-core path stage Z for every token of a pass
    odd = sk.params(48, 100, 3, 16 * 25 / 300)
    assert sk.sketch_workspace_bytes(odd, 5, sk.F32) >= 5 * 4 * 3 * 25
    # bf16 prefill goes to the matrix-core GEMM, which needs no workspace
    assert sk.sketch_workspace_bytes(p, 2048, sk.BF16) == 0
    # float32 activations never take the bf16 GEMM: the decode path runs in
    # passes of 16 tokens, each computing Z once into the workspace
    assert sk.sketch_workspace_bytes(p, 2048, sk.F32) == 16 * 8 * 1024 * 4 + 16 * 32 * 4
    assert sk.sketch_workspace_bytes(odd, 2048, sk.F32) >= 16 * 4 * 3 * 25
    assert sk.sketch_workspace_bytes(p, 0, sk.BF16) == 0
    # multi-row prefill: an optional workspace for the parts of a K split
    # when its 512-token x 128-output tiles would leave compute units idle
    # (256 of them when no device answers): 128 tiles at 2048 tokens, split
    # in two (one extra [2048][4096] float32 part); 32 tiles at 512 tokens,
    # split in four (three parts); none on the decode path
    r2 = sk.params(4096, 4096, 8, 0.5, rows=2)
    assert sk.sketch_workspace_bytes(r2, 2048, sk.BF16) == 2048 * 4096 * 4
    assert sk.sketch_workspace_bytes(r2, 512, sk.BF16) == 3 * 512 * 4096 * 4
    assert sk.sketch_workspace_bytes(r2, 16, sk.BF16) == 0
    assert sk.sketch_workspace_bytes(r2, 2048, sk.F32) == 0
    # 4096 tiles already fill a round: no split
    assert sk.sketch_workspace_bytes(sk.params(4096 * 32, 4096, 8, 0.5, rows=2), 2048, sk.BF16) == 0


def test_device_calls_validate_before_launching():
    L = sk.lib()
    p = sk.params(16, 64)
    vp = ctypes.c_void_p
    # NULL projection -> EINVAL, nothing launched
    assert L.sketch_encode(ctypes.byref(p), None, vp(16), None, vp(16), vp(16), None) == sk.EINVAL
    # misaligned status word -> EINVAL; a NULL status word (the call then
    # waits for the stream and reports the flags itself) is validated the
    # same way before anything runs: misaligned W or tables -> EINVAL
    assert L.sketch_encode(ctypes.byref(p), vp(256), vp(16), None, vp(16), vp(18), None) == sk.EINVAL
    assert L.sketch_encode(ctypes.byref(p), vp(256), vp(18), None, vp(16), None, None) == sk.EINVAL
    assert L.sketch_encode(ctypes.byref(p), vp(256), vp(16), None, vp(24), None, None) == sk.EINVAL
    # misaligned W
    assert L.sketch_encode(ctypes.byref(p), vp(256), vp(18), None, vp(16), vp(16), None) == sk.EINVAL
    # empty M is a no-op, with or without a status word
    p0 = sk.params(0, 64)
    assert L.sketch_encode(ctypes.byref(p0), vp(256), None, None, None, vp(16), None) == sk.OK
    assert L.sketch_encode(ctypes.byref(p0), vp(256), None, None, None, None, None) == sk.OK
    # matmul: batch 0 no-op, negative batch and bad dtype rejected, small workspace
    assert L.sketch_matmul(ctypes.byref(p), vp(256), vp(16), vp(16), sk.BF16, 0, vp(16), None, 0, None) == sk.OK
    assert L.sketch_matmul(ctypes.byref(p), vp(256), vp(16), vp(16), sk.BF16, -1, vp(16), None, 0, None) == sk.EINVAL
    assert L.sketch_matmul(ctypes.byref(p), vp(256), vp(16), vp(16), 5, 1, vp(16), None, 0, None) == sk.EINVAL
    podd = sk.params(48, 100, 3, 16 * 25 / 300)
    assert L.sketch_matmul(ctypes.byref(podd), vp(256), vp(16), vp(16), sk.BF16, 1, vp(16), vp(16), 8, None) == sk.ESMALL
    assert L.sketch_matmul(ctypes.byref(podd), vp(256), vp(16), vp(16), sk.BF16, 1, vp(16), None, 0, None) == sk.EINVAL
    assert L.sketch_projection_build(ctypes.byref(p), vp(256), 16, None) == sk.ESMALL


def test_decode_validates_before_launching():
    L = sk.lib()
    p = sk.params(16, 64)
    vp = ctypes.c_void_p
    assert L.sketch_decode(ctypes.byref(p), None, vp(256), vp(256), sk.BF16, None) == sk.EINVAL
    assert L.sketch_decode(ctypes.byref(p), vp(256), None, vp(256), sk.BF16, None) == sk.EINVAL
    assert L.sketch_decode(ctypes.byref(p), vp(256), vp(256), vp(264), sk.BF16, None) == sk.EINVAL   # misaligned
    assert L.sketch_decode(ctypes.byref(p), vp(256), vp(256), vp(256), 7, None) == sk.EINVAL
    assert L.sketch_decode_hashed(ctypes.byref(p), None, vp(256), sk.F16, None) == sk.EINVAL
    assert L.sketch_decode_hashed(ctypes.byref(p), vp(256), vp(256), 9, None) == sk.EINVAL
    bad = sk.params(10, 64, 3, 0.5)
    assert L.sketch_decode_hashed(ctypes.byref(bad), vp(256), vp(256), sk.F16, None) == sk.EINVAL
    p0 = sk.params(0, 64)   # empty M is a no-op
    assert L.sketch_decode(ctypes.byref(p0), None, None, None, sk.F32, None) == sk.OK
    assert L.sketch_decode_hashed(ctypes.byref(p0), None, None, sk.F32, None) == sk.OK


def test_encode_status_flags():
    assert sk.sketch_encode_status(0) == sk.OK
    assert sk.sketch_encode_status(sk.FLAG_WEIGHT_RANGE) == sk.ERANGE
    assert sk.sketch_encode_status(sk.FLAG_IMPORTANCE) == sk.EINVAL
    assert sk.sketch_encode_status(sk.FLAG_PROJECTION) == sk.EINVAL
    assert sk.sketch_encode_status(sk.FLAG_WEIGHT_RANGE | sk.FLAG_IMPORTANCE) == sk.EINVAL


# ---------------------------------------------------------------------------
# importance-aware allocation: host-only plan and parameter validation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(8))
def test_alloc_plan_matches_oracle(seed):
    """sketch_alloc_plan (library, host) gives the oracle's counts exactly on
    the same float64 scores (sparse, tied and zero scores included)."""
    import numpy as np
    import torch
    g = np.random.default_rng(seed)
    nb = int(g.integers(1, 400))
    s = g.gamma(0.5, 1.0, nb) * (g.random(nb) < 0.8)
    if seed % 3 == 0:
        s = np.round(s * 4) / 4          # many exact ties
    if seed == 5:
        s = np.zeros(nb)
    lo = int(g.integers(1, 30))
    total = nb * lo + int(g.integers(0, 60 * nb))
    off, mx = sk.sketch_alloc_plan(nb, total, lo, torch.from_numpy(s))
    bg = oracle.alloc_plan(s, total, lo)
    assert off[0].item() == 0 and off[-1].item() == total
    assert np.array_equal(np.diff(off.numpy()), bg)
    assert mx == int(bg.max())


def test_alloc_plan_rejections():
    import torch
    with pytest.raises(sk.SketchError):
        sk.sketch_alloc_plan(4, 7, 2, torch.ones(4, dtype=torch.float64))          # below the floor
    with pytest.raises(sk.SketchError):
        sk.sketch_alloc_plan(2, 10, 1, torch.tensor([1.0, -1.0], dtype=torch.float64))
    with pytest.raises(sk.SketchError):
        sk.sketch_alloc_plan(2, 10, 1, torch.tensor([1.0, float("inf")], dtype=torch.float64))
    with pytest.raises(sk.SketchError):
        sk.sketch_alloc_plan(1, 20000, 1, torch.ones(1, dtype=torch.float64))      # one block above the cap


def test_alloc_params_validation():
    """An allocation needs rows == 1, a 4-byte aligned offsets pointer and
    1 <= block_bg_max <= the cap; its projection is the header plus one
    uint32 hash per local index."""
    p = sk.params(4096, 4096, 8, 0.5)
    p.block_offsets = 0x1000        # never dereferenced by host validation
    p.block_bg_max = 2048
    nb, bg, tb = sk.sketch_layout(p)
    assert (nb, bg, tb) == (512, 1024, 512 * 1024 * 2)
    assert sk.sketch_projection_bytes(p) == 256 + 4 * 8 * 4096
    assert sk.sketch_workspace_bytes(p, 1, sk.BF16) == 0
    for field, value in (("block_bg_max", 0), ("block_bg_max", 16385), ("block_offsets", 0x1002), ("rows", 2)):
        q = sk.params(4096, 4096, 8, 0.5)
        q.block_offsets, q.block_bg_max = 0x1000, 2048
        setattr(q, field, value)
        with pytest.raises(sk.SketchError) as e:
            sk.sketch_layout(q)
        assert e.value.code == sk.EINVAL, field


# ---------------------------------------------------------------------------
# 4-bit buckets: layout and validation (host only)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,R,bpw", [(256, 512, 8, 0.5), (4096, 4096, 8, 0.5), (28672, 8192, 16, 0.5),
                                       (48, 100, 4, 0.64)])
def test_q4_layout_matches_oracle(M, N, R, bpw):
    p = sk.params(M, N, R, bpw, bits=4)
    nb, bg, tb = sk.sketch_layout(p)
    assert (nb, bg) == oracle.layout_q4(M, N, R, bpw)
    assert tb == ((nb * bg // 2 + 255) // 256) * 256 + 2 * nb
    assert sk.sketch_workspace_bytes(p, 1, sk.BF16) == 0
    # the projection is the binary16 sketch's for Bg buckets
    q16 = sk.params(M, N, R, bpw * 4)
    assert sk.sketch_projection_bytes(p) == sk.sketch_projection_bytes(q16)


def test_q4_rejections():
    for kw in ({"bits": 4, "bpw": 0.3}, {"bits": 8}, {"bits": 4, "rows": 2}):
        bpw = kw.pop("bpw", 0.5)
        with pytest.raises(sk.SketchError):
            sk.sketch_layout(sk.params(64, 96, 8, bpw, **kw))
    p = sk.params(8, 12, 1, 1.0, bits=4)     # Bg = 3: odd
    with pytest.raises(sk.SketchError):
        sk.sketch_layout(p)


def test_noalloc_refuses_products_beyond_its_scratch_before_launching():
    """sketch_matmul_noalloc validates like sketch_matmul and refuses a
    product whose Z would not fit the static scratch (SKETCH_ENOSPACE),
    before any device work; batch 0 is a no-op."""
    L = sk.lib()
    vp = ctypes.c_void_p
    big = sk.params(64 * 4096, 4096, 32, 2.0)      # R = 32, Bg = 16384: Z of 16 float32 tokens is 32 MiB
    assert sk.sketch_workspace_bytes(big, 16, sk.F32) > sk.NOALLOC_SCRATCH_BYTES
    assert L.sketch_matmul_noalloc(ctypes.byref(big), vp(256), vp(256), vp(256), sk.F32, 16, vp(256), None) \
        == sk.ENOSPACE
    p = sk.params(16, 64)
    assert L.sketch_matmul_noalloc(ctypes.byref(p), vp(256), vp(16), vp(16), sk.BF16, 0, vp(16), None) == sk.OK
    assert L.sketch_matmul_noalloc(ctypes.byref(p), vp(256), vp(16), vp(16), sk.BF16, -1, vp(16), None) == sk.EINVAL
    assert L.sketch_matmul_noalloc(ctypes.byref(p), vp(256), vp(16), vp(16), 7, 1, vp(16), None) == sk.EINVAL


def test_group_rejects_unsupported_items_before_launching():
    """sketch_group_bytes / _plan / sketch_matmul_group check every item on
    the host: uniform single-row sketches with R in {2, 4, 8}, all with
    binary16 buckets (Bg a multiple of 32) or all with 4-bit codes (Bg a
    multiple of 128), x within 120 KiB, aligned pointers; nothing runs for a
    rejected group."""
    vp = 256

    def items_of(ps, align=vp):
        arr = (sk.GroupItem * len(ps))()
        for i, p in enumerate(ps):
            arr[i].p = ctypes.pointer(p)
            arr[i].proj, arr[i].tables, arr[i].x, arr[i].y = align, align, align, align
        arr._keep = ps
        return arr

    L = sk.lib()
    pb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    good = items_of([sk.params(4096, 4096, 8, 0.5), sk.params(4096, 11008, 8, 0.5)])
    assert L.sketch_group_bytes(good, 2, sk.BF16, ctypes.byref(pb), ctypes.byref(wb)) == sk.OK
    # fragments: (1024 + 2752) / 32 K-steps x 64 lanes x 16 bytes, then the
    # scales, then the partial sums of the split tiles: 16 + 16 tiles of 32
    # blocks for the 3,072 stream waves (256 compute units when no device
    # answers), so every tile is split into min(3072 / 32, 16, 8 chunks of
    # the shorter linear) = 8 pieces, one float per piece and row (8192 rows)
    assert wb.value == (1024 + 2752) // 32 * 64 * 16 + 256 + 8 * 8192 * 4 and pb.value > 0
    # 4-bit codes: Bg = 4096 and 11008 codes per block; fragments per K-step of 32 codes
    q4 = items_of([sk.params(4096, 4096, 8, 0.5, bits=4), sk.params(4096, 11008, 8, 0.5, bits=4)])
    assert L.sketch_group_bytes(q4, 2, sk.BF16, ctypes.byref(pb), ctypes.byref(wb)) == sk.OK
    # 8 + 8 tiles of 64 blocks for 2,048 waves: min(128, 16, 16 chunks) = 16 pieces
    assert wb.value == (4096 + 11008) // 32 * 64 * 16 + 256 + 16 * 8192 * 4 and pb.value > 0
    for bad in ([sk.params(4096, 4096, 16, 0.5)],                 # R = 16
                [sk.params(4096, 4096, 8, 0.5, rows=2)],          # multi-row
                [sk.params(80, 120, 8, 16 * 20 / 960)],           # Bg = 20, not a multiple of 32
                [sk.params(64, 1024, 8, 0.5), sk.params(64, 1024, 8, 0.5, bits=4)],   # two bucket formats
                [sk.params(64, 96, 8, 4 * 64 / 768, bits=4)],     # 4-bit, Bg = 64, not a multiple of 128
                [sk.params(64, 1024, 16, 0.5, bits=4)]):          # 4-bit, R = 16
        arr = items_of(bad)
        n = len(bad)
        assert L.sketch_group_bytes(arr, n, sk.BF16, ctypes.byref(pb), ctypes.byref(wb)) == sk.EINVAL
        assert L.sketch_group_plan(arr, n, sk.BF16, ctypes.c_void_p(256), 1 << 20, None) == sk.EINVAL
        assert L.sketch_matmul_group(arr, n, sk.BF16, ctypes.c_void_p(256), ctypes.c_void_p(256), 1 << 30,
                                     None) == sk.EINVAL
    # x beyond 120 KiB of LDS: N = 40960 fits as 16-bit x, not as float32 (above 30720)
    wide = items_of([sk.params(64, 40960, 8, 0.5)])
    assert L.sketch_group_bytes(wide, 1, sk.BF16, ctypes.byref(pb), ctypes.byref(wb)) == sk.OK
    assert L.sketch_group_bytes(wide, 1, sk.F32, ctypes.byref(pb), ctypes.byref(wb)) == sk.EINVAL
    assert L.sketch_group_bytes(good, 0, sk.BF16, ctypes.byref(pb), ctypes.byref(wb)) == sk.EINVAL
    assert L.sketch_group_bytes(good, 2, 9, ctypes.byref(pb), ctypes.byref(wb)) == sk.EINVAL
    assert L.sketch_group_bytes(items_of([sk.params(64, 512)], align=264), 1, sk.BF16, ctypes.byref(pb),
                                ctypes.byref(wb)) == sk.EINVAL
    # a plan buffer too small, a workspace too small
    assert L.sketch_group_plan(good, 2, sk.BF16, ctypes.c_void_p(256), 64, None) == sk.ESMALL
    assert L.sketch_matmul_group(good, 2, sk.BF16, ctypes.c_void_p(256), ctypes.c_void_p(256), 64,
                                 None) == sk.ESMALL
