"""Helpers shared by the GPU tests: device transfer of synth arrays and the
output tolerance (per element |dY| <= 1e-3 * max(|Y_ref|, rms of the Y_ref row))."""
import numpy as np
import torch

import oracle

RTOL = 1e-3


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda:0")


def to_dev(a, kind):
    """NumPy array -> device tensor: kind 'f32' (float32), 'bf16' or 'f16' (uint16 bit patterns)."""
    a = np.ascontiguousarray(a)
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32)).to(dev())
    t = torch.from_numpy(a.view(np.int16)).to(dev())
    return t.view(torch.bfloat16 if kind == "bf16" else torch.float16)


def oracle_dtype(kind):
    return {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}[kind]


def tables_np(t):
    return t.tables.cpu().numpy().view(np.uint16)


def assert_tables_equal(got, ref, what=""):
    got = np.asarray(got, dtype=np.uint16)
    ref = np.asarray(ref, dtype=np.uint16)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    bad = np.flatnonzero(got.ravel() != ref.ravel())
    assert bad.size == 0, "%s: %d of %d buckets differ; first at %s: got 0x%04x want 0x%04x" % (
        what, bad.size, ref.size, np.unravel_index(bad[0], ref.shape), got.ravel()[bad[0]], ref.ravel()[bad[0]])


def assert_y_close(y_gpu, y_ref, row_rms=None, what=""):
    """Per-element relative tolerance floored at the rms of the reference row."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape
    if row_rms is None:
        row_rms = np.sqrt(np.mean(y_ref ** 2, axis=-1, keepdims=True))
    scale = np.maximum(np.abs(y_ref), row_rms)
    err = np.abs(y_gpu - y_ref)
    ok = err <= RTOL * scale
    if not np.all(ok):
        i = np.unravel_index(np.argmax(err / np.maximum(scale, 1e-300)), y_ref.shape)
        raise AssertionError("%s: %d of %d outputs out of tolerance; worst at %s: got %r want %r (rel %.3g)" % (
            what, (~ok).sum(), ok.size, i, y_gpu[i], y_ref[i], err[i] / scale[i]))
    rel = np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    assert rel < RTOL, (what, rel)
    return rel
