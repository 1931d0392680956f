"""GPU parity of the 4-bit bucket sketch ("Resumen Técnico" › Resultados:
0.5 bits per weight combined with 4-bit quantization) against the oracle:
codes and scales bit-exact, decoded weights bit-exact, products within the
1e-3 relative tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y_close, dev, oracle_dtype, to_dev

import sub_bit_weight_sketch_amd as sk

pytestmark = pytest.mark.gpu


def _w(shape, kind, seed, std=0.05):
    Wf = synth.normal_f32(shape, std, seed)
    if kind == "f32":
        return Wf
    if kind == "bf16":
        return synth.bf16_bits(Wf)
    return Wf.astype(np.float16).view(np.uint16)


def _split(t):
    """(codes uint8[nb, Bg/2], scales uint16[nb]) from the GPU tables buffer."""
    torch.cuda.synchronize()
    nb, bg, tb = sk.sketch_layout(t.params)
    raw = t.tables.cpu().numpy()
    off = ((nb * bg // 2 + 255) // 256) * 256
    return raw[:nb * bg // 2].reshape(nb, bg // 2), raw[off:off + 2 * nb].view(np.uint16)


def _bf16_rne_bits(f32):
    u = np.asarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


CASES = [
    # M, N, R, bpw, w kind
    (256, 512, 8, 0.5, "f32"),
    (272, 1024, 16, 0.5, "bf16"),
    (48, 100, 4, 0.64, "f32"),      # N % 8 != 0: the scalar paths
    (96, 256, 32, 0.5, "f16"),
    (64, 264, 8, 0.5, "bf16"),      # N % 256 != 0: prefill on the per-weight-decode GEMM
    (64, 2048, 16, 0.5, "f16"),     # 32 KiB table + 64 KiB block: encode with packed words
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%d_R%d_%s" % (c[0], c[1], c[2], c[4]))
@pytest.mark.parametrize("rule_name,rule", [("absmin", oracle.ABSMIN), ("absmax", oracle.ABSMAX)])
def test_q4_encode_decode_product(case, rule_name, rule):
    M, N, R, bpw, kind = case
    W = _w((M, N), kind, 7 + M)
    imp = synth.uniform_f32(N, 0.5, 1.5, 8 + N)
    t = sk.encode(to_dev(W, kind), torch.from_numpy(imp).to(dev()), bpw=bpw, seed=3, R=R, rule=rule_name, bits=4)
    T, sc = oracle.encode_q4(W, imp, R, bpw, 3, rule, w_dtype=oracle_dtype(kind))
    Tg, scg = _split(t)
    assert np.array_equal(scg, sc), "scales"
    bad = int((Tg != T).sum())
    assert bad == 0, "%d of %d code bytes differ" % (bad, T.size)
    ref = oracle.decode_q4(T, sc, M, N, R, bpw, 3)
    want = {torch.float16: ref.astype(np.float16).view(np.uint16),
            torch.float32: ref.astype(np.float32).view(np.uint32),
            torch.bfloat16: _bf16_rne_bits(ref.astype(np.float32))}
    for dt, bits in want.items():
        for hashed in (False, True):
            out = sk.decode(t, dt, hashed=hashed)
            torch.cuda.synchronize()
            g = out.view(torch.int32 if dt == torch.float32 else torch.int16).cpu().numpy()
            g = g.view(np.uint32 if dt == torch.float32 else np.uint16)
            assert int((g != bits).sum()) == 0, (dt, hashed)
    batches = [(1, "f32"), (5, "bf16"), (16, "f16")]
    if N % 8 == 0:
        batches += [(17, "bf16"), (300, "bf16")]
    for b, xk in batches:
        X = synth.normal_f32((b, N), 1.0, b) if xk == "f32" else synth.normal_bf16((b, N), b)
        if xk == "f16":
            X = synth.bf16_to_f32(X).reshape(b, N).astype(np.float16).view(np.uint16)
        Y = sk.matmul(t, to_dev(X, xk)).cpu().numpy()
        Yr = oracle.matmul_q4(T, sc, X, M, N, R, bpw, 3, x_dtype=oracle_dtype(xk))
        assert_y_close(Y, Yr, what="q4 %s batch %d %s" % (case, b, xk))


@pytest.mark.parametrize("T_", [1, 2048])
def test_q4_attention_shape(T_):
    """attn_4096x4096 at 0.5 bpw with 4-bit buckets (4096 per block): codes
    and scales bit-exact; the batch-1 product in full, the 2048-token product
    on 16 tokens x 256 sampled outputs."""
    M = N = 4096
    W = synth.student_t_bf16((M, N), 0.02, 91)
    imp = synth.uniform_f32(N, 0.5, 1.5, 92)
    t = sk.encode(to_dev(W, "bf16"), torch.from_numpy(imp).to(dev()), bpw=0.5, seed=1, R=8, bits=4)
    T, sc = oracle.encode_q4(W, imp, 8, 0.5, 1, w_dtype=oracle.BF16)
    Tg, scg = _split(t)
    assert np.array_equal(scg, sc) and np.array_equal(Tg, T)
    X = synth.normal_bf16((T_, N), 93)
    Y = sk.matmul(t, to_dev(X, "bf16")).cpu().numpy()
    if T_ == 1:
        assert_y_close(Y, oracle.matmul_q4(T, sc, X, M, N, 8, 0.5, 1, x_dtype=oracle.BF16), what="q4 attention b1")
        return
    g = np.random.default_rng(94)
    toks = g.choice(T_, size=16, replace=False)
    ti = np.repeat(toks, 256)
    ii = g.integers(0, M, size=ti.size)
    ys = oracle.matmul_sampled_q4(T, sc, X, M, N, 8, 0.5, ti, ii, 1, x_dtype=oracle.BF16)
    rms = np.sqrt((ys.reshape(16, 256) ** 2).mean(axis=1))
    assert_y_close(Y[ti, ii].reshape(16, 256), ys.reshape(16, 256), row_rms=rms[:, None], what="q4 attention T2048")


def test_q4_with_the_projection_of_another_bucket_count_is_nan():
    """The binary16 sketch's projection for a quarter of the buckets (same
    R, N, seed; a smaller buffer, of which only the header is read): encode
    flags it, decode and products are NaN."""
    M, N, R = 64, 512, 8
    Wd = to_dev(_w((M, N), "bf16", 101), "bf16")
    p = sk.params(M, N, R, 0.5, 1, sk.ABSMIN, sk.BF16, bits=4)
    other = sk.projection(sk.params(M, N, R, 0.5, 1, sk.ABSMIN, sk.BF16), dev())
    nb, bg, tb = sk.sketch_layout(p)
    tables = torch.zeros(tb, dtype=torch.uint8, device=dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    sk.sketch_encode(p, other, Wd, None, tables, status)
    torch.cuda.synchronize()
    assert int(status.item()) & sk.FLAG_PROJECTION
    t = sk.Tables(p, tables, other)
    assert bool(torch.isnan(sk.decode(t, torch.float32)).all())
    for b in (1, 40):
        Y = sk.matmul(t, to_dev(synth.normal_bf16((b, N), 102), "bf16"))
        torch.cuda.synchronize()
        assert bool(torch.isnan(Y).all()), b
