"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tables must match bit for bit; Y must satisfy the per-element tolerance
|Y_gpu - Y_ref| <= 1e-3 * max(|Y_ref|, rms(Y_ref row)) with Y_ref in float64.
Every workload shape is covered at its full size, both selection rules, the
decode batches 1/4/16, the 256-step decoder layer and the 2048-token prefill
(sampled outputs plus whole rows), then ragged shapes, special values, error
paths and determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_tables_equal, assert_y_close, dev, oracle_dtype, tables_np, to_dev

sk = pytest.importorskip("sub_bit_weight_sketch_amd")

pytestmark = pytest.mark.gpu

RULES = [("absmin", oracle.ABSMIN), ("absmax", oracle.ABSMAX)]


def _encode_both(lin, rule_name, rule):
    Wd = to_dev(lin.W, lin.w_dtype)
    imp = torch.from_numpy(lin.imp).to(dev())
    t = sk.encode(Wd, imp, bpw=lin.bpw, seed=lin.seed, R=lin.R, rule=rule_name)
    ref = oracle.encode(lin.W, lin.imp, lin.R, lin.bpw, lin.seed, rule, w_dtype=oracle_dtype(lin.w_dtype))
    assert_tables_equal(tables_np(t), ref, "%s %s" % (lin.name, rule_name))
    return t, ref


def _product_check(t, S_ref, lin, X, x_kind, what):
    Xd = to_dev(X, x_kind)
    Y = sk.matmul(t, Xd).cpu().numpy()
    Yr = oracle.matmul(S_ref, X, lin.M, lin.N, lin.R, lin.bpw, lin.seed, x_dtype=oracle_dtype(x_kind))
    return assert_y_close(Y, Yr, what=what)


# ---------------------------------------------------------------------------
# workload shapes at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rule_name,rule", RULES)
def test_small_linear_256x512(rule_name, rule):
    lin, x = synth.linear_256x512()
    t, S = _encode_both(lin, rule_name, rule)
    _product_check(t, S, lin, x, "f32", "linear_256x512 y")
    X4 = synth.normal_f32((5, lin.N), 1.0, 1777)
    _product_check(t, S, lin, X4, "f32", "linear_256x512 batch 5")


@pytest.mark.parametrize("rule_name,rule", RULES)
def test_attn_4096x4096(rule_name, rule):
    lin, x = synth.attn_4096x4096()
    t, S = _encode_both(lin, rule_name, rule)
    _product_check(t, S, lin, x, "bf16", "attn_4096x4096 b=1")
    # batch 1 sums Z in place; from batch 2 on, Z is summed once into the workspace
    for b in (2, 16):
        X = synth.normal_bf16((b, lin.N), 4100 + b)
        _product_check(t, S, lin, X, "bf16", "attn_4096x4096 b=%d" % b)


@pytest.mark.parametrize("bpw", [0.5, 0.75])
@pytest.mark.parametrize("rule_name,rule", RULES)
def test_mlp_up_11008x4096(bpw, rule_name, rule):
    lin, xs = synth.mlp_up_11008x4096(bpw)
    t, S = _encode_both(lin, rule_name, rule)
    for b in (1, 4, 16):
        _product_check(t, S, lin, xs[b], "bf16", "mlp_up %g bpw %s b=%d" % (bpw, rule_name, b))


@pytest.mark.parametrize("rule_name,rule", RULES)
def test_layer_7b_256_steps(rule_name, rule):
    """Seven linears encoded once under each rule (tables bit-exact); 256
    batch-1 steps with fresh x per linear, through sketch_matmul per linear
    and through one grouped call per step (sketch_matmul_group over the 7).
    Steps 0, 1 and 255 are compared in full, every step on 64 sampled
    outputs per linear, for both paths."""
    g = np.random.default_rng(99 + rule)
    lins, tabs, refs, xds, xs_all, ys1, ys2 = [], [], [], [], [], [], []
    for idx in range(7):
        lin = synth.layer_7b_linear(idx)
        t, S = _encode_both(lin, rule_name, rule)
        xs = synth.layer_7b_tokens(idx)                       # [256, N] bf16 bits
        Xd = to_dev(xs, "bf16")
        ws = sk.workspace_for(t, 1, sk.BF16, dev())
        Y = torch.empty((256, lin.M), dtype=torch.float32, device=dev())
        for s in range(256):
            sk.matmul(t, Xd[s:s + 1], out=Y[s:s + 1], workspace=ws)
        lins.append(lin); tabs.append(t); refs.append(S); xds.append(Xd); xs_all.append(xs); ys1.append(Y)
        ys2.append(torch.full((256, lin.M), float("nan"), dtype=torch.float32, device=dev()))
    for s in range(256):
        sk.Group(tabs, [Xd[s] for Xd in xds], [Y[s] for Y in ys2]).run()
    torch.cuda.synchronize()
    for lin, S, xs, Y1, Y2 in zip(lins, refs, xs_all, ys1, ys2):
        full = [0, 1, 255]
        Yr = oracle.matmul(S, xs[full], lin.M, lin.N, lin.R, lin.bpw, lin.seed, x_dtype=oracle.BF16)
        rms = np.sqrt(np.mean(Yr ** 2))
        ti = np.repeat(np.arange(256), 64)
        ii = g.integers(0, lin.M, size=ti.size)
        ysmp = oracle.matmul_sampled(S, xs, lin.M, lin.N, lin.R, lin.bpw, ti, ii, lin.seed, x_dtype=oracle.BF16)
        for path, Y in (("per linear", Y1), ("grouped", Y2)):
            Y = Y.cpu().numpy()
            assert_y_close(Y[full], Yr, what="%s %s %s full steps" % (lin.name, rule_name, path))
            assert_y_close(Y[ti, ii], ysmp, row_rms=rms, what="%s %s %s sampled steps" % (lin.name, rule_name, path))


@pytest.fixture(scope="module")
def prefill_70b():
    """The 70B-style prefill inputs, generated once for both rules."""
    return synth.mlp_70b_prefill()


# one whole token row in each of the eight 256-token tiles of the 2048-token
# prefill, at different offsets inside the tiles (first, last, inner rows)
PREFILL_ROWS = [0, 300, 600, 767, 1023, 1100, 1290, 1600, 1800, 2047]


@pytest.mark.parametrize("rule_name,rule", RULES)
def test_prefill_70b_28672x8192(prefill_70b, rule_name, rule):
    """Encode the 70B-style MLP weight (R = 16, N = 8192: R*N = 2^17, the
    largest block the packed bucket words take) under each rule, bit-exact,
    and run the 2048-token prefill through the bf16 matrix-core path: one
    whole output row from every 256-token tile plus 16 tokens x 512 sampled
    outputs against the oracle."""
    lin, X = prefill_70b
    t, S = _encode_both(lin, rule_name, rule)
    assert sk.sketch_workspace_bytes(t.params, X.shape[0], sk.BF16) == 0   # GEMM path
    Xd = to_dev(X, "bf16")
    Y = sk.matmul(t, Xd)
    torch.cuda.synchronize()
    assert sorted({r // 256 for r in PREFILL_ROWS}) == list(range(8))
    Yr = oracle.matmul(S, X[PREFILL_ROWS], lin.M, lin.N, lin.R, lin.bpw, lin.seed, x_dtype=oracle.BF16)
    assert_y_close(Y[PREFILL_ROWS].cpu().numpy(), Yr, what="prefill whole rows %s" % rule_name)
    g = np.random.default_rng(5 + rule)
    toks = g.choice(2048, size=16, replace=False)
    ti = np.repeat(toks, 512)
    ii = g.integers(0, lin.M, size=ti.size)
    ys = oracle.matmul_sampled(S, X, lin.M, lin.N, lin.R, lin.bpw, ti, ii, lin.seed, x_dtype=oracle.BF16)
    yg = Y.cpu().numpy()[ti, ii]
    rms = np.sqrt((ys.reshape(16, 512) ** 2).mean(axis=1))
    assert_y_close(yg.reshape(16, 512), ys.reshape(16, 512), row_rms=rms[:, None],
                   what="prefill sampled %s" % rule_name)


@pytest.mark.parametrize("pattern", ["random", "ties", "last_wins"])
@pytest.mark.parametrize("rule_name,rule", RULES)
def test_packed_words_at_the_2_17_limit(pattern, rule_name, rule):
    """Blocks of R*N = 2^17 bfloat16 weights (R = 16, N = 8192) take the
    packed bucket words (31-bit key, 17-bit tie, 16-bit value), whose tie
    field is l for AbsMin and the low 17 bits of ~l for AbsMax, so the
    largest local index 2^17 - 1 gets tie 0 under AbsMax.  "ties": every
    weight of equal magnitude, so each bucket goes to its smallest colliding
    index (the sign shows which); "last_wins": the largest index of every
    block holds the unique extreme magnitude of its bucket under the rule."""
    M, N, R = 32, 8192, 16
    g = np.random.default_rng(2 ** 17 + len(pattern))
    if pattern == "random":
        Wf = (g.standard_normal((M, N)) * 0.05).astype(np.float32)
    elif pattern == "ties":
        Wf = np.where(g.random((M, N)) < 0.5, np.float32(0.375), np.float32(-0.375)).astype(np.float32)
    else:
        Wf = np.where(g.random((M, N)) < 0.5, np.float32(0.25), np.float32(-0.25)).astype(np.float32)
        Wf[R - 1::R, N - 1] = 8.0 if rule == oracle.ABSMAX else 2.0 ** -20
    W = synth.bf16_bits(Wf)
    imp = None if pattern != "random" else synth.uniform_f32(N, 0.5, 1.5, 2 ** 17)
    t = sk.encode(to_dev(W, "bf16"), torch.from_numpy(imp).to(dev()) if imp is not None else None, bpw=0.5,
                  seed=1, R=R, rule=rule_name)
    S = oracle.encode(W, imp, R, 0.5, 1, rule, w_dtype=oracle.BF16)
    assert_tables_equal(tables_np(t), S, "packed 2^17 %s %s" % (pattern, rule_name))
    if pattern == "last_wins":
        # the bucket of the last local index holds that weight in every block
        kmap = oracle.bucket_map(R, N, 1, R * N // 32)
        want = np.uint16(0x4800) if rule == oracle.ABSMAX else np.uint16(0x0010)
        assert np.all(S[:, kmap[-1]] == want)


# ---------------------------------------------------------------------------
# ragged shapes, dtypes, paths
# ---------------------------------------------------------------------------

RAGGED = [
    # M, N, R, bpw, w_kind
    (48, 100, 3, 16 * 25 / 300, "f32"),      # N % 8 != 0 (scalar encode), Bg = 25 (generic product)
    (64, 96, 8, 0.5, "bf16"),                # Bg = 24
    (136, 512, 8, 0.5, "bf16"),              # Bg = 128, 17 blocks (ragged MFMA tile)
    (272, 1024, 16, 0.5, "bf16"),            # R = 16, Bg = 512
    (96, 256, 32, 0.5, "f16"),               # R = 32
    (40, 200, 1, 0.64, "bf16"),              # R = 1, Bg = 8
    (200, 776, 8, 0.5, "f32"),               # N % 16 != 0, Bg = 194
    (384, 1000, 8, 1.024, "bf16"),           # Bg = 512, N % 8 == 0 but not % 16
]


def _rand_w(shape, kind, seed):
    Wf = synth.normal_f32(shape, 0.05, seed)
    if kind == "f32":
        return Wf, Wf
    if kind == "bf16":
        b = synth.bf16_bits(Wf)
        return b, synth.bf16_to_f32(b).reshape(shape)
    h = Wf.astype(np.float16)
    return h.view(np.uint16), h.astype(np.float32)


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "%dx%d_R%d_%s" % (c[0], c[1], c[2], c[4]))
@pytest.mark.parametrize("rule_name,rule", RULES)
def test_ragged_shapes(case, rule_name, rule):
    M, N, R, bpw, kind = case
    W, _ = _rand_w((M, N), kind, 10 + M)
    imp = synth.uniform_f32(N, 0.5, 1.5, 20 + N)
    Wd = to_dev(W, kind)
    t = sk.encode(Wd, torch.from_numpy(imp).to(dev()), bpw=bpw, seed=7, R=R, rule=rule_name)
    S = oracle.encode(W, imp, R, bpw, 7, rule, w_dtype=oracle_dtype(kind))
    assert_tables_equal(tables_np(t), S, "ragged %s" % (case,))
    for b, xk in ((1, "f32"), (3, "bf16"), (16, "f16"), (17, "bf16"), (130, "bf16"), (33, "f32")):
        if xk == "f32":
            X = synth.normal_f32((b, N), 1.0, b)
        else:
            X = synth.normal_bf16((b, N), b)
            if xk == "f16":
                X = synth.bf16_to_f32(X).reshape(b, N).astype(np.float16).view(np.uint16)
        Y = sk.matmul(t, to_dev(X, xk)).cpu().numpy()
        Yr = oracle.matmul(S, X, M, N, R, bpw, 7, x_dtype=oracle_dtype(xk))
        assert_y_close(Y, Yr, what="ragged %s batch %d %s" % (case, b, xk))


@pytest.mark.parametrize("N", [4000, 12000])
def test_generic_product_narrow_and_wide_rows(N):
    """R = 3 (the float32 product after a separate Z pass, which needs a
    workspace) on 24 rows of 4000 and of 12000 columns, batch 1 to 40 with
    float32 and bfloat16 activations, against the oracle."""
    M, R, bpw = 24, 3, 0.5
    W = synth.normal_bf16((M, N), 40 + N % 7)
    t = sk.encode(to_dev(W, "bf16"), None, bpw=bpw, seed=5, R=R)
    S = oracle.encode(W, None, R, bpw, 5, oracle.ABSMIN, w_dtype=oracle.BF16)
    assert_tables_equal(tables_np(t), S, "generic N=%d" % N)
    for b, xk in ((1, "f32"), (3, "bf16"), (17, "f32"), (40, "bf16")):
        X = synth.normal_f32((b, N), 1.0, b) if xk == "f32" else synth.normal_bf16((b, N), b)
        assert sk.sketch_workspace_bytes(t.params, b, sk.F32 if xk == "f32" else sk.BF16) > 0
        Y = sk.matmul(t, to_dev(X, xk)).cpu().numpy()
        Yr = oracle.matmul(S, X, M, N, R, bpw, 5, x_dtype=oracle_dtype(xk))
        assert_y_close(Y, Yr, what="generic N=%d batch %d %s" % (N, b, xk))


@pytest.mark.parametrize("kind", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rule_name,rule", RULES)
def test_encode_of_blocks_beyond_the_lds_copy(kind, rule_name, rule):
    """R = 16 rows of 4096 columns: the 128 KiB (bf16/f16) or 256 KiB (f32)
    block does not fit beside its table at two workgroups per CU.  16-bit
    weights carry their bits in the packed bucket words, float32 ones are
    read again from memory; tables bit-exact, both rules."""
    M, N, R = 64, 4096, 16
    W, _ = _rand_w((M, N), kind, 500 + R)
    imp = synth.uniform_f32(N, 0.5, 1.5, 501)
    t = sk.encode(to_dev(W, kind), torch.from_numpy(imp).to(dev()), bpw=0.5, seed=9, R=R, rule=rule_name)
    S = oracle.encode(W, imp, R, 0.5, 9, rule, w_dtype=oracle_dtype(kind))
    assert_tables_equal(tables_np(t), S, "R16 N4096 %s" % kind)
    X = synth.normal_bf16((3, N), 502)
    Y = sk.matmul(t, to_dev(X, "bf16")).cpu().numpy()
    assert_y_close(Y, oracle.matmul(S, X, M, N, R, 0.5, 9, x_dtype=oracle.BF16), what="R16 N4096 %s" % kind)


STACKED = [
    # M, N, R: at least 8192 row blocks, so Z is staged once per call and every
    # wave streams whole 16-block tiles; R = 4 and 8 combine hi/lo across
    # lanes, R = 16 across column tiles
    (32768, 2048, 4),
    (65536, 1024, 8),
    (131072, 512, 16),
]


@pytest.mark.parametrize("case", STACKED, ids=lambda c: "%dx%d_R%d" % c)
def test_stacked_tables_streaming_path(case):
    M, N, R = case
    W = synth.normal_bf16((M, N), 300 + R)
    imp = synth.uniform_f32(N, 0.5, 1.5, 301 + R)
    t = sk.encode(to_dev(W, "bf16"), torch.from_numpy(imp).to(dev()), bpw=0.5, seed=3, R=R)
    S = oracle.encode(W, imp, R, 0.5, 3, oracle.ABSMIN, w_dtype=oracle.BF16)
    assert_tables_equal(tables_np(t), S, "stacked %s" % (case,))
    for b in (1, 5, 16):
        assert sk.sketch_workspace_bytes(t.params, b, sk.BF16) > 0   # staged-Z mode
        X = synth.normal_bf16((b, N), 302 + b)
        Y = sk.matmul(t, to_dev(X, "bf16")).cpu().numpy()
        Yr = oracle.matmul(S, X, M, N, R, 0.5, 3, x_dtype=oracle.BF16)
        assert_y_close(Y, Yr, what="stacked %s batch %d" % (case, b))


@pytest.mark.parametrize("R", [1, 2, 4, 8, 16, 32])
@pytest.mark.parametrize("shape", ["half", "full", "mixed"])
def test_gemm_tile_every_row_block_size(R, shape):
    """The matrix-core tiles for every power-of-two R they take, with a
    ragged last output tile and a ragged last token tile.  On a 256-CU
    device: "half" has 4 tiles, fewer than half the CUs, so they run as
    256 x 128 tiles (N = 768: three 256-column chunks of the forward map,
    both LDS buffers, one reused); "full" has 160 tiles, more than half the
    CUs, so they run as 256 x 256 tiles; "mixed" has 300 tiles: one whole
    round of 256 x 256 tiles, then the other 44 as 88 tiles of 256 x 128, in
    one call.  The larger shapes are checked on rows from every token tile."""
    rows = np.concatenate([np.arange(0, 8), np.arange(250, 262), np.arange(500, 516), np.arange(760, 776),
                           np.arange(990, 1000)])
    if shape == "half":
        M, T, N, rows = 256 + 4 * R, 300, 768, None
    elif shape == "full":
        M, T, N = 40 * 256 - 4 * R, 1000, 768
    else:
        M, T, N = 75 * 256 - 4 * R, 1000, 1024
    W, _ = _rand_w((M, N), "bf16", 40 + R)
    imp = synth.uniform_f32(N, 0.5, 1.5, 50 + R)
    t = sk.encode(to_dev(W, "bf16"), torch.from_numpy(imp).to(dev()), bpw=0.5, seed=11, R=R)
    S = oracle.encode(W, imp, R, 0.5, 11, oracle.ABSMIN, w_dtype=oracle.BF16)
    assert_tables_equal(tables_np(t), S, "gemm tile R=%d %s" % (R, shape))
    assert sk.sketch_workspace_bytes(t.params, T, sk.BF16) == 0   # GEMM path
    X = synth.normal_bf16((T, N), 60 + R)
    Xd = to_dev(X, "bf16")
    Y = sk.matmul(t, Xd).cpu().numpy()
    if rows is not None:
        Y, X = Y[rows], X[rows]
    Yr = oracle.matmul(S, X, M, N, R, 0.5, 11, x_dtype=oracle.BF16)
    assert_y_close(Y, Yr, what="gemm tile R=%d %s" % (R, shape))


# ---------------------------------------------------------------------------
# decode: W_hat materialised (forward map and per-weight hash)
# ---------------------------------------------------------------------------

def _bf16_rne_bits(f32):
    """bfloat16 bits of float32 values, round to nearest even (finite inputs)."""
    u = np.asarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


DECODE = [
    # M, N, R, bpw, w_kind
    (4096, 4096, 8, 0.5, "bf16"),        # the attention shape
    (272, 1024, 16, 0.5, "bf16"),        # R = 16, 17 blocks (ragged block group)
    (96, 256, 32, 0.5, "f16"),           # R = 32
    (200, 776, 8, 0.5, "f32"),           # N % 16 != 0, float32 buckets (bf16 output rounds)
    (48, 100, 3, 16 * 25 / 300, "f32"),  # N % 8 != 0: scalar paths
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "%dx%d_R%d_%s" % (c[0], c[1], c[2], c[4]))
def test_decode_matches_oracle(case):
    """W_hat = S * P^T element by element: binary16 output equals the bucket
    bits, float32 output its exact value, bfloat16 output its round to
    nearest even; the per-weight hash path gives the same bits."""
    M, N, R, bpw, kind = case
    W, _ = _rand_w((M, N), kind, 70 + M)
    imp = synth.uniform_f32(N, 0.5, 1.5, 80 + N)
    t = sk.encode(to_dev(W, kind), torch.from_numpy(imp).to(dev()), bpw=bpw, seed=5, R=R)
    S = oracle.encode(W, imp, R, bpw, 5, oracle.ABSMIN, w_dtype=oracle_dtype(kind))
    assert_tables_equal(tables_np(t), S, "decode %s" % (case,))
    ref = oracle.decode(S, M, N, R, bpw, 5)                      # float64, every value a binary16 value
    want = {torch.float16: ref.astype(np.float16).view(np.uint16),
            torch.float32: ref.astype(np.float32).view(np.uint32),
            torch.bfloat16: _bf16_rne_bits(ref.astype(np.float32))}
    for dt, bits in want.items():
        for hashed in (False, True):
            got = sk.decode(t, dt, hashed=hashed)
            torch.cuda.synchronize()
            g = got.view(torch.int32 if dt == torch.float32 else torch.int16).cpu().numpy()
            g = g.view(np.uint32 if dt == torch.float32 else np.uint16)
            bad = int((g != bits).sum())
            assert bad == 0, "%s %s hashed=%s: %d of %d differ" % (case, dt, hashed, bad, bits.size)
    if kind == "bf16":   # buckets of bfloat16 weights are exact in bfloat16
        assert np.array_equal(want[torch.bfloat16], (want[torch.float32] >> 16).astype(np.uint16))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16, torch.float16])
def test_decode_with_wrong_projection_is_nan(dt):
    M, N = 64, 512
    W, _ = _rand_w((M, N), "bf16", 91)
    t = sk.encode(to_dev(W, "bf16"), None, bpw=0.5, R=8)
    for other in (sk.projection(sk.params(M, N, 8, 0.5, 2), dev()),       # another seed
                  sk.projection(sk.params(M, N, 16, 0.5, 1), dev())):     # another (larger) shape
        out = torch.empty((M, N), dtype=dt, device=dev())
        sk.sketch_decode(t.params, other, t.tables, out)
        torch.cuda.synchronize()
        assert bool(torch.isnan(out.float()).all())


def test_gemm_and_gemv_paths_agree():
    """batch 17 takes the bf16 GEMM, its 16-token prefix the GEMV: same answers."""
    M, N = 512, 2048
    W, _ = _rand_w((M, N), "bf16", 3)
    Wd = to_dev(W, "bf16")
    t = sk.encode(Wd, None, bpw=0.5, R=8)
    X = to_dev(synth.normal_bf16((17, N), 4), "bf16")
    Y17 = sk.matmul(t, X)
    Y16 = sk.matmul(t, X[:16].contiguous())
    ref = Y16.double()
    err = (Y17[:16].double() - ref).abs()
    rms = ref.pow(2).mean(dim=1, keepdim=True).sqrt()
    assert bool((err <= 2e-3 * torch.maximum(ref.abs(), rms)).all())


def test_special_values_and_ties():
    """Subnormal, signed-zero, tied and huge-but-finite weights; zero importance."""
    g = np.random.default_rng(17)
    pool = np.array([0.0, -0.0, 1e-40, -1e-40, 2.0 ** -24, 3e-8, -6e-8, 0.5, -0.5, 1.0, -1.0, 65504.0,
                     -65519.0, 1e-5, -1e-5, 0.25], dtype=np.float32)
    M, N, R = 64, 128, 8
    W = pool[g.integers(0, pool.size, size=(M, N))]
    imp = g.choice(np.array([0.0, -0.0, 1.0, 0.5, 2.0], dtype=np.float32), size=N)
    for rule_name, rule in RULES:
        t = sk.encode(to_dev(W, "f32"), torch.from_numpy(imp).to(dev()), bpw=0.5, R=R, rule=rule_name)
        S = oracle.encode(W, imp, R, 0.5, 1, rule)
        assert_tables_equal(tables_np(t), S, "special values " + rule_name)
        # bfloat16 rounds 65504 and -65519 up to 65536 (out of binary16 range): keep them out
        Wb = synth.bf16_bits(np.where(np.abs(W) > 60000, np.float32(0.75), W))
        t = sk.encode(to_dev(Wb, "bf16"), None, bpw=0.5, R=R, rule=rule_name)
        S = oracle.encode(Wb, None, R, 0.5, 1, rule, w_dtype=oracle.BF16)
        assert_tables_equal(tables_np(t), S, "special values bf16 " + rule_name)


def test_tiny_and_huge_activations_scale():
    """Activation scales far from 1 still meet the tolerance (per-token scaling of Z)."""
    M, N = 256, 1024
    W, _ = _rand_w((M, N), "bf16", 8)
    t = sk.encode(to_dev(W, "bf16"), None, bpw=0.5, R=8)
    S = oracle.encode(W, None, 8, 0.5, 1, w_dtype=oracle.BF16)
    for scale in (1e-30, 1e-6, 1e4, 1e30):
        X = (synth.normal_f32((2, N), 1.0, 6) * np.float32(scale)).astype(np.float32)
        Y = sk.matmul(t, to_dev(X, "f32")).cpu().numpy()
        Yr = oracle.matmul(S, X, M, N, 8, 0.5, 1)
        assert_y_close(Y, Yr, what="activation scale %g" % scale)


def test_nonfinite_activations_propagate():
    M, N = 64, 256
    W, _ = _rand_w((M, N), "bf16", 9)
    t = sk.encode(to_dev(W, "bf16"), None, bpw=0.5, R=8)
    X = synth.normal_f32((2, N), 1.0, 7)
    X[1, 5] = np.nan
    Y = sk.matmul(t, to_dev(X, "f32")).cpu().numpy()
    assert np.all(np.isfinite(Y[0]))
    S = oracle.encode(W, None, 8, 0.5, 1, w_dtype=oracle.BF16)
    Yr = oracle.matmul(S, X, M, N, 8, 0.5, 1)
    assert np.array_equal(np.isnan(Y[1]), np.isnan(Yr[1]))
    assert_y_close(Y[:1], Yr[:1], what="finite token next to a NaN token")


# ---------------------------------------------------------------------------
# errors, empty inputs, determinism
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf, 65520.0, -1e6])
def test_encode_rejects_out_of_range_weights(bad):
    W = synth.normal_f32((16, 64), 0.1, 1)
    W[5, 7] = bad
    with pytest.raises(sk.SketchError) as e:
        sk.encode(to_dev(W, "f32"), None, bpw=0.5, R=8)
    assert e.value.code == sk.ERANGE
    with pytest.raises(oracle.OracleError):
        oracle.encode(W, None, 8, 0.5, 1)


def test_bf16_rounding_to_65536_is_rejected_on_both_sides():
    W = np.full((16, 64), 0.5, dtype=np.float32)
    W[2, 3] = 65504.0
    Wb = synth.bf16_bits(W)                 # 65504 -> bf16 65536
    with pytest.raises(sk.SketchError) as e:
        sk.encode(to_dev(Wb, "bf16"), None, bpw=0.5, R=8)
    assert e.value.code == sk.ERANGE
    with pytest.raises(oracle.OracleError):
        oracle.encode(Wb, None, 8, 0.5, 1, w_dtype=oracle.BF16)


@pytest.mark.parametrize("bad", [-1.0, np.nan, np.inf])
def test_encode_rejects_bad_importance(bad):
    W = synth.normal_f32((16, 64), 0.1, 1)
    imp = np.ones(64, dtype=np.float32)
    imp[3] = bad
    with pytest.raises(sk.SketchError) as e:
        sk.encode(to_dev(W, "f32"), torch.from_numpy(imp).to(dev()), bpw=0.5, R=8)
    assert e.value.code == sk.EINVAL


def test_projection_mismatch_is_loud():
    W = to_dev(synth.normal_f32((16, 64), 0.1, 1), "f32")
    p_good = sk.params(16, 64, 8, 0.5, 1, sk.ABSMIN, sk.F32)
    p_other = sk.params(16, 64, 8, 0.5, 2, sk.ABSMIN, sk.F32)   # other seed
    proj_other = sk.projection(p_other, dev())
    tables = torch.empty((2, 16), dtype=torch.int16, device=dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    sk.sketch_encode(p_good, proj_other, W, None, tables, status)
    assert int(status.item()) & sk.FLAG_PROJECTION
    # product with a projection of another shape (at least as large as this
    # shape's, the documented condition): every output NaN
    p_shape = sk.params(16, 64, 16, 0.5, 1, sk.ABSMIN, sk.F32)
    proj_shape = sk.projection(p_shape, dev())
    good = sk.encode(W, None, bpw=0.5, R=8)
    bad = sk.Tables(good.params, good.tables, proj_shape)
    Y = sk.matmul(bad, to_dev(synth.normal_f32((1, 64), 1.0, 2), "f32"))
    assert bool(torch.isnan(Y).all())


@pytest.mark.parametrize("batch", [1, 5, 17])
def test_projection_of_another_seed_gives_nan(batch):
    """A projection built with another hash seed: every product path (batch
    1 and 5 on the decode product, 17 bf16 tokens on the matrix cores) and
    decode give NaN everywhere instead of a silently wrong answer."""
    M, N = 512, 1024
    W, _ = _rand_w((M, N), "bf16", 93)
    t = sk.encode(to_dev(W, "bf16"), None, bpw=0.5, R=8)
    other = sk.projection(sk.params(M, N, 8, 0.5, 2, sk.ABSMIN, sk.BF16), dev())   # seed 2
    bad = sk.Tables(t.params, t.tables, other)
    X = to_dev(synth.normal_bf16((batch, N), 94), "bf16")
    Y = sk.matmul(bad, X)
    torch.cuda.synchronize()
    assert bool(torch.isnan(Y).all())
    assert bool(torch.isfinite(sk.matmul(t, X)).all())


def test_empty_inputs():
    W = torch.empty((0, 64), dtype=torch.bfloat16, device=dev())
    t = sk.encode(W, None, bpw=0.5, R=8)
    assert t.tables.shape == (0, 16)
    Y = sk.matmul(t, torch.zeros((3, 64), dtype=torch.bfloat16, device=dev()))
    assert Y.shape == (3, 0)
    W = to_dev(synth.bf16_bits(synth.normal_f32((16, 64), 0.1, 1)), "bf16")
    t = sk.encode(W, None, bpw=0.5, R=8)
    Y = sk.matmul(t, torch.zeros((0, 64), dtype=torch.bfloat16, device=dev()))
    assert Y.shape == (0, 16)


def test_determinism_and_stream_independence():
    lin, x = synth.attn_4096x4096()
    Wd = to_dev(lin.W, "bf16")
    imp = torch.from_numpy(lin.imp).to(dev())
    t1 = sk.encode(Wd, imp, bpw=0.5, R=8)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        t2 = sk.encode(Wd, imp, bpw=0.5, R=8)
    s.synchronize()
    assert torch.equal(t1.tables, t2.tables)
    X = to_dev(synth.normal_bf16((4, 4096), 3), "bf16")
    assert torch.equal(sk.matmul(t1, X), sk.matmul(t1, X))
    X = to_dev(synth.normal_bf16((64, 4096), 3), "bf16")
    assert torch.equal(sk.matmul(t1, X), sk.matmul(t1, X))


def test_graph_replay_matches_eager():
    """encode + product captured in a HIP graph: every replay (with eager work
    and synchronisations in between) reproduces the eager results bit for bit."""
    lin, x = synth.attn_4096x4096()
    Wd = to_dev(lin.W, "bf16")
    imp = torch.from_numpy(lin.imp).to(dev())
    X = to_dev(synth.normal_bf16((1, lin.N), 31), "bf16")
    ref = sk.encode(Wd, imp, bpw=0.5, R=8)
    y_ref = sk.matmul(ref, X)
    p = ref.params
    tables = torch.zeros_like(ref.tables)
    y = torch.zeros_like(y_ref)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    ws = sk.workspace_for(ref, 1, sk.BF16, dev())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sh = sk._stream_handle(dev())
        sk.sketch_encode(p, ref.proj, Wd, imp, tables, status, sh)
        sk.sketch_matmul(p, ref.proj, tables, X, y, ws, sh)
    other = to_dev(synth.bf16_bits(synth.normal_f32((4096, 4096), 0.02, 5)), "bf16")
    for rep in range(3):
        tables.zero_()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(tables, ref.tables), rep
        assert torch.equal(y, y_ref), rep
        sk.encode(other, None, bpw=0.5, R=8)      # eager work between replays
    assert int(status.item()) == 0


def test_encode_without_status_word_waits_and_reports():
    """sketch_encode with status_dev == NULL: the call waits for its stream
    and returns the flags as a status -- OK with tables equal to the
    oracle's, SKETCH_ERANGE for a NaN weight, SKETCH_EINVAL for a negative
    importance -- and a later call starts from a clear word."""
    M, N = 16, 64
    W = synth.normal_f32((M, N), 0.1, 12)
    p = sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.F32)
    proj = sk.projection(p, dev())
    tables = torch.empty((2, 16), dtype=torch.int16, device=dev())
    sk.sketch_encode(p, proj, to_dev(W, "f32"), None, tables, None)
    assert_tables_equal(tables.cpu().numpy().view(np.uint16), oracle.encode(W, None, 8, 0.5, 1), "status NULL")
    bad = W.copy()
    bad[3, 9] = np.nan
    with pytest.raises(sk.SketchError) as e:
        sk.sketch_encode(p, proj, to_dev(bad, "f32"), None, tables, None)
    assert e.value.code == sk.ERANGE
    imp = np.ones(N, dtype=np.float32)
    imp[7] = -1.0
    with pytest.raises(sk.SketchError) as e:
        sk.sketch_encode(p, proj, to_dev(W, "f32"), torch.from_numpy(imp).to(dev()), tables, None)
    assert e.value.code == sk.EINVAL
    sk.sketch_encode(p, proj, to_dev(W, "f32"), None, tables, None)   # the word was cleared again
