"""GPU parity of the grouped decode product (sketch_group_plan +
sketch_matmul_group, through the C ABI): every item's y against the oracle's
product of its tables and its own token, with the per-element tolerance
|dY| <= 1e-3 * max(|Y_ref|, rms(Y_ref)); tables are checked bit-exact first."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_tables_equal, assert_y_close, dev, oracle_dtype, tables_np, to_dev

sk = pytest.importorskip("sub_bit_weight_sketch_amd")

pytestmark = pytest.mark.gpu


def _encode(W, kind, imp, R, bpw, seed, rule="absmin"):
    M, N = W.shape
    t = sk.encode(to_dev(W, kind), torch.from_numpy(imp).to(dev()) if imp is not None else None, bpw=bpw, seed=seed,
                  R=R, rule=rule)
    S = oracle.encode(W, imp, R, bpw, seed, oracle.ABSMIN if rule == "absmin" else oracle.ABSMAX,
                      w_dtype=oracle_dtype(kind))
    assert_tables_equal(tables_np(t), S, "group item %dx%d R=%d" % (M, N, R))
    return t, S


def _check_group(entries, xk, what):
    """entries: (Tables, S_ref, x numpy [N], seed).  Runs the group and checks every y."""
    xs = [to_dev(x[None, :], xk)[0] for (_, _, x, _) in entries]
    ys = [torch.full((t.params.M,), float("nan"), dtype=torch.float32, device=dev()) for (t, _, _, _) in entries]
    g = sk.Group([t for (t, _, _, _) in entries], xs, ys)
    g.run()
    torch.cuda.synchronize()
    for i, ((t, S, x, seed), y) in enumerate(zip(entries, ys)):
        p = t.params
        yr = oracle.matmul(S, x[None, :], p.M, p.N, p.R, p.bpw, seed, x_dtype=oracle_dtype(xk))[0]
        assert_y_close(y.cpu().numpy(), yr, what="%s item %d (%dx%d R=%d)" % (what, i, p.M, p.N, p.R))
    return g, xs, ys


def test_group_plan_holds_the_items_and_balanced_wave_ranges():
    """The planner alone: the plan copied back holds every item's pointers
    and geometry, wave ranges that cover the tile order in sequence, each
    starting inside the item recorded with it, and the linear of every Z
    workgroup (64 buckets each: the group has fewer than 256 slices of 256
    buckets)."""
    import struct
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)] + [(8 * (1 + i % 39), 512) for i in range(40)]
    keep = []
    for (M, N) in shapes:
        p = sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.BF16)
        nb, bg, _ = sk.sketch_layout(p)
        keep.append((p, sk.projection(p, dev()), torch.zeros((nb, bg), dtype=torch.int16, device=dev()),
                     torch.zeros(N, dtype=torch.bfloat16, device=dev()), torch.zeros(M, dtype=torch.float32, device=dev())))
    items = sk.group_items(keep)
    pb, _ = sk.sketch_group_bytes(items, sk.BF16)
    plan = torch.full((pb,), 0xAB, dtype=torch.uint8, device=dev())
    sk.sketch_group_plan(items, sk.BF16, plan)
    h = plan.cpu().numpy().tobytes()
    magic, count, ntiles, nwaves, nfrag, xdt, nzb, tb, bits, pieces, rows, zs = struct.unpack_from("<12I", h, 0)
    assert (magic, count, xdt, bits) == (0x50524753, len(shapes), sk.BF16, 16) and tb % 16 == 0
    assert sum((sk.sketch_layout(p)[1] + 255) // 256 for p, *_ in keep) < 256 and zs == 64
    assert rows == sum(M for M, _ in shapes)
    a256 = lambda v: (v + 255) & ~255
    tile0 = frag0 = zb0 = 0
    spans, zb_want = [], []
    for i, (p, proj, tables, x, y) in enumerate(keep):
        f = struct.unpack_from("<7Q8I", h, 256 + 96 * i)
        nb, bg, _ = sk.sketch_layout(p)
        assert f[:4] == (tables.data_ptr(), x.data_ptr(), y.data_ptr(), proj.data_ptr()), i
        assert f[6] == 0, i   # no block scales: binary16 buckets
        assert f[7:15] == (p.N, p.R, bg, p.seed, nb, tile0, frag0, zb0), i
        spans.append((tile0, (nb + tb - 1) // tb))
        zb_want += [i] * ((bg + zs - 1) // zs)
        zb0 += (bg + zs - 1) // zs
        tile0 += (nb + tb - 1) // tb
        frag0 += bg // 32 * 64
    assert (ntiles, nfrag, nzb) == (tile0, frag0, zb0)
    L_wt = a256(256 + 96 * count)
    wt = np.frombuffer(h, dtype=np.uint32, count=nwaves + 1, offset=L_wt).astype(np.int64)
    L_wi = a256(L_wt + 4 * (nwaves + 1))
    wi = np.frombuffer(h, dtype=np.uint32, count=nwaves, offset=L_wi)
    zbi = np.frombuffer(h, dtype=np.uint32, count=nzb, offset=a256(L_wi + 4 * nwaves))
    assert zbi.tolist() == zb_want
    assert wt[0] == 0 and wt[-1] == ntiles and np.all(np.diff(wt) >= 0)
    for v in range(nwaves):
        if wt[v] < ntiles:
            t0, nt = spans[int(wi[v])]
            assert t0 <= wt[v] < t0 + nt, v


def test_group_decoder_layer_three_steps():
    """The seven linears of the 7B-style decoder layer (4096x4096 x4,
    11008x4096 x2, 4096x11008), one token step each with fresh x per
    linear, as one group per step."""
    entries_base = []
    for idx in range(7):
        lin = synth.layer_7b_linear(idx)
        t, S = _encode(lin.W, "bf16", lin.imp, lin.R, lin.bpw, lin.seed)
        entries_base.append((t, S, synth.layer_7b_tokens(idx, steps=3), lin.seed))
    for s in range(3):
        entries = [(t, S, xs[s], seed) for (t, S, xs, seed) in entries_base]
        _check_group(entries, "bf16", "layer step %d" % s)


MIXED = [
    # M, N, R, bpw: Bg = R*N*bpw/16 a multiple of 32
    (2 * 16 * 3 + 2, 4096, 2, 0.5),        # R = 2, Bg = 256, a ragged last tile
    (4 * 37, 2048, 4, 0.5),                # R = 4, Bg = 256
    (8 * 20, 3000, 8, 16 * 96 / 24000),    # R = 8, N % 8 != 0, Bg = 96
    (8 * 16 * 5, 11008, 8, 0.5),           # Bg = 2752: chunks of 8 K-steps with a partial last one
    (8 * 3, 512, 8, 1.0),                  # Bg = 256, a single partial tile
]


@pytest.mark.parametrize("xk", ["bf16", "f16", "f32"])
def test_group_mixed_shapes_and_dtypes(xk):
    entries = []
    for i, (M, N, R, bpw) in enumerate(MIXED):
        W = synth.normal_bf16((M, N), 800 + i)
        imp = synth.uniform_f32(N, 0.5, 1.5, 810 + i)
        t, S = _encode(W, "bf16", imp, R, bpw, 3 + i)
        x = synth.normal_f32((1, N), 1.0, 820 + i)[0] if xk == "f32" else synth.normal_bf16((1, N), 820 + i)[0]
        if xk == "f16":
            x = synth.bf16_to_f32(x).astype(np.float16).view(np.uint16)
        entries.append((t, S, x, 3 + i))
    _check_group(entries, xk, "mixed %s" % xk)


def test_group_many_small_items_both_rules():
    """300 small linears: each wave's range of tiles crosses many items."""
    entries = []
    g = np.random.default_rng(31)
    for i in range(300):
        M = 8 * int(g.integers(1, 40))
        W = synth.normal_bf16((M, 512), 900 + i)
        t, S = _encode(W, "bf16", None, 8, 0.5, 1 + i % 3, rule="absmax" if i % 2 else "absmin")
        entries.append((t, S, synth.normal_bf16((1, 512), 1900 + i)[0], 1 + i % 3))
    _check_group(entries, "bf16", "many items")


def test_group_projection_of_another_seed_gives_nan_for_that_item_only():
    W0, W1 = synth.normal_bf16((256, 1024), 41), synth.normal_bf16((128, 1024), 42)
    t0, S0 = _encode(W0, "bf16", None, 8, 0.5, 1)
    t1, _ = _encode(W1, "bf16", None, 8, 0.5, 1)
    wrong = sk.projection(sk.params(128, 1024, 8, 0.5, 2, sk.ABSMIN, sk.BF16), dev())   # seed 2
    bad = sk.Tables(t1.params, t1.tables, wrong)
    x0, x1 = synth.normal_bf16((1, 1024), 43)[0], synth.normal_bf16((1, 1024), 44)[0]
    xs = [to_dev(x0[None], "bf16")[0], to_dev(x1[None], "bf16")[0]]
    ys = [torch.zeros(256, dtype=torch.float32, device=dev()), torch.zeros(128, dtype=torch.float32, device=dev())]
    sk.Group([t0, bad], xs, ys).run()
    torch.cuda.synchronize()
    assert bool(torch.isnan(ys[1]).all())
    yr = oracle.matmul(S0, x0[None], 256, 1024, 8, 0.5, 1, x_dtype=oracle.BF16)[0]
    assert_y_close(ys[0].cpu().numpy(), yr, what="good item next to a bad one")


def test_group_nonfinite_x_stays_in_its_item():
    W = synth.normal_bf16((128, 1024), 51)
    t, S = _encode(W, "bf16", None, 8, 0.5, 1)
    x0 = synth.normal_f32((1, 1024), 1.0, 52)[0]
    x1 = x0.copy()
    x1[17] = np.nan
    xs = [to_dev(x0[None], "f32")[0], to_dev(x1[None], "f32")[0]]
    ys = [torch.zeros(128, dtype=torch.float32, device=dev()) for _ in range(2)]
    sk.Group([t, t], xs, ys).run()
    torch.cuda.synchronize()
    yr = oracle.matmul(S, x0[None], 128, 1024, 8, 0.5, 1)[0]
    assert_y_close(ys[0].cpu().numpy(), yr, what="finite item")
    assert not bool(torch.isfinite(ys[1]).all())


def test_group_keeps_the_buffers_its_plan_names():
    """A Group whose tables and xs are otherwise unreferenced (built inside a
    function that returns only the group and its ys): after a garbage
    collection and torch.cuda.empty_cache() -- which capturing a graph also
    calls -- the plan's pointers still name live memory and the products
    still match the oracle."""
    import gc
    refs = []

    def make():
        tabs, xs, ys = [], [], []
        for i, (M, N) in enumerate(((256, 1024), (512, 2048))):
            W = synth.normal_bf16((M, N), 150 + i)
            t, S = _encode(W, "bf16", None, 8, 0.5, 1)
            x = synth.normal_bf16((1, N), 160 + i)[0]
            refs.append((S, x, M, N))
            tabs.append(t)
            xs.append(to_dev(x[None], "bf16")[0])
            ys.append(torch.zeros(M, dtype=torch.float32, device=dev()))
        return sk.Group(tabs, xs, ys), ys

    grp, ys = make()
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    grp.run()
    torch.cuda.synchronize()
    for (S, x, M, N), y in zip(refs, ys):
        yr = oracle.matmul(S, x[None], M, N, 8, 0.5, 1, x_dtype=oracle.BF16)[0]
        assert_y_close(y.cpu().numpy(), yr, what="group built in a function, %dx%d" % (M, N))


def test_group_graph_replay_matches_eager():
    """plan + products captured in a HIP graph; every replay (eager work and
    synchronisations in between, x refilled) reproduces the eager result."""
    tabs, xs_np = [], []
    for i, (M, N) in enumerate(((512, 4096), (1376, 4096), (256, 11008))):
        W = synth.normal_bf16((M, N), 60 + i)
        t, _ = _encode(W, "bf16", None, 8, 0.5, 1)
        tabs.append(t)
        xs_np.append([synth.normal_bf16((1, N), 70 + 10 * i + r)[0] for r in range(3)])
    xs = [torch.empty(t.params.N, dtype=torch.bfloat16, device=dev()) for t in tabs]
    ys = [torch.empty(t.params.M, dtype=torch.float32, device=dev()) for t in tabs]
    grp = sk.Group(tabs, xs, ys)
    refs = []
    for r in range(3):
        for x, xn in zip(xs, xs_np):
            x.copy_(to_dev(xn[r][None], "bf16")[0])
        grp.run()
        torch.cuda.synchronize()
        refs.append([y.clone() for y in ys])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        grp.run(sk._stream_handle(dev()))
    for r in range(3):
        for x, xn in zip(xs, xs_np):
            x.copy_(to_dev(xn[r][None], "bf16")[0])
        for y in ys:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for y, yr in zip(ys, refs[r]):
            assert torch.equal(y, yr), r
        sk.matmul(tabs[0], xs[0][None])          # eager work between replays


# ---------------------------------------------------------------- 4-bit codes
def _encode_q4(W, kind, imp, R, bpw, seed, rule="absmin"):
    """4-bit sketch on the GPU; codes and block scales bit-exact against the
    oracle's ("Resumen Técnico" › Resultados: 0.5 bpw with 4-bit codes)."""
    M, N = W.shape
    t = sk.encode(to_dev(W, kind), torch.from_numpy(imp).to(dev()) if imp is not None else None, bpw=bpw, seed=seed,
                  R=R, rule=rule, bits=4)
    T, sc = oracle.encode_q4(W, imp, R, bpw, seed, oracle.ABSMIN if rule == "absmin" else oracle.ABSMAX,
                             w_dtype=oracle_dtype(kind))
    torch.cuda.synchronize()
    nb, bg, _ = sk.sketch_layout(t.params)
    raw = t.tables.cpu().numpy().view(np.uint8)
    off = ((nb * bg // 2 + 255) // 256) * 256
    assert np.array_equal(raw[:nb * bg // 2].reshape(nb, bg // 2), T), "codes %dx%d R=%d" % (M, N, R)
    assert np.array_equal(raw[off:off + 2 * nb].view(np.uint16), sc), "scales %dx%d R=%d" % (M, N, R)
    return t, (T, sc)


def _check_group_q4(entries, xk, what):
    """entries: (Tables, (codes, scales), x numpy [N], seed); every y against
    the oracle's 4-bit product of its own token."""
    xs = [to_dev(x[None, :], xk)[0] for (_, _, x, _) in entries]
    ys = [torch.full((t.params.M,), float("nan"), dtype=torch.float32, device=dev()) for (t, _, _, _) in entries]
    g = sk.Group([t for (t, _, _, _) in entries], xs, ys)
    g.run()
    torch.cuda.synchronize()
    for i, ((t, (T, sc), x, seed), y) in enumerate(zip(entries, ys)):
        p = t.params
        yr = oracle.matmul_q4(T, sc, x[None, :], p.M, p.N, p.R, p.bpw, seed, x_dtype=oracle_dtype(xk))[0]
        assert_y_close(y.cpu().numpy(), yr, what="%s item %d (%dx%d R=%d)" % (what, i, p.M, p.N, p.R))
    return g, xs, ys


Q4_SHAPES = [
    # M, N, R, bpw: Bg = R*N*bpw/4 codes per block, a multiple of 128
    (4096, 4096, 8, 0.5),        # 512 blocks: 8 tiles of 64, 16 chunks of 256 codes each
    (8 * 71, 1024, 8, 0.5),      # 71 blocks: a ragged last tile
    (2 * 100, 2048, 2, 0.5),     # R = 2, Bg = 512
    (4 * 33, 1536, 4, 0.5),      # R = 4, Bg = 768: three whole chunks
    (8 * 9, 640, 8, 0.5),        # Bg = 640: a last chunk of 4 of its 8 K-steps
    (8 * 5, 11008, 8, 0.5),      # Bg = 11008 codes, 5 blocks
]


@pytest.mark.parametrize("xk", ["bf16", "f16", "f32"])
def test_group_q4_items_match_the_oracle(xk):
    entries = []
    for i, (M, N, R, bpw) in enumerate(Q4_SHAPES):
        W = synth.normal_bf16((M, N), 1200 + i)
        imp = synth.uniform_f32(N, 0.5, 1.5, 1210 + i)
        t, ref = _encode_q4(W, "bf16", imp, R, bpw, 5 + i, rule="absmax" if i % 2 else "absmin")
        x = synth.normal_f32((1, N), 1.0, 1220 + i)[0] if xk == "f32" else synth.normal_bf16((1, N), 1220 + i)[0]
        if xk == "f16":
            x = synth.bf16_to_f32(x).astype(np.float16).view(np.uint16)
        entries.append((t, ref, x, 5 + i))
    _check_group_q4(entries, xk, "q4 %s" % xk)


def test_group_q4_decoder_layer():
    """The seven linears of the 7B-style decoder layer with 4-bit codes at
    0.5 bpw, one token each, as one group."""
    entries = []
    for idx in range(7):
        lin = synth.layer_7b_linear(idx)
        t, ref = _encode_q4(lin.W, "bf16", lin.imp, lin.R, lin.bpw, lin.seed)
        entries.append((t, ref, synth.layer_7b_tokens(idx, steps=1)[0], lin.seed))
    _check_group_q4(entries, "bf16", "q4 layer")


def test_group_q4_plan_records_block_scales():
    """The plan of a 4-bit group: header with 4-bit buckets and 64-block
    tiles; each item's scale pointer is where the tables buffer keeps the
    block scales."""
    import struct
    keep = []
    for (M, N) in ((4096, 4096), (8 * 71, 1024)):
        p = sk.params(M, N, 8, 0.5, 1, sk.ABSMIN, sk.BF16, bits=4)
        nb, bg, tb = sk.sketch_layout(p)
        keep.append((p, sk.projection(p, dev()), torch.zeros(tb, dtype=torch.uint8, device=dev()),
                     torch.zeros(N, dtype=torch.bfloat16, device=dev()), torch.zeros(M, dtype=torch.float32, device=dev())))
    items = sk.group_items(keep)
    pb, _ = sk.sketch_group_bytes(items, sk.BF16)
    plan = torch.zeros(pb, dtype=torch.uint8, device=dev())
    sk.sketch_group_plan(items, sk.BF16, plan)
    h = plan.cpu().numpy().tobytes()
    magic, count, ntiles, nwaves, nfrag, xdt, nzb, tile_blocks, bits, pieces, rows, zs = struct.unpack_from("<12I", h, 0)
    assert (magic, count, tile_blocks, bits) == (0x50524753, 2, 64, 4)
    # few Z slices of 256 codes (16 + 4): slices of 128, the 4-bit fragment order's span
    assert (zs, nzb) == (128, 4096 // 128 + 1024 // 128)
    assert ntiles == 512 // 64 + (71 + 63) // 64
    # 10 tiles for the waves: every tile is split, into as many pieces as
    # the shorter linear has chunks (1024 codes: 4 chunks of 256)
    assert (pieces, rows) == (4, 4096 + 8 * 71)
    row0 = 0
    for i, (p, proj, tables, x, y) in enumerate(keep):
        f = struct.unpack_from("<7Q9I", h, 256 + 96 * i)
        nb, bg, _ = sk.sketch_layout(p)
        assert f[6] == tables.data_ptr() + ((nb * bg // 2 + 255) // 256) * 256, i
        assert f[15] == row0, i   # first row among the partial sums
        row0 += p.M


def test_group_q4_projection_of_another_seed_gives_nan_for_that_item_only():
    W0, W1 = synth.normal_bf16((256, 1024), 141), synth.normal_bf16((128, 1024), 142)
    t0, ref0 = _encode_q4(W0, "bf16", None, 8, 0.5, 1)
    t1, _ = _encode_q4(W1, "bf16", None, 8, 0.5, 1)
    wrong = sk.projection(sk.params(128, 1024, 8, 0.5, 2, sk.ABSMIN, sk.BF16, bits=4), dev())   # seed 2
    bad = sk.Tables(t1.params, t1.tables, wrong)
    x0, x1 = synth.normal_bf16((1, 1024), 143)[0], synth.normal_bf16((1, 1024), 144)[0]
    xs = [to_dev(x0[None], "bf16")[0], to_dev(x1[None], "bf16")[0]]
    ys = [torch.zeros(256, dtype=torch.float32, device=dev()), torch.zeros(128, dtype=torch.float32, device=dev())]
    sk.Group([t0, bad], xs, ys).run()
    torch.cuda.synchronize()
    assert bool(torch.isnan(ys[1]).all())
    yr = oracle.matmul_q4(ref0[0], ref0[1], x0[None], 256, 1024, 8, 0.5, 1, x_dtype=oracle.BF16)[0]
    assert_y_close(ys[0].cpu().numpy(), yr, what="good 4-bit item next to a bad one")


@pytest.mark.parametrize("bits", [16, 4])
def test_group_z_slice_size_leaves_y_unchanged(bits):
    """A linear's outputs do not depend on the Z slice its group takes: three
    linears alone (fewer than 256 slices of 256 buckets: small slices) and
    the same three inside a group of 64 (256 slices: slices of 256) give the
    same bits.  Both groups split their tiles into the same number of pieces,
    so nothing else differs; random finite tables."""
    import struct
    g = torch.Generator(device=dev())
    g.manual_seed(77 + bits)
    N = 4096 if bits == 16 else 1024   # 4 slices of 256 buckets per linear
    keep = []
    for i in range(64):
        p = sk.params(64, N, 8, 0.5, 1 + i % 3, sk.ABSMIN, sk.BF16, bits=bits)
        nb, bg, tb = sk.sketch_layout(p)
        if bits == 16:
            t = torch.randint(0, 0x3C00, (nb, bg), generator=g, device=dev(), dtype=torch.int32).to(torch.int16)
        else:   # bytes below 0x3C: finite binary16 block scales
            t = torch.randint(0, 0x3C, (tb,), generator=g, device=dev(), dtype=torch.int32).to(torch.uint8)
        x = torch.randn(N, generator=g, device=dev()).to(torch.bfloat16)
        keep.append((sk.Tables(p, t, sk.projection(p, dev())), x))

    def run(entries):
        ys = [torch.full((64,), float("nan"), dtype=torch.float32, device=dev()) for _ in entries]
        grp = sk.Group([t for t, _ in entries], [x for _, x in entries], ys)
        grp.run()
        torch.cuda.synchronize()
        zslice = struct.unpack_from("<12I", grp.plan[:48].cpu().numpy().tobytes(), 0)[11]
        return ys, zslice

    few, z_few = run(keep[:3])
    many, z_many = run(keep)
    assert (z_few, z_many) == ((64 if bits == 16 else 128), 256)
    for i in range(3):
        assert torch.isfinite(few[i]).all(), i
        assert torch.equal(few[i], many[i]), i


@pytest.mark.parametrize("bits", [16, 4])
def test_group_tall_linear_sampled(bits):
    """One 2,097,152 x 4096 linear at 0.5 bpw, R = 8 (512 MiB of tables: the
    tall-linear workload the bench times, in the same launch), random tables
    (finite binary16 buckets, or any 4-bit codes with finite block scales)
    and one bfloat16 token: 4096 sampled outputs, the first and last rows
    among them, against the oracle's one-output-at-a-time products."""
    M, N, R = 2097152, 4096, 8
    p = sk.params(M, N, R, 0.5, 1, sk.ABSMIN, sk.BF16, bits=bits)
    nb, bg, tb = sk.sketch_layout(p)
    g = torch.Generator(device=dev())
    g.manual_seed(77 + bits)
    if bits == 16:
        tt = torch.randint(0, 0x3C00, (nb, bg), generator=g, device=dev(), dtype=torch.int16)
    else:   # bytes below 0x3C: every block scale finite
        tt = torch.randint(0, 0x3C, (tb,), generator=g, device=dev(), dtype=torch.uint8)
    x = synth.normal_bf16((1, N), 78)[0]
    y = torch.full((M,), float("nan"), dtype=torch.float32, device=dev())
    sk.Group([sk.Tables(p, tt, sk.projection(p, dev()))], [to_dev(x[None], "bf16")[0]], [y]).run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(79)
    ii = np.concatenate([np.arange(48), rng.integers(0, M, 4000), np.arange(M - 48, M)]).astype(np.int64)
    ti = np.zeros_like(ii)
    if bits == 16:
        ys = oracle.matmul_sampled(tt.cpu().numpy().view(np.uint16), x[None], M, N, R, 0.5, ti, ii, 1,
                                   x_dtype=oracle.BF16)
    else:
        raw = tt.cpu().numpy()
        off = ((nb * bg // 2 + 255) // 256) * 256
        ys = oracle.matmul_sampled_q4(raw[:nb * bg // 2].reshape(nb, bg // 2), raw[off:off + 2 * nb].view(np.uint16),
                                      x[None], M, N, R, 0.5, ti, ii, 1, x_dtype=oracle.BF16)
    rms = np.sqrt(np.mean(ys ** 2))
    assert_y_close(y.cpu().numpy()[ii][None], ys[None], row_rms=np.array([[rms]]),
                   what="tall linear, %d-bit buckets" % bits)


@pytest.mark.parametrize("xk,N", [("bf16", 61440), ("f32", 30720)])
def test_group_x_at_the_lds_limit(xk, N):
    """x of 120 KiB, the most group_z_kernel holds in LDS (N = 61440 for
    16-bit x, 30720 for float32), next to a small item: both against the
    oracle."""
    entries = []
    for i, (M, n) in enumerate(((64, N), (256, 1024))):
        W = synth.normal_bf16((M, n), 1300 + i)
        t, S = _encode(W, "bf16", None, 8, 0.5, 11 + i)
        x = synth.normal_f32((1, n), 1.0, 1310 + i)[0] if xk == "f32" else synth.normal_bf16((1, n), 1310 + i)[0]
        entries.append((t, S, x, 11 + i))
    _check_group(entries, xk, "x at the LDS limit (%s, N=%d)" % (xk, N))
