"""GPU dequant-GEMV (q4nx_gemv, q4nx_gemv_batched) vs the float64 oracle.

Bar: every output finite and |y - y_ref| <= 2e-3 * sum_k |w x| per element.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_bf16, dev_u8, gemv, have_gpu, host, q, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

KINDS = [("q4_1", None), ("q4_k", None), ("q8", "A"), ("q8", "B")]


def _gen(kind, layout, N, K, tag):
    g = synth.rng("gpu-gemv", tag, kind, layout or "-", N, K)
    if kind == "q4_1":
        return synth.gen_q4_1(g, N, K, zero="normal")
    if kind == "q4_k":
        return synth.gen_q4_k(g, N, K)
    return synth.gen_q8(g, N, K, layout)


def _check(y, ch, kind, N, K, x, layout, rows=None):
    W = oracle.weights_exact(ch, kind, N, K, layout)
    yr, a = oracle.gemv_ref(W, x)
    if rows is not None:
        yr, a, y = yr[:, rows], a[:, rows], y[:, rows]
    r = oracle.tol_ratio(y, yr, a)
    assert r <= 1.0, f"max error / (2e-3 * sum|wx|) = {r}"
    return r


def test_single_q4_1_gemv_1024():
    spec = synth.single_gemv_spec()
    ch = spec.generate()
    x = synth.gen_x(synth.rng("q4_1_gemv_1024", 0, "x"), 1, spec.K)
    y = gemv(dev_u8(ch), spec.N, spec.K, "q4_1", x)
    print("tolerance ratio", _check(y, ch, "q4_1", spec.N, spec.K, x, None))


@pytest.mark.parametrize("kind,layout", KINDS)
@pytest.mark.parametrize("N,K", [(32, 256), (96, 768), (160, 1280), (64, 2560), (288, 3328)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_gemv_shapes(kind, layout, N, K, M):
    ch = _gen(kind, layout, N, K, "shapes")
    x = synth.gen_x(synth.rng("gpu-gemv", "x", N, K, M), M, K)
    y = gemv(dev_u8(ch), N, K, kind, x, layout)
    _check(y, ch, kind, N, K, x, layout)


@pytest.mark.parametrize("M", [5, 6, 7])
def test_gemv_other_m(M):
    N, K = 96, 1280
    ch = _gen("q4_1", None, N, K, "otherm")
    x = synth.gen_x(synth.rng("gpu-gemv", "xm", M), M, K)
    _check(gemv(dev_u8(ch), N, K, "q4_1", x), ch, "q4_1", N, K, x, None)


@pytest.mark.parametrize("M", [1, 2, 4])
def test_q8_layouts_of_one_weight(M):
    """The same codes stored in layout A and in layout B: each result is within
    the bar of the oracle and repeats bit for bit.  The two layouts put
    different columns in a lane, so their sums run in different orders and
    may differ in the last bits."""
    N, K = 2048, 2560
    A = synth.gen_q8(synth.rng("gpu-gemv", "q8ab"), N, K, "A")
    B = synth.q8_relayout(A, "A", "B")
    x = synth.gen_x(synth.rng("gpu-gemv", "q8ab-x", M), M, K)
    dA, dB = dev_u8(A), dev_u8(B)
    ya = gemv(dA, N, K, "q8", x, "A")
    yb = gemv(dB, N, K, "q8", x, "B")
    _check(ya, A, "q8", N, K, x, "A")
    _check(yb, A, "q8", N, K, x, "A")
    np.testing.assert_array_equal(gemv(dA, N, K, "q8", x, "A").view(np.uint32), ya.view(np.uint32))
    np.testing.assert_array_equal(gemv(dB, N, K, "q8", x, "B").view(np.uint32), yb.view(np.uint32))


def _one_hot_check(ch, kind, layout, N, K, cols):
    W32 = oracle.weights_f32(ch, kind, N, K, layout)
    x = np.zeros((len(cols), K), np.uint16)
    for i, k in enumerate(cols):
        x[i, k] = 0x3F80
    for i0 in range(0, len(cols), 4):
        xs = x[i0:i0 + 4]
        y = gemv(dev_u8(ch), N, K, kind, xs, layout)
        for j in range(xs.shape[0]):
            np.testing.assert_array_equal(y[j].view(np.uint32), W32[:, cols[i0 + j]].view(np.uint32))


@pytest.mark.parametrize("kind,layout", KINDS)
def test_one_hot_activation_gives_the_column(kind, layout):
    """x = e_k returns column k of the decoded weights bit for bit: the signed
    codes and their center make s (c - c0) + (z + c0 s) one rounding of s c + z.
    The columns go in calls of up to 4 rows (M = 4 and 3: the matrix-core
    products; a single row: the dot chain), so the pin holds for both."""
    N, K = 64, 512
    _one_hot_check(_gen(kind, layout, N, K, "onehot"), kind, layout, N, K, [0, 5, 31, 32, 255, 256, 511])


def test_one_hot_q4_k_signed_metadata():
    """The same pin on Q4_K with S of either sign and M = -dmin <= 0 (as a GGUF
    Q4_K maps), sc/mn over 0..255, at moderate |M mn / (S sc)| (below 2^8, so
    z + c0 s is exact in fp32)."""
    N, K = 64, 512
    g = synth.rng("gpu-gemv", "onehot-q4k-signed")
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    sc = g.integers(16, 256, (N, K // 32), dtype=np.uint8)
    mn = g.integers(0, 256, (N, K // 32), dtype=np.uint8)
    S = synth.bf16_bits((g.standard_normal((N, K // 256)) * 1e-3).astype(np.float32))
    Mv = synth.bf16_bits((-np.abs(g.standard_normal((N, K // 256))) * 1e-3).astype(np.float32))
    ch = synth.pack_q4_k(codes, sc, mn, S, Mv)
    _one_hot_check(ch, "q4_k", None, N, K, [0, 7, 33, 300, 511])


def test_q4_0_style_zero_rows_are_exactly_zero():
    """Codes all 8 with zero = -8*scale decode to w = 0: the GEMV must return exactly 0."""
    N, K = 64, 1024
    g = synth.rng("gpu-gemv", "zero-rows")
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    codes[5, :] = 8
    codes[40, :] = 8
    s = synth.bf16_bits(np.abs(g.standard_normal((N, K // 32)).astype(np.float32)) * 0.02)
    z = synth.bf16_bits(-8 * synth.bf16_to_f32(s))
    ch = synth.pack_q4_1(codes, s, z)
    x = synth.gen_x(g, 4, K)
    y = gemv(dev_u8(ch), N, K, "q4_1", x)
    assert np.all(y[:, 5] == 0) and np.all(y[:, 40] == 0)
    _check(y, ch, "q4_1", N, K, x, None)


def test_zero_activations_give_zero():
    N, K = 96, 768
    for kind, layout in KINDS:
        ch = _gen(kind, layout, N, K, "zx")
        y = gemv(dev_u8(ch), N, K, kind, np.zeros((2, K), np.uint16), layout)
        assert np.all(y == 0), kind


def test_nan_scale_poisons_exactly_its_row():
    N, K = 64, 512
    ch = _gen("q4_1", None, N, K, "nan")
    # (scale, zero) of tile row 0, row r=3, group g=2 -> chunk (0, 0), byte 4096 + 4*(8*3+2)
    ch[0, 0, 4096 + 4 * 26:4096 + 4 * 26 + 2] = np.frombuffer(np.uint16(0x7FC0).tobytes(), np.uint8)
    x = synth.gen_x(synth.rng("gpu-gemv", "nanx"), 1, K)
    y = gemv(dev_u8(ch), N, K, "q4_1", x)
    bad = ~np.isfinite(y[0])
    assert bad[3] and bad.sum() == 1
    keep = [r for r in range(N) if r != 3]
    _check(y, ch, "q4_1", N, K, x, None, rows=keep)


def test_repeat_runs_are_bit_identical():
    N, K = 1024, 2560
    ch = dev_u8(_gen("q4_1", None, N, K, "det"))
    x = synth.gen_x(synth.rng("gpu-gemv", "detx"), 4, K)
    ys = [gemv(ch, N, K, "q4_1", x) for _ in range(5)]
    for y in ys[1:]:
        np.testing.assert_array_equal(y.view(np.uint32), ys[0].view(np.uint32))


def test_batched_matches_single_calls():
    shapes = [(4096, 2560), (1024, 2560), (1024, 2560), (320, 768)]
    chs = [_gen("q4_1", None, N, K, f"b{i}") for i, (N, K) in enumerate(shapes)]
    chs.append(_gen("q8", "B", 256, 512, "b8"))
    shapes.append((256, 512))
    kinds = ["q4_1"] * 4 + ["q8"]
    lays = [None] * 4 + ["B"]
    M = 2
    xs = [synth.gen_x(synth.rng("gpu-gemv", "bx", i), M, K) for i, (N, K) in enumerate(shapes)]
    dch = [dev_u8(c) for c in chs]
    dx = [dev_bf16(x) for x in xs]
    dy = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for N, K in shapes]
    jobs = [(weight(dch[i], N, K, kinds[i], lays[i]), dx[i], dy[i]) for i, (N, K) in enumerate(shapes)]
    q().gemv_batched(jobs, M)
    for i, (N, K) in enumerate(shapes):
        _check(host(dy[i]), chs[i], kinds[i], N, K, xs[i], lays[i])


def _sampled_rows(N, seed, n=96):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, N - 1], g.integers(0, N, n)]))


def test_qwen3_4b_layer_and_lm_head_full_size():
    """One layer's seven projections and the lm_head at full size, sampled rows checked."""
    specs = synth.qwen3_4b_decode_specs(1, True)
    for i, spec in enumerate(specs):
        ch = spec.generate()
        x = synth.gen_x(synth.rng("qwen3_4b_decode", "x", spec.name), 1, spec.K)
        y = gemv(dev_u8(ch), spec.N, spec.K, "q4_1", x)
        rows = _sampled_rows(spec.N, i)
        tr = np.unique(rows // 32)
        sub = ch[tr]
        W = oracle.weights_exact(sub, "q4_1", 32 * len(tr), spec.K)
        yr, a = oracle.gemv_ref(W, x)
        ysub = np.concatenate([y[:, 32 * t:32 * t + 32] for t in tr], axis=1)
        assert oracle.tol_ratio(ysub, yr, a) <= 1.0, spec.name


@pytest.mark.parametrize("layout", ["A", "B"])
def test_mixed_q4k_layer_and_q8_lm_head_full_size(layout):
    specs = synth.mixed_decode_specs(1, "A")
    for i, spec in enumerate(specs):
        ch = spec.generate()
        lay = None
        if spec.kind == "q8":
            lay = layout
            if layout == "B":
                ch = synth.q8_relayout(ch, "A", "B")
        x = synth.gen_x(synth.rng("mixed_decode", "x", spec.name), 1, spec.K)
        y = gemv(dev_u8(ch), spec.N, spec.K, spec.kind, x, lay)
        tr = np.unique(_sampled_rows(spec.N, 100 + i) // 32)
        W = oracle.weights_exact(ch[tr], spec.kind, 32 * len(tr), spec.K, lay)
        yr, a = oracle.gemv_ref(W, x)
        ysub = np.concatenate([y[:, 32 * t:32 * t + 32] for t in tr], axis=1)
        assert oracle.tol_ratio(ysub, yr, a) <= 1.0, spec.name


@pytest.mark.parametrize("kind,layout", KINDS)
@pytest.mark.parametrize("M", [2, 3, 4, 5, 8])
def test_verify_window_slot_invariance(kind, layout, M):
    """A verify window of M tokens (Strata article, section 6.2, batch slots):
    a token's result does not depend on the slot it occupies -- permuting the
    rows of x permutes the rows of y bit for bit."""
    N, K = 2560, 2560
    ch = _gen(kind, layout, N, K, "slots")
    d = dev_u8(ch)
    x = synth.gen_x(synth.rng("gpu-gemv", "slots", kind, M), M, K)
    perm = np.roll(np.arange(M), 1)
    y = gemv(d, N, K, kind, x, layout)
    yp = gemv(d, N, K, kind, x[perm], layout)
    np.testing.assert_array_equal(yp.view(np.uint32), y[perm].view(np.uint32))


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("N,K,M", [(64, 14336, 2), (64, 14336, 4), (96, 7424, 3), (32, 40960, 1), (160, 3328, 8),
                                   (416, 14336, 3), (1056, 4608, 4), (96, 14336, 5), (160, 14336, 8)])
def test_long_activation_rows(kind, N, K, M):
    """Activation rows too long for one register load per thread (several
    rows, long K, odd tile-column counts; 4-, 8- and 16-wave workgroups, the
    8-wave ones at M = 3 and 4 over at least 17 tile columns; at M = 5 and 8
    over 56 tile columns, two overlapping 4-row passes): against the oracle,
    and a permutation of the rows of x permutes the rows of y bit for bit."""
    ch = _gen(kind, None, N, K, "longrows")
    d = dev_u8(ch)
    x = synth.gen_x(synth.rng("gpu-gemv", "longrows", kind, N, K, M), M, K)
    y = gemv(d, N, K, kind, x)
    _check(y, ch, kind, N, K, x, None)
    if M > 1:
        perm = np.roll(np.arange(M), 1)
        yp = gemv(d, N, K, kind, x[perm])
        np.testing.assert_array_equal(yp.view(np.uint32), y[perm].view(np.uint32))


@pytest.mark.parametrize("M", [1, 2])
def test_batched_at_the_job_limit(M):
    """64 jobs in one call (the API's limit), all three kinds and both Q8 layouts
    mixed, of varied shapes: each job's result against the oracle."""
    g = np.random.default_rng(64 + M)
    kinds = [("q4_1", None), ("q4_k", None), ("q8", "A"), ("q8", "B")]
    jobs, refs = [], []
    for i in range(64):
        kind, lay = kinds[i % 4]
        N, K = 32 * int(g.integers(1, 5)), 256 * int(g.integers(1, 4))
        ch = _gen(kind, lay, N, K, f"lim{M}-{i}")
        x = synth.gen_x(synth.rng("gpu-gemv", "limx", M, i), M, K)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        jobs.append((weight(dev_u8(ch), N, K, kind, lay), dev_bf16(x), y))
        refs.append((ch, kind, lay, N, K, x, y))
    q().gemv_batched(jobs, M)
    for ch, kind, lay, N, K, x, y in refs:
        _check(host(y), ch, kind, N, K, x, lay)


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("M", [1, 2, 4])
def test_launch_of_several_rounds(kind, M):
    """A launch of more workgroups than the CUs hold at once (the 28672 x 4096
    gate|up of an 8B layer; at M >= 3, whose matrix-core launches give each
    wave a whole K range and so take fewer workgroups, three of them side by
    side): sampled tile rows against the oracle, and its first 512 tile rows
    bit for bit against the same rows as a launch that fits in one round (the
    same K split and chunk order)."""
    N, K = (28672 if M <= 2 else 86016), 4096
    g = synth.rng("gpu-gemv", "upw", kind)
    ch = synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)
    x = synth.gen_x(synth.rng("gpu-gemv", "upw-x", kind, M), M, K)
    y = gemv(dev_u8(ch), N, K, kind, x)
    tr = np.unique(_sampled_rows(N, 31 + M) // 32)
    W = oracle.weights_exact(ch[tr], kind, 32 * len(tr), K)
    yr, a = oracle.gemv_ref(W, x)
    ysub = np.concatenate([y[:, 32 * t:32 * t + 32] for t in tr], axis=1)
    assert oracle.tol_ratio(ysub, yr, a) <= 1.0
    part = gemv(dev_u8(np.ascontiguousarray(ch[:512])), 16384, K, kind, x)
    np.testing.assert_array_equal(part.view(np.uint32), y[:, :16384].view(np.uint32))


@pytest.mark.parametrize("N,M", [(151936, 1), (151936, 2), (40960, 1), (40960, 3)])
def test_q4k_whole_tile_launches_sampled(N, M):
    """Q4_K launches of more than 1024 tile rows (whole-tile units, metadata
    handed out through the per-wave LDS slot): sampled rows against the oracle."""
    K = 2560
    ch = synth.gen_q4_k(synth.rng("gpu-gemv", "q4k-whole", N), N, K)
    x = synth.gen_x(synth.rng("gpu-gemv", "q4k-whole-x", N, M), M, K)
    y = gemv(dev_u8(ch), N, K, "q4_k", x)
    tr = np.unique(_sampled_rows(N, 7 + M) // 32)
    W = oracle.weights_exact(ch[tr], "q4_k", 32 * len(tr), K)
    yr, a = oracle.gemv_ref(W, x)
    ysub = np.concatenate([y[:, 32 * t:32 * t + 32] for t in tr], axis=1)
    assert oracle.tol_ratio(ysub, yr, a) <= 1.0
