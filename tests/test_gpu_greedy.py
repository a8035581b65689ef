"""Q8 embedding row gather (q4nx_q8_rows) and greedy argmax (q4nx_argmax).

Row gather: every value is d * code, exact in fp32, so the device rows must
equal the oracle's exact decode bit for bit, in both Q8 code layouts.
Argmax: the decision is taken on fp32 values on both sides -- the oracle runs
numpy's first-maximum argmax (NaNs skipped) on the device's own logits; the
chosen logit is also checked against the float64 reference within the GEMV
tolerance.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_bf16, dev_f32, dev_i32, dev_u8, gemv, have_gpu, host, q, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.mark.parametrize("layout", ["A", "B"])
def test_q8_rows_exact(layout):
    N, K = 96, 768
    ch = synth.gen_q8(synth.rng("gpu-rows", layout), N, K, layout)
    W = oracle.weights_exact(ch, "q8", N, K, layout)
    ids = np.array([0, 5, 31, 32, 95, 40, 40, -1, 96], dtype=np.int32)
    out = torch.full((len(ids), K), float("nan"), dtype=torch.float32, device="cuda")
    q().q8_rows(weight(dev_u8(ch), N, K, "q8", layout), dev_i32(ids), len(ids), out)
    got = host(out)
    for t, r in enumerate(ids):
        want = W[r] if 0 <= r < N else np.zeros(K)
        np.testing.assert_array_equal(got[t].astype(np.float64), want)


def _argmax_ref(y):
    y = np.asarray(y, dtype=np.float32)
    if np.all(np.isnan(y)):
        return -1
    return int(np.nanargmax(y))


def _argmax(y, n, M, idx, val=None, ldy=None, split=False):
    """q4nx_argmax with (split) or without a workspace."""
    ws = None
    if split:
        ws = torch.full((q().argmax_ws(n, M),), 0xAB, dtype=torch.uint8, device="cuda")  # stale contents
    q().argmax(y, n, M, idx, val, ldy=ldy, ws=ws)


@pytest.mark.parametrize("split", [False, True])
def test_argmax_ties_nans_and_rows(split):
    g = np.random.default_rng(7)
    M, n, ldy = 5, 3000, 3072
    y = g.standard_normal((M, ldy)).astype(np.float32)
    y[0, [17, 2900]] = 9.0             # tie: lowest index wins
    y[1, :] = np.nan
    y[1, 1234] = -3.0                  # only one number among NaNs
    y[2, :] = np.nan                   # all NaN -> -1
    y[3, 100] = np.inf
    y[4, n:] = 100.0                   # past n: ignored
    idx = torch.zeros(M, dtype=torch.int32, device="cuda")
    val = torch.zeros(M, dtype=torch.float32, device="cuda")
    _argmax(dev_f32(y), n, M, idx, val, ldy=ldy, split=split)
    got = host(idx)
    for m in range(M):
        assert got[m] == _argmax_ref(y[m, :n]), m
    assert got[0] == 17 and got[1] == 1234 and got[2] == -1 and got[3] == 100


@pytest.mark.parametrize("layout", ["A", "B"])
def test_greedy_head_q8(layout):
    """Q8 lm_head GEMV, then argmax: the pick is the first maximum of the GPU
    logits, and within tolerance of the float64 maximum."""
    N, K = 4096, 2560
    ch = synth.gen_q8(synth.rng("gpu-greedy", layout), N, K, layout)
    x = synth.gen_x(synth.rng("gpu-greedy-x", layout), 2, K)
    d = dev_u8(ch)
    w = weight(d, N, K, "q8", layout)
    y = torch.empty((2, N), dtype=torch.float32, device="cuda")
    q().gemv(w, dev_bf16(x), y, 2)
    idx = torch.zeros(2, dtype=torch.int32, device="cuda")
    idx2 = torch.zeros(2, dtype=torch.int32, device="cuda")
    q().argmax(y, N, 2, idx)
    _argmax(y, N, 2, idx2, split=True)
    yh, got = host(y), host(idx)
    np.testing.assert_array_equal(host(idx2), got)
    yr, a = oracle.gemv_ref(oracle.weights_exact(ch, "q8", N, K, layout), x)
    for m in range(2):
        assert got[m] == _argmax_ref(yh[m])
        assert yr[m, got[m]] >= yr[m].max() - 2 * 2e-3 * a[m, got[m]] - 2 * 2e-3 * a[m, np.argmax(yr[m])]


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("n,ldy", [(3001, 3003), (3001, 3004), (5, 5), (1, 1), (4096, 4096), (4099, 4100),
                                   (151936, 151936)])
def test_argmax_tail_and_unaligned_rows(n, ldy, split):
    """Rows whose length is not a multiple of 4, rows that start off a 16-byte
    boundary, and the full 151936-wide head: maxima in the last element and a
    tie between the first and last elements."""
    g = np.random.default_rng(n + ldy)
    M = 3
    y = g.standard_normal((M, ldy)).astype(np.float32)
    y[0, n - 1] = 50.0
    y[1, 0] = 60.0
    y[1, n - 1] = 60.0
    y[2, g.integers(0, n)] = 70.0
    idx = torch.zeros(M, dtype=torch.int32, device="cuda")
    val = torch.zeros(M, dtype=torch.float32, device="cuda")
    _argmax(dev_f32(y), n, M, idx, val, ldy=ldy, split=split)
    got, gv = host(idx), host(val)
    for m in range(M):
        assert got[m] == _argmax_ref(y[m, :n]), m
        assert gv[m] == y[m, got[m]]


@pytest.mark.parametrize("split", [False, True])
def test_argmax_signed_zeros_are_equal(split):
    """A row whose maximum is zero, held as -0.0 before +0.0 (and the reverse):
    the first of them wins, and val is the value stored there."""
    n = 9000
    y = -np.abs(np.random.default_rng(3).standard_normal((2, n))).astype(np.float32) - 1.0
    y[0, 4500], y[0, 8000] = -0.0, 0.0
    y[1, 100], y[1, 5000] = 0.0, -0.0
    idx = torch.zeros(2, dtype=torch.int32, device="cuda")
    val = torch.zeros(2, dtype=torch.float32, device="cuda")
    _argmax(dev_f32(y), n, 2, idx, val, split=split)
    got, gv = host(idx), host(val)
    assert got.tolist() == [4500, 100]
    assert np.signbit(gv[0]) and not np.signbit(gv[1])


# ----------------------------------------------------------------------------
# q4nx_gemv_topk: the head GEMV with its top-k pick in the same launch
# ----------------------------------------------------------------------------
def _head(kind, layout, N, K, tag):
    g = synth.rng("gpu-topk", tag, kind, layout or "-", N, K)
    if kind == "q4_1":
        return synth.gen_q4_1(g, N, K, zero="normal")
    if kind == "q4_k":
        return synth.gen_q4_k(g, N, K)
    return synth.gen_q8(g, N, K, layout)


def _topk(w, x, M, k, with_y=True, with_vals=True, ws=None):
    N = w.rows
    ids = torch.full((M, k), -7, dtype=torch.int32, device="cuda")
    vals = torch.full((M, k), float("nan"), dtype=torch.float32, device="cuda") if with_vals else None
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") if with_y else None
    if ws is None:
        ws = torch.zeros(q().gemv_topk_ws(w, M, k), dtype=torch.uint8, device="cuda")
    q().gemv_topk(w, dev_bf16(x), M, k, ids, ws, y=y, vals=vals)
    return host(ids), (host(vals) if with_vals else None), (host(y) if with_y else None), ws


@pytest.mark.parametrize("kind,layout", [("q8", "A"), ("q8", "B"), ("q4_1", None), ("q4_k", None)])
@pytest.mark.parametrize("k", [1, 10])
def test_gemv_topk_full_size_head(kind, layout, k):
    """151936 x 2560 head (the tied embedding / lm_head shape): the logits equal
    q4nx_gemv's bit for bit, the picks equal the oracle's on those logits, the
    values are the logits at the picks, and the workspace counters are back to
    zero after every call."""
    N, K, M = 151936, 2560, 1
    ch = _head(kind, layout, N, K, "full")
    w = weight(dev_u8(ch), N, K, kind, layout)
    x = synth.gen_x(synth.rng("gpu-topk", "x", kind, k), M, K)
    y_plain = gemv(dev_u8(ch), N, K, kind, x, layout)
    ws = None
    for rep in range(2):
        ids, vals, y, ws = _topk(w, x, M, k, ws=ws)
        np.testing.assert_array_equal(y.view(np.uint32), y_plain.view(np.uint32))
        np.testing.assert_array_equal(ids, oracle.head_topk(y, k))
        np.testing.assert_array_equal(vals.view(np.uint32), y[0, ids[0]].view(np.uint32)[None, :])
        assert torch.count_nonzero(ws[:256]).item() == 0
    # the picked logits against the float64 reference of those rows
    rows = ids[0]
    W = oracle.weights_exact(ch[rows // 32], kind, 32 * len(rows), K, layout)
    sel = (rows % 32) + 32 * np.arange(len(rows))
    yr, a = oracle.gemv_ref(W[sel], x)
    assert oracle.tol_ratio(vals, yr, a) <= 1.0


@pytest.mark.parametrize("M", [1, 2, 3])
def test_gemv_topk_without_logits_rows_and_m(M):
    """No logits written (y = NULL), M activation rows, k = 16, a 40960-row q4_1
    head split into 16-row units: the picks equal the oracle's on q4nx_gemv's logits."""
    N, K, k = 40960, 2560, 16
    ch = _head("q4_1", None, N, K, "rows")
    w = weight(dev_u8(ch), N, K, "q4_1")
    x = synth.gen_x(synth.rng("gpu-topk", "xm", M), M, K)
    y_plain = gemv(dev_u8(ch), N, K, "q4_1", x)
    ids, vals, _, _ = _topk(w, x, M, k, with_y=False)
    np.testing.assert_array_equal(ids, oracle.head_topk(y_plain, k))
    for m in range(M):
        np.testing.assert_array_equal(vals[m].view(np.uint32), y_plain[m, ids[m]].view(np.uint32))


def test_gemv_topk_ties_nans_and_small_heads():
    """Equal rows (identical chunks give identical logits: the lower row wins),
    rows poisoned by a NaN scale (never picked), a head of one tile row with
    k larger than its numbers (then -1), and a Q8 head."""
    N, K = 96, 512
    ch = _head("q4_1", None, N, K, "ties")
    ch[1] = ch[0]                       # tile row 1 repeats tile row 0: rows 32..63 tie with 0..31
    # NaN scale in tile row 2, row r = 5, group 0 of every chunk: row 69 is NaN
    for tc in range(K // 256):
        ch[2, tc, 4096 + 4 * (8 * 5):4096 + 4 * (8 * 5) + 2] = np.frombuffer(np.uint16(0x7FC0).tobytes(), np.uint8)
    w = weight(dev_u8(ch), N, K, "q4_1")
    x = synth.gen_x(synth.rng("gpu-topk", "xt"), 2, K)
    ids, vals, y, _ = _topk(w, x, 2, 16)
    assert np.isnan(y[:, 69]).all()
    np.testing.assert_array_equal(ids, oracle.head_topk(y, 16))
    assert 69 not in ids
    # one tile row, every row NaN but 3: k = 8 gives 3 picks, then -1
    ch1 = _head("q4_1", None, 32, 256, "one")
    for r in range(32):
        if r not in (4, 17, 30):
            ch1[0, 0, 4096 + 4 * (8 * r):4096 + 4 * (8 * r) + 2] = np.frombuffer(np.uint16(0x7FC0).tobytes(), np.uint8)
    w1 = weight(dev_u8(ch1), 32, 256, "q4_1")
    x1 = synth.gen_x(synth.rng("gpu-topk", "x1"), 1, 256)
    ids1, vals1, y1, _ = _topk(w1, x1, 1, 8)
    np.testing.assert_array_equal(ids1, oracle.head_topk(y1, 8))
    assert list(ids1[0, 3:]) == [-1] * 5 and np.isnan(vals1[0, 3:]).all()
    # a Q8 head of 2048 rows in layout B
    ch8 = _head("q8", "B", 2048, 1024, "q8small")
    w8 = weight(dev_u8(ch8), 2048, 1024, "q8", "B")
    x8 = synth.gen_x(synth.rng("gpu-topk", "x8"), 3, 1024)
    ids8, _, y8, _ = _topk(w8, x8, 3, 5)
    np.testing.assert_array_equal(ids8, oracle.head_topk(y8, 5))


def test_gemv_topk_graph_replays():
    """The one-launch head captured in a graph and replayed on new activations."""
    N, K, k = 151936, 2560, 4
    ch = _head("q8", "A", N, K, "graph")
    w = weight(dev_u8(ch), N, K, "q8", "A")
    xs = [synth.gen_x(synth.rng("gpu-topk", "gx", i), 1, K) for i in range(3)]
    xd = dev_bf16(xs[0])
    ids = torch.full((1, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(q().gemv_topk_ws(w, 1, k), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        q().gemv_topk(w, xd, 1, k, ids, ws)
    torch.cuda.synchronize()
    for rep, i in enumerate((1, 2, 0, 1)):
        xd.copy_(dev_bf16(xs[i]))
        ids.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.head_topk(gemv(dev_u8(ch), N, K, "q8", xs[i], "A"), k)
        np.testing.assert_array_equal(host(ids), want)
