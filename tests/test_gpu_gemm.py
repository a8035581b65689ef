"""GPU block GEMM (q4nx_gemm_block, M <= 64) vs the float64 oracle.

Bar: |Y - Y_ref| <= 2e-3 * sum_k |w x| per element.  The kernel rounds each
dequantised weight to bf16 (at most 2^-8 of its size); with random signs the
error of a K-term sum stays far inside the bar, as these tests measure.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_bf16, dev_u8, gemv, have_gpu, host, q, shift_xcd_start, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _gen(kind, N, K, tag):
    g = synth.rng("gpu-gemm", tag, kind, N, K)
    return synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)


_WS = {}


def _ws(w):
    """One zero-initialised workspace per size, reused by every call (as the API allows)."""
    n = q().gemm_block_ws(w)
    if n == 0:
        return None
    if n not in _WS:
        _WS[n] = torch.zeros(n, dtype=torch.uint8, device="cuda")
    return _WS[n]


def _gemm(ch_dev, N, K, kind, X):
    M = X.shape[0]
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    w = weight(ch_dev, N, K, kind)
    q().gemm_block(w, dev_bf16(X), Y, M, _ws(w))
    return host(Y)


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("N,K", [(32, 256), (96, 512), (160, 1280), (256, 2560), (288, 4096),
                                 (64, 14336)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 16, 31, 32, 33, 48, 63, 64])
def test_gemm_shapes(kind, N, K, M):
    ch = _gen(kind, N, K, "shapes")
    X = synth.gen_x(synth.rng("gpu-gemm", "X", N, K, M), M, K)
    Y = _gemm(dev_u8(ch), N, K, kind, X)
    yr, a = oracle.gemv_ref(oracle.weights_exact(ch, kind, N, K), X)
    r = oracle.tol_ratio(Y, yr, a)
    assert r <= 1.0, r


def test_gemm_rows_agree_with_gemv():
    N, K, M = 256, 2048, 64
    ch = _gen("q4_1", N, K, "vs-gemv")
    X = synth.gen_x(synth.rng("gpu-gemm", "vsX"), M, K)
    d = dev_u8(ch)
    Y = _gemm(d, N, K, "q4_1", X)
    yv = np.concatenate([gemv(d, N, K, "q4_1", X[m:m + 4]) for m in range(0, M, 4)])
    yr, a = oracle.gemv_ref(oracle.weights_exact(ch, "q4_1", N, K), X)
    assert oracle.tol_ratio(Y, yv, a) <= 1.0


def test_gemm_repeat_bit_identical_and_zero_rows():
    N, K, M = 128, 1024, 40
    ch = dev_u8(_gen("q4_k", N, K, "det"))
    X = synth.gen_x(synth.rng("gpu-gemm", "detX"), M, K)
    X[7] = 0
    Ys = [_gemm(ch, N, K, "q4_k", X) for _ in range(4)]
    for Y in Ys[1:]:
        np.testing.assert_array_equal(Y.view(np.uint32), Ys[0].view(np.uint32))
    assert np.all(Ys[0][7] == 0)


def test_dense_8b_layer_full_size_m64():
    """One 8B-dense layer's seven projections at M = 64, sampled tile rows checked."""
    X_all = {}
    for i, spec in enumerate(synth.dense_8b_block_specs(1)):
        ch = spec.generate()
        if spec.K not in X_all:
            X_all[spec.K] = synth.gen_x(synth.rng("dense_8b_block", "X", spec.K), 64, spec.K)
        X = X_all[spec.K]
        Y = _gemm(dev_u8(ch), spec.N, spec.K, "q4_1", X)
        g = np.random.default_rng(i)
        tr = np.unique(np.concatenate([[0, spec.N // 32 - 1], g.integers(0, spec.N // 32, 3)]))
        W = oracle.weights_exact(ch[tr], "q4_1", 32 * len(tr), spec.K)
        yr, a = oracle.gemv_ref(W, X)
        ysub = np.concatenate([Y[:, 32 * t:32 * t + 32] for t in tr], axis=1)
        assert oracle.tol_ratio(ysub, yr, a) <= 1.0, spec.name


def test_split_k_workspace_is_left_zeroed_and_reusable():
    """A weight whose K is split over workgroups: the counters return to zero after every call."""
    N, K = 1024, 8192
    w_ch = _gen("q4_1", N, K, "ws")
    d = dev_u8(w_ch)
    w = weight(d, N, K, "q4_1")
    n = q().gemm_block_ws(w)
    assert n > 0
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    yr_all = oracle.gemv_ref(oracle.weights_exact(w_ch, "q4_1", N, K),
                             synth.gen_x(synth.rng("gpu-gemm", "wsX"), 64, K))
    X = synth.gen_x(synth.rng("gpu-gemm", "wsX"), 64, K)
    for M in (64, 17, 64):
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        q().gemm_block(w, dev_bf16(X[:M]), Y, M, ws)
        assert oracle.tol_ratio(host(Y), yr_all[0][:M], yr_all[1][:M]) <= 1.0
    # the 256 arrival counters are back at zero
    assert torch.count_nonzero(ws[:4 * 256]).item() == 0


def _ws_bytes(n):
    if n == 0:
        return None
    if n not in _WS:
        _WS[n] = torch.zeros(n, dtype=torch.uint8, device="cuda")
    return _WS[n]


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("M", [1, 17, 64])
def test_gemm_batched_each_job_matches_oracle(kind, M):
    """Weights sharing X in one launch: q/k/v-like rows, one with a ragged last workgroup."""
    K = 1280
    shapes = [256, 64, 96, 32]
    chs = [_gen(kind, N, K, f"batched{i}") for i, N in enumerate(shapes)]
    X = synth.gen_x(synth.rng("gpu-gemm", "batchedX", M), M, K)
    devs = [dev_u8(c) for c in chs]
    ws_ = [weight(d, N, K, kind) for d, N in zip(devs, shapes)]
    Ys = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for N in shapes]
    jobs = list(zip(ws_, Ys))
    q().gemm_batched(jobs, dev_bf16(X), M, _ws_bytes(q().gemm_batched_ws(jobs)))
    for c, N, Y in zip(chs, shapes, Ys):
        yr, a = oracle.gemv_ref(oracle.weights_exact(c, kind, N, K), X)
        assert oracle.tol_ratio(host(Y), yr, a) <= 1.0, N


def test_gemm_batched_dense_8b_qkv_and_gate_up_full_size():
    """The 8B-dense q/k/v and gate/up launches at M = 64, sampled tile rows of every job."""
    specs = {s.name: s for s in synth.dense_8b_block_specs(1)}
    X = synth.gen_x(synth.rng("dense_8b_block", "X", 4096), 64, 4096)
    Xd = dev_bf16(X)
    for group in (("L0.q", "L0.k", "L0.v"), ("L0.gate", "L0.up")):
        chs = [specs[n].generate() for n in group]
        ws_ = [weight(dev_u8(c), specs[n].N, specs[n].K, "q4_1") for c, n in zip(chs, group)]
        Ys = [torch.full((64, specs[n].N), float("nan"), dtype=torch.float32, device="cuda") for n in group]
        jobs = list(zip(ws_, Ys))
        q().gemm_batched(jobs, Xd, 64, _ws_bytes(q().gemm_batched_ws(jobs)))
        for i, (c, n, Y) in enumerate(zip(chs, group, Ys)):
            TR = specs[n].N // 32
            g = np.random.default_rng(100 + i)
            tr = np.unique(np.concatenate([[0, TR - 1], g.integers(0, TR, 3)]))
            yr, a = oracle.gemv_ref(oracle.weights_exact(c[tr], "q4_1", 32 * len(tr), 4096), X)
            Yh = host(Y)
            ysub = np.concatenate([Yh[:, 32 * t:32 * t + 32] for t in tr], axis=1)
            assert oracle.tol_ratio(ysub, yr, a) <= 1.0, n


def test_one_workspace_serves_gemms_of_different_shapes():
    """Split-K GEMMs of different workgroup-row counts (4, 12, 32) through one
    workspace, with new X each call and the starting XCD moved between calls."""
    K = 4096
    shapes = [8192, 1024, 3072, 8192, 1024]
    chs = {N: _gen("q4_1", N, K, f"seqws{N}") for N in set(shapes)}
    Ws = {N: oracle.weights_exact(chs[N], "q4_1", N, K) for N in chs}
    devs = {N: dev_u8(c) for N, c in chs.items()}
    need = max(q().gemm_block_ws(weight(devs[N], N, K, "q4_1")) for N in chs)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, N in enumerate(shapes):
        w = weight(devs[N], N, K, "q4_1")
        assert q().gemm_block_ws(w) > 0
        M = 64 if i % 2 == 0 else 23
        X = synth.gen_x(synth.rng("gpu-gemm", "seqwsX", i), M, K)
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        shift_xcd_start(i + 1)
        q().gemm_block(w, dev_bf16(X), Y, M, ws)
        yr, a = oracle.gemv_ref(Ws[N], X)
        assert oracle.tol_ratio(host(Y), yr, a) <= 1.0, (i, N)
        assert torch.count_nonzero(ws[:4 * 256]).item() == 0


def test_split_k_graph_replays_with_new_inputs():
    """A captured split-K GEMM replayed on new X, the starting XCD moved between
    replays: every replay bit-identical to the eager call on the same X."""
    N, K = 1024, 8192
    ch = _gen("q4_1", N, K, "graphk")
    W = oracle.weights_exact(ch, "q4_1", N, K)
    w = weight(dev_u8(ch), N, K, "q4_1")
    ws = torch.zeros(q().gemm_block_ws(w), dtype=torch.uint8, device="cuda")
    Xs = [synth.gen_x(synth.rng("gpu-gemm", "graphkX", i), 64, K) for i in range(3)]
    Xd = dev_bf16(Xs[0])
    Y = torch.full((64, N), float("nan"), dtype=torch.float32, device="cuda")
    eager = []
    for i, X in enumerate(Xs):
        Xd.copy_(dev_bf16(X))
        shift_xcd_start(i)
        q().gemm_block(w, Xd, Y, 64, ws)
        eager.append(host(Y).copy())
        yr, a = oracle.gemv_ref(W, X)
        assert oracle.tol_ratio(eager[-1], yr, a) <= 1.0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        q().gemm_block(w, Xd, Y, 64, ws)
    torch.cuda.synchronize()
    for rep, i in enumerate((1, 2, 0, 2)):
        Xd.copy_(dev_bf16(Xs[i]))
        Y.fill_(float("nan"))
        shift_xcd_start(rep + 3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(Y).view(np.uint32), eager[i].view(np.uint32))
    assert torch.count_nonzero(ws[:4 * 256]).item() == 0


@pytest.mark.parametrize("M", [5, 64])
def test_gemm_batched_at_the_job_limit(M):
    """Eight jobs in one call (the API's limit) with rows from 32 to 512: each against the oracle."""
    K = 768
    shapes = [32, 512, 64, 96, 256, 32, 160, 128]
    chs = [_gen("q4_k", N, K, f"lim{i}") for i, N in enumerate(shapes)]
    X = synth.gen_x(synth.rng("gpu-gemm", "limX", M), M, K)
    ws_ = [weight(dev_u8(c), N, K, "q4_k") for c, N in zip(chs, shapes)]
    Ys = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for N in shapes]
    jobs = list(zip(ws_, Ys))
    q().gemm_batched(jobs, dev_bf16(X), M, _ws_bytes(q().gemm_batched_ws(jobs)))
    for c, N, Y in zip(chs, shapes, Ys):
        yr, a = oracle.gemv_ref(oracle.weights_exact(c, "q4_k", N, K), X)
        assert oracle.tol_ratio(host(Y), yr, a) <= 1.0, N
