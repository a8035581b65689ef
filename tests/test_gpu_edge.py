"""Edge cases of the dequant-GEMV and the block GEMM against the float64 oracle.

Weights that stress the factored sum (rows whose weights are almost all
exactly zero, zero crossings away from the middle code), metadata of both
signs and of the full u8 range (NPU engine page, "From a GGUF": Q4_K stores
M = -dmin), Q8's code -128 and subnormal scales, and activations outside the
range the fp16 records hold exactly (values spanning more than 2^32 within a
32-column group, bf16 subnormals, zeros).

Bars:
* GEMV: every output finite and |y - y_ref| <= 2e-3 * sum |w x|.
* block GEMM on dense random codes: the same bar (the bf16 rounding of each
  weight has random sign); on sparse rows, where a sum may hold a single
  term, the bound the bf16 rounding of each weight gives: 2^-8 * sum |w x|
  plus the fp32 sums.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_bf16, dev_u8, gemv, have_gpu, host, q, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

SMALL = (96, 768)
FULL = (4096, 2560)       # the q projection of the 4B decode step
FULL_K = (2560, 9728)     # its down projection (long K)


def _bf(a):
    return synth.bf16_bits(np.asarray(a, np.float32))


def _ref(ch, kind, N, K, x, layout=None):
    return oracle.gemv_ref(oracle.weights_exact(ch, kind, N, K, layout), x)


def _gemm(ch, N, K, kind, X):
    M = X.shape[0]
    w = weight(dev_u8(ch), N, K, kind)
    ws_n = q().gemm_block_ws(w)
    ws = torch.zeros(max(ws_n, 256), dtype=torch.uint8, device="cuda")
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    q().gemm_block(w, dev_bf16(X), Y, M, ws)
    return host(Y)


def _x_spread(g, M, K, small_cols):
    """x ~ N(0, 1) * 10, with |x| ~ 1e-3 at the given columns."""
    x = g.standard_normal((M, K)).astype(np.float32) * 10
    x[:, small_cols] = g.standard_normal((M, len(small_cols))).astype(np.float32) * 1e-3
    return _bf(x)


def _sparse_q4_1(g, N, K, center, rows_sparse):
    """q4_1 rows whose codes are all `center` (w = 0 exactly: zero = -center * scale)
    except three codes per sparse row at chosen columns; other rows random."""
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    # scales with 4 significant bits so that center * scale is exact in bf16
    s = np.ldexp(g.integers(8, 16, (N, K // 32)).astype(np.float32), g.integers(-12, -8, (N, K // 32)))
    z = -np.float32(center) * s
    cols = np.sort(g.choice(K, 3, replace=False))
    for r in rows_sparse:
        codes[r, :] = center
        codes[r, cols] = (center + g.integers(1, 15, 3)) % 16
    return synth.pack_q4_1(codes, _bf(s), _bf(z)), cols


@pytest.mark.parametrize("center", [8, 0, 3, 12, 15])
@pytest.mark.parametrize("N,K", [SMALL, FULL])
@pytest.mark.parametrize("M", [1, 4])
def test_gemv_sparse_rows(center, N, K, M):
    """Rows of exactly-zero weights but for three codes, at columns where |x| is
    small next to |x| ~ 10 elsewhere: the error must still scale with the few
    nonzero terms."""
    g = synth.rng("gpu-edge", "sparse", center, N, K, M)
    rows = list(range(0, N, 7))
    ch, cols = _sparse_q4_1(g, N, K, center, rows)
    x = _x_spread(g, M, K, cols)
    y = gemv(dev_u8(ch), N, K, "q4_1", x)
    yr, a = _ref(ch, "q4_1", N, K, x)
    r = oracle.tol_ratio(y, yr, a)
    assert r <= 1.0, r


@pytest.mark.parametrize("center", [8, 0])
@pytest.mark.parametrize("M", [1, 3, 4])
def test_gemv_sparse_rows_long_k(center, M):
    """The same rows at the 4B step's down projection (38 tile columns: 16-wave
    workgroups at M = 1, 8-wave ones at M = 3 and 4)."""
    N, K = FULL_K
    g = synth.rng("gpu-edge", "sparse-long", center, M)
    rows = list(range(0, N, 7))
    ch, cols = _sparse_q4_1(g, N, K, center, rows)
    x = _x_spread(g, M, K, cols)
    y = gemv(dev_u8(ch), N, K, "q4_1", x)
    yr, a = _ref(ch, "q4_1", N, K, x)
    r = oracle.tol_ratio(y, yr, a)
    assert r <= 1.0, r


@pytest.mark.parametrize("M", [1, 64])
def test_gemm_sparse_rows(M):
    N, K = 256, 1024
    g = synth.rng("gpu-edge", "gemm-sparse", M)
    rows = list(range(0, N, 5))
    ch, cols = _sparse_q4_1(g, N, K, 8, rows)
    X = _x_spread(g, M, K, cols)
    Y = _gemm(ch, N, K, "q4_1", X)
    yr, a = _ref(ch, "q4_1", N, K, X)
    # bf16 weights: 2^-8 of each term, plus the fp32 sums (K terms)
    r = oracle.tol_ratio(Y, yr, a, rel=2.0 ** -8 + K * 2.0 ** -24)
    assert r <= 1.0, r


def _q4k_signed(g, N, K):
    """Q4_K with S of either sign, M = -dmin <= 0 (as a GGUF Q4_K maps), sc/mn over 0..255."""
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    sc = g.integers(0, 256, (N, K // 32), dtype=np.uint8)
    mn = g.integers(0, 256, (N, K // 32), dtype=np.uint8)
    S = _bf(g.standard_normal((N, K // 256)).astype(np.float32) * 1e-3)
    Mv = _bf(-np.abs(g.standard_normal((N, K // 256)).astype(np.float32)) * 1e-3)
    return synth.pack_q4_k(codes, sc, mn, S, Mv)


@pytest.mark.parametrize("N,K", [SMALL, FULL, FULL_K])
@pytest.mark.parametrize("M", [1, 4])
def test_gemv_q4k_signed_full_range(N, K, M):
    g = synth.rng("gpu-edge", "q4k-signed", N, K, M)
    ch = _q4k_signed(g, N, K)
    x = synth.gen_x(g, M, K)
    y = gemv(dev_u8(ch), N, K, "q4_k", x)
    yr, a = _ref(ch, "q4_k", N, K, x)
    assert oracle.tol_ratio(y, yr, a) <= 1.0


@pytest.mark.parametrize("N,K", [(256, 1024), (4096, 4096)])
@pytest.mark.parametrize("M", [1, 64])
def test_gemm_q4k_signed_full_range(N, K, M):
    g = synth.rng("gpu-edge", "gemm-q4k-signed", N, K, M)
    ch = _q4k_signed(g, N, K)
    X = synth.gen_x(g, M, K)
    Y = _gemm(ch, N, K, "q4_k", X)
    yr, a = _ref(ch, "q4_k", N, K, X)
    assert oracle.tol_ratio(Y, yr, a) <= 1.0


def _q8_edge(g, N, K, layout):
    codes = g.integers(-128, 128, (N, K)).astype(np.int8)
    codes[:, ::37] = -128
    d = np.abs(g.standard_normal((N, K // 32)).astype(np.float32)) * 0.02
    d[::3, ::2] = np.ldexp(np.float32(1.5), -130)          # subnormal bf16 scales
    return synth.pack_q8(codes, _bf(d), layout)


@pytest.mark.parametrize("layout", ["A", "B"])
@pytest.mark.parametrize("N,K", [SMALL, (151936 // 4, 2560)])
@pytest.mark.parametrize("M", [1, 4])
def test_gemv_q8_minus128_and_subnormal_scales(layout, N, K, M):
    g = synth.rng("gpu-edge", "q8", layout, N, K, M)
    ch = _q8_edge(g, N, K, layout)
    x = synth.gen_x(g, M, K)
    y = gemv(dev_u8(ch), N, K, "q8", x, layout)
    yr, a = _ref(ch, "q8", N, K, x, layout)
    assert oracle.tol_ratio(y, yr, a) <= 1.0


def _q4_1_subnormal(g, N, K):
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    s = np.abs(g.standard_normal((N, K // 32)).astype(np.float32)) * 0.02
    z = s * (-8 + 0.1 * g.standard_normal((N, K // 32)).astype(np.float32))
    s[::2, ::3] = np.ldexp(np.float32(1.25), -129)          # subnormal scale and zero
    z[::2, ::3] = -np.ldexp(np.float32(1.75), -127)
    return synth.pack_q4_1(codes, _bf(s), _bf(z))


@pytest.mark.parametrize("M", [1, 4])
def test_gemv_q4_1_subnormal_metadata(M):
    N, K = SMALL
    g = synth.rng("gpu-edge", "q41-sub", M)
    ch = _q4_1_subnormal(g, N, K)
    x = synth.gen_x(g, M, K)
    y = gemv(dev_u8(ch), N, K, "q4_1", x)
    yr, a = _ref(ch, "q4_1", N, K, x)
    assert oracle.tol_ratio(y, yr, a) <= 1.0


@pytest.mark.parametrize("M", [1, 64])
def test_gemm_q4_1_subnormal_metadata(M):
    N, K = 256, 1024
    g = synth.rng("gpu-edge", "gemm-q41-sub", M)
    ch = _q4_1_subnormal(g, N, K)
    X = synth.gen_x(g, M, K)
    Y = _gemm(ch, N, K, "q4_1", X)
    yr, a = _ref(ch, "q4_1", N, K, X)
    assert oracle.tol_ratio(Y, yr, a) <= 1.0


def _x_extreme(g, M, K):
    """Activations the fp16 records cannot hold exactly in some groups: one value
    of 2^40 among values near 1 (span above 2^32), bf16 subnormals, a group of
    zeros, values near 2^-100 and 2^100 in groups of their own."""
    x = g.standard_normal((M, K)).astype(np.float32)
    x[:, 5] = 2.0 ** 40
    x[:, 64 + 3] = np.ldexp(np.float32(1.5), -130)
    x[:, 96:128] = 0.0
    x[:, 160:192] *= 2.0 ** -100
    x[:, 224:256] *= 2.0 ** 100
    if M > 1:
        x[1, :] = g.standard_normal(K).astype(np.float32)    # an ordinary row next to them
    return _bf(x)


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 6, 8])
def test_gemv_activation_extremes(kind, M):
    N, K = SMALL
    g = synth.rng("gpu-edge", "x-extreme", kind, M)
    ch = synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)
    x = _x_extreme(g, M, K)
    y = gemv(dev_u8(ch), N, K, kind, x)
    yr, a = _ref(ch, kind, N, K, x)
    assert oracle.tol_ratio(y, yr, a) <= 1.0


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
def test_gemv_batched_rows_of_both_record_forms(kind):
    """Two jobs in one launch, one with ordinary activations and one whose
    activations need the exact fallback, each against the oracle."""
    N, K = 160, 1280
    g = synth.rng("gpu-edge", "mixed-records", kind)
    chs = [synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)
           for _ in range(2)]
    xs = [synth.gen_x(g, 1, K), _x_extreme(g, 1, K)]
    ys = [torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda") for _ in range(2)]
    devs = [dev_u8(c) for c in chs]
    xd = [dev_bf16(x) for x in xs]
    jobs = [(weight(devs[i], N, K, kind), xd[i], ys[i]) for i in range(2)]
    q().gemv_batched(jobs, 1)
    for i in range(2):
        yr, a = _ref(chs[i], kind, N, K, xs[i])
        assert oracle.tol_ratio(host(ys[i]), yr, a) <= 1.0


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
def test_gemv_long_k_many_rows(kind):
    """M = 4 at K = 14336 (the dense 8B down projection's K): prepared records
    beyond 64 KB of LDS."""
    N, K, M = 256, 14336, 4
    g = synth.rng("gpu-edge", "longk", kind)
    ch = synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)
    x = synth.gen_x(g, M, K)
    y = gemv(dev_u8(ch), N, K, kind, x)
    yr, a = _ref(ch, kind, N, K, x)
    assert oracle.tol_ratio(y, yr, a) <= 1.0
