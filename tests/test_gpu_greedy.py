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

from _gpu import dev_bf16, dev_f32, dev_i32, dev_u8, have_gpu, host, q, torch, weight

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
