"""The allocation-free block GEMM (q4nx_gemm_block_noalloc) against q4nx_gemm_block.

Both run the same kernels; the allocation-free one takes its workspace from the
library's static array.  Two calls in a row, the second on a smaller input
(fewer rows, shorter K, smaller M, the other chunk kind), each checked against
q4nx_gemm_block on the same inputs and against the float64 oracle, to the
floating-point bar |y - y_ref| <= 2e-3 * sum |w x|.  A third call needs no
split (and so no workspace at all).
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_bf16, dev_u8, have_gpu, host, q, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _case(kind, N, K, M, tag):
    g = synth.rng("gpu-noalloc", tag, kind, N, K, M)
    ch = synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)
    X = synth.gen_x(g, M, K)
    return ch, X


def _both(kind, N, K, M, tag):
    ch, X = _case(kind, N, K, M, tag)
    w = weight(dev_u8(ch), N, K, kind)
    Xd = dev_bf16(X)
    Ya = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    Yb = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    n = q().gemm_block_ws(w)
    assert n <= q().gemm_block_noalloc_max()
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")
    q().gemm_block_noalloc(w, Xd, Yb, M)     # first: in a fresh process, before any probe of the XCDs
    q().gemm_block(w, Xd, Ya, M, ws)
    yr, a = oracle.gemv_ref(oracle.weights_exact(ch, kind, N, K), X)
    return host(Ya), host(Yb), yr, a, n


def test_two_calls_in_a_row_second_smaller():
    print("noalloc: q4_1 2048 x 8192, M = 64", flush=True)
    ya, yb, yr, a, n = _both("q4_1", 2048, 8192, 64, "first")
    assert n > 4096                                   # K is split: the workspace is used
    assert np.isfinite(yb).all()
    assert oracle.tol_ratio(yb, ya, a) <= 1.0
    assert oracle.tol_ratio(yb, yr, a) <= 1.0
    print("noalloc: q4_k 1024 x 4096, M = 16", flush=True)
    ya, yb, yr, a, n = _both("q4_k", 1024, 4096, 16, "second")
    assert n > 4096
    assert np.isfinite(yb).all()
    assert oracle.tol_ratio(yb, ya, a) <= 1.0
    assert oracle.tol_ratio(yb, yr, a) <= 1.0


def test_call_without_split_and_repeat():
    print("noalloc: q4_1 8192 x 512, M = 3 (no split), then a split call again", flush=True)
    ya, yb, yr, a, n = _both("q4_1", 8192, 512, 3, "nosplit")
    assert n == 0
    assert oracle.tol_ratio(yb, ya, a) <= 1.0
    assert oracle.tol_ratio(yb, yr, a) <= 1.0
    ya, yb, yr, a, n = _both("q4_k", 1024, 8192, 1, "again")
    assert n > 4096
    assert oracle.tol_ratio(yb, ya, a) <= 1.0
    assert oracle.tol_ratio(yb, yr, a) <= 1.0


def test_rejects_bad_arguments():
    ch, X = _case("q4_1", 64, 512, 2, "bad")
    w = weight(dev_u8(ch), 64, 512, "q4_1")
    Y = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(q().Q4nxError):
        q().gemm_block_noalloc(w, dev_bf16(X), Y, 0)
    with pytest.raises(q().Q4nxError):
        q().gemm_block_noalloc(w, dev_bf16(X), Y, 65)
