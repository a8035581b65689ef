"""The block GEMM's split-K exchange: correct wherever the workgroups land.

* Every exchange mode (q4nx_gemm_exchange_mode) against the float64 oracle:
  the XCD-local exchange, the same with every odd group's workgroups acting
  displaced (they compute their rows whole), and the device-coherent exchange.
  After each call the workspace header (arrival counters, claim words, rescue
  flags) is back to zero.
* Split-K GEMMs on one stream while another stream of the same priority runs
  GEMVs, so that the two kernels' workgroups interleave on the XCDs: both
  against the oracle.
* A fresh process whose first library call is a split-K GEMM inside a graph
  capture (the XCD probe never runs on the caller's stream or during capture).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_bf16, dev_u8, gemv, have_gpu, host, q, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

HDR_WORDS = 768      # counters, claim words, rescue flags (the diagnostic words follow)


def _gen(kind, N, K, tag):
    g = synth.rng("gpu-gemm-x", tag, kind, N, K)
    return synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)


@pytest.fixture
def exchange_mode():
    yield q().gemm_exchange_mode
    q().gemm_exchange_mode(0)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("M", [1, 64])
def test_exchange_modes_match_oracle(exchange_mode, mode, kind, M):
    N, K = 1024, 8192                        # few tile rows, long K: K is split
    ch = _gen(kind, N, K, "modes")
    w = weight(dev_u8(ch), N, K, kind)
    n = q().gemm_block_ws(w)
    assert n > 4096
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    X = synth.gen_x(synth.rng("gpu-gemm-x", "modesX", M), M, K)
    yr, a = oracle.gemv_ref(oracle.weights_exact(ch, kind, N, K), X)
    exchange_mode(mode)
    for rep in range(3):
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        q().gemm_block(w, dev_bf16(X), Y, M, ws)
        r = oracle.tol_ratio(host(Y), yr, a)
        assert r <= 1.0, (mode, rep, r)
        hdr = host(ws[:4 * HDR_WORDS]).view(np.uint32)
        assert np.count_nonzero(hdr) == 0, np.nonzero(hdr)


def test_split_k_concurrent_with_gemvs_on_another_stream():
    N, K, M = 1024, 8192, 64
    ch = _gen("q4_1", N, K, "conc")
    w = weight(dev_u8(ch), N, K, "q4_1")
    ws = torch.zeros(q().gemm_block_ws(w), dtype=torch.uint8, device="cuda")
    X = synth.gen_x(synth.rng("gpu-gemm-x", "concX"), M, K)
    yr, a = oracle.gemv_ref(oracle.weights_exact(ch, "q4_1", N, K), X)
    # GEMVs of a 2560 x 2560 weight, 40 launches per round, on a second stream
    gN, gK = 2560, 2560
    gch = synth.gen_q4_1(synth.rng("gpu-gemm-x", "concw"), gN, gK, zero="normal")
    gw = weight(dev_u8(gch), gN, gK, "q4_1")
    gx = synth.gen_x(synth.rng("gpu-gemm-x", "concx"), 1, gK)
    gyr, ga = oracle.gemv_ref(oracle.weights_exact(gch, "q4_1", gN, gK), gx)
    gxd = dev_bf16(gx)
    other = torch.cuda.Stream()
    main = torch.cuda.Stream()
    Xd = dev_bf16(X)
    gys = [torch.full((1, gN), float("nan"), dtype=torch.float32, device="cuda") for _ in range(40)]
    Ys = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for _ in range(8)]
    torch.cuda.synchronize()
    for rnd in range(4):
        with torch.cuda.stream(other):
            for gy in gys:
                q().gemv(gw, gxd, gy, 1, stream=other)
        with torch.cuda.stream(main):
            for Y in Ys:
                q().gemm_block(w, Xd, Y, M, ws, stream=main)
        torch.cuda.synchronize()
        for Y in Ys:
            assert oracle.tol_ratio(host(Y), yr, a) <= 1.0, rnd
            Y.fill_(float("nan"))
        for gy in gys:
            assert oracle.tol_ratio(host(gy), gyr, ga) <= 1.0, rnd
            gy.fill_(float("nan"))
        hdr = host(ws[:4 * HDR_WORDS]).view(np.uint32)
        assert np.count_nonzero(hdr) == 0
    displaced = int(host(ws[q().GEMM_WS_DIAG_OFFSET:q().GEMM_WS_DIAG_OFFSET + 4]).view(np.uint32)[0])
    print("workgroups that found their XCD slot taken:", displaced)


_CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import gemm_q4nx_chunk_amd as q
import oracle, synth
N, K, M = 1024, 8192, 64
g = synth.rng("gpu-gemm-x", "child")
ch = synth.gen_q4_1(g, N, K, zero="normal")
X = synth.gen_x(g, M, K)
dev = torch.from_numpy(ch.reshape(-1)).cuda()
w = q.weight(dev, N, K, "q4_1")
ws = torch.zeros(q.gemm_block_ws(w), dtype=torch.uint8, device="cuda")
Xd = torch.from_numpy(X.view(np.int16)).cuda()
Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
s = torch.cuda.Stream()
torch.cuda.synchronize()
gr = torch.cuda.CUDAGraph()
with torch.cuda.graph(gr, stream=s):
    q.gemm_block(w, Xd, Y, M, ws)          # the first library call of the process
torch.cuda.synchronize()
yr, a = oracle.gemv_ref(oracle.weights_exact(ch, "q4_1", N, K), X)
for rep in range(3):
    Y.fill_(float("nan"))
    torch.cuda.synchronize()
    gr.replay()
    torch.cuda.synchronize()
    r = oracle.tol_ratio(Y.cpu().numpy(), yr, a)
    assert r <= 1.0, r
# an eager call after the capture, then the graph again
q.gemm_block(w, Xd, Y, M, ws)
torch.cuda.synchronize()
assert oracle.tol_ratio(Y.cpu().numpy(), yr, a) <= 1.0
gr.replay()
torch.cuda.synchronize()
assert oracle.tol_ratio(Y.cpu().numpy(), yr, a) <= 1.0
print("child ok")
"""


def test_first_call_inside_graph_capture_in_a_fresh_process():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("child: split-K GEMM captured as the first library call", flush=True)
    r = subprocess.run([sys.executable, "-c", _CHILD, root], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "child ok" in r.stdout
