"""GPU MoE router (q4nx_moe_router) vs the oracle.

Logits: fp32 dot products against the float64 reference, within the GEMV bar
2e-3 * sum |r x|.  Picks and weights: the ranking is an fp32 decision, so the
oracle's top-k (oracle.router_topk) runs on the device's own fp32 logits and
the ids must match exactly (lower id first among equal logits); the weights
match that float64 softmax within fp32 rounding.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_bf16, dev_f32, dev_i32, have_gpu, host, q, torch

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _router_inputs(tag, T, E, D, dup=False):
    g = synth.rng("gpu-router", tag, T, E, D)
    R = synth.bf16_bits((g.standard_normal((E, D)) * 0.05).astype(np.float32))
    if dup:   # equal rows give equal fp32 logits: ties broken by the lower id
        R[7] = R[300 % E]
        R[11] = R[7]
    X = synth.gen_x(g, T, D)
    return R, X


def _run(R, X, k, renorm=True):
    T, D = X.shape
    E = R.shape[0]
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    p = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    q().moe_router(dev_bf16(R), dev_bf16(X), T, D, E, k, ids, p, lg, renorm=renorm)
    return host(ids), host(p), host(lg)


@pytest.mark.parametrize("T", [1, 5, 64])
@pytest.mark.parametrize("renorm", [True, False])
def test_router_matches_oracle(T, renorm):
    E, D, k = 512, 2048, 10
    R, X = _router_inputs("main", T, E, D)
    ids, p, lg = _run(R, X, k, renorm)
    z, a = oracle.router_logits_ref(R, X)
    assert oracle.tol_ratio(lg, z, a) <= 1.0
    want_ids, want_p = oracle.router_topk(lg, k, renormalize=renorm)
    np.testing.assert_array_equal(ids, want_ids)
    np.testing.assert_allclose(p, want_p, rtol=4e-6, atol=0)


def test_router_ties_and_small_shapes():
    for E, D, k in ((512, 2048, 10), (64, 512, 16), (10, 1024, 10)):
        R, X = _router_inputs("ties", 3, E, D, dup=E > 300)
        ids, p, lg = _run(R, X, k)
        want_ids, want_p = oracle.router_topk(lg, k)
        np.testing.assert_array_equal(ids, want_ids)
        np.testing.assert_allclose(p, want_p, rtol=4e-6, atol=0)
        for t in range(3):
            assert len(set(ids[t].tolist())) == k


def test_router_feeds_moe_on_device():
    """Router ids/p straight into q4nx_moe_experts give the same bits as the
    same ids/p passed in from the host."""
    from test_gpu_moe import Layer
    E, D, De, Ds, k, T = 16, 512, 256, 256, 4, 6
    layer = Layer("router-chain", "q4_1", E, D, De, Ds)
    g = synth.rng("gpu-router", "chain")
    R = synth.bf16_bits((g.standard_normal((E, D)) * 0.05).astype(np.float32))
    X = synth.gen_x(g, T, D)
    ids_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    p_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    Xd = dev_bf16(X)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    q().moe_router(dev_bf16(R), Xd, T, D, E, k, ids_d, p_d, lg)
    ws = torch.zeros(q().moe_ws(layer.L, T, k), dtype=torch.uint8, device="cuda")
    Y1 = torch.empty((T, D), dtype=torch.float32, device="cuda")
    q().moe_experts(layer.L, Xd, ids_d, p_d, Y1, T, k, ws)
    ids_h, p_h = host(ids_d), host(p_d)
    Y2 = torch.empty((T, D), dtype=torch.float32, device="cuda")
    q().moe_experts(layer.L, Xd, dev_i32(ids_h), dev_f32(p_h), Y2, T, k, ws)
    np.testing.assert_array_equal(host(Y1).view(np.uint32), host(Y2).view(np.uint32))
