"""GPU routed-expert MoE layer (q4nx_moe_experts) vs the float64 oracle.

Stage-wise checks:
  h  vs silu(G x) * (U x) from the oracle, within the GEMV bar of g and u
     propagated through silu(g) * u;
  d  vs the oracle's Down applied to the GPU's own h (fp32), within
     2e-3 * sum |w h|;
  y  vs the oracle combine of the GPU's own d (fp32 sum of k+1 terms);
and end to end against the all-float64 layer within 2e-3 * a with
a = sum_j |p| sum |Down| |h| + the shared expert's sum |Down_s| |h_s|.

With hot_tokens > 0, experts of prompt-block calls chosen by at least that
many pairs (and the shared expert when T reaches it) run on the bf16 matrix
cores; the same checks hold there.  A token's bits are independent of the
other tokens of the call only with that path off (the default), so the
batch-invariance checks run with it off, and the matrix-core path is checked
against the oracle.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_bf16, dev_f32, dev_i32, dev_u8, have_gpu, host, q, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


class Layer:
    """Routed experts in three device arenas plus a shared expert."""

    def __init__(self, tag, kind, n_exp, D, De, Ds, experts_needed=None, hot_tokens=0):
        self.kind, self.n, self.D, self.De, self.Ds = kind, n_exp, D, De, Ds
        cb = oracle.KIND_BYTES[kind]
        self.gu_bytes = (De // 32) * (D // 256) * cb
        self.dn_bytes = (D // 32) * (De // 256) * cb
        self.host = {}
        arenas = {p: np.zeros((n_exp, b), np.uint8)
                  for p, b in (("gate", self.gu_bytes), ("up", self.gu_bytes), ("down", self.dn_bytes))}
        need = range(n_exp) if experts_needed is None else sorted(set(experts_needed))
        for e in need:
            for p in ("gate", "up", "down"):
                N, K = (De, D) if p != "down" else (D, De)
                ch = self._gen(tag, p, e, N, K)
                arenas[p][e] = ch.reshape(-1)
                self.host[(p, e)] = ch
        self.dev = {p: dev_u8(a) for p, a in arenas.items()}
        self.shared_host = {}
        shared = None
        if Ds:
            sw = []
            for p in ("gate", "up", "down"):
                N, K = (Ds, D) if p != "down" else (D, Ds)
                ch = self._gen(tag, p, "shared", N, K)
                self.shared_host[p] = ch
                d = dev_u8(ch)
                self.dev["s" + p] = d
                sw.append(weight(d, N, K, kind))
            shared = tuple(sw)
        self.L = q().moe_layer(n_exp, D, De, kind, self.dev["gate"], self.dev["up"], self.dev["down"],
                               self.gu_bytes, self.gu_bytes, self.dn_bytes, shared=shared, d_shared=Ds,
                               hot_tokens=hot_tokens)

    def _gen(self, tag, p, e, N, K):
        g = synth.rng("gpu-moe", tag, p, e)
        return synth.gen_q4_1(g, N, K, zero="normal") if self.kind == "q4_1" else synth.gen_q4_k(g, N, K)

    def W(self, e):
        D, De = self.D, self.De
        return (oracle.weights_exact(self.host[("gate", e)], self.kind, De, D),
                oracle.weights_exact(self.host[("up", e)], self.kind, De, D),
                oracle.weights_exact(self.host[("down", e)], self.kind, D, De))

    def Wsh(self):
        if not self.Ds:
            return None
        D, Ds = self.D, self.Ds
        h = self.shared_host
        return (oracle.weights_exact(h["gate"], self.kind, Ds, D),
                oracle.weights_exact(h["up"], self.kind, Ds, D),
                oracle.weights_exact(h["down"], self.kind, D, Ds))

    def run(self, X, ids, p, dbg=True):
        T, k = ids.shape
        ws = torch.zeros(q().moe_ws(self.L, T, k), dtype=torch.uint8, device="cuda")
        Y = torch.full((T, self.D), float("nan"), dtype=torch.float32, device="cuda")
        out = {}
        if dbg:
            out = {"h": torch.zeros((T, k, self.De), dtype=torch.float32, device="cuda"),
                   "d": torch.zeros((T, k, self.D), dtype=torch.float32, device="cuda")}
            if self.Ds:
                out["h_shared"] = torch.zeros((T, self.Ds), dtype=torch.float32, device="cuda")
                out["d_shared"] = torch.zeros((T, self.D), dtype=torch.float32, device="cuda")
        q().moe_experts(self.L, dev_bf16(X), dev_i32(ids), dev_f32(p), Y, T, k, ws, dbg=out or None)
        res = {name: host(t) for name, t in out.items()}
        res["y"] = host(Y)
        res["err"] = int(host(ws[:4]).view(np.uint32)[0])
        return res


def _x64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _check_stages(layer, X, ids, p, r):
    T, k = ids.shape
    D = layer.D
    xs = _x64(X)
    d_ok = np.zeros((T, k), bool)
    worst = {"h": 0.0, "d": 0.0}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if not (0 <= e < layer.n):
                assert np.all(r["d"][t, j] == 0)
                continue
            G, U, Dn = layer.W(e)
            g, u = G @ xs[t], U @ xs[t]
            ag, au = np.abs(G) @ np.abs(xs[t]), np.abs(U) @ np.abs(xs[t])
            h_ref = oracle.swiglu(g, u)
            sil = oracle.silu(g)
            bound = 2e-3 * (1.1 * np.abs(u) * ag + np.abs(sil) * au) + 1e-30
            hg = r["h"][t, j].astype(np.float64)
            worst["h"] = max(worst["h"], float(np.max(np.abs(hg - h_ref) / bound)))
            dref, ad = oracle.gemv_ref(Dn, hg[None, :], x_is_bits=False)
            worst["d"] = max(worst["d"], oracle.tol_ratio(r["d"][t, j][None, :], dref, ad))
            d_ok[t, j] = True
    if layer.Ds:
        G, U, Dn = layer.Wsh()
        for t in range(T):
            g, u = G @ xs[t], U @ xs[t]
            ag, au = np.abs(G) @ np.abs(xs[t]), np.abs(U) @ np.abs(xs[t])
            h_ref = oracle.swiglu(g, u)
            bound = 2e-3 * (1.1 * np.abs(u) * ag + np.abs(oracle.silu(g)) * au) + 1e-30
            hg = r["h_shared"][t].astype(np.float64)
            worst["h"] = max(worst["h"], float(np.max(np.abs(hg - h_ref) / bound)))
            dref, ad = oracle.gemv_ref(Dn, hg[None, :], x_is_bits=False)
            worst["d"] = max(worst["d"], oracle.tol_ratio(r["d_shared"][t][None, :], dref, ad))
    assert worst["h"] <= 1.0 and worst["d"] <= 1.0, worst
    # combine of the GPU's own d, fixed order, fp32: k+1 roundings of sum |p d|
    pv = np.where(d_ok, p.astype(np.float64), 0.0)
    y_ref, _ = oracle.moe_combine_ref(r["d"].astype(np.float64), pv,
                                      r["d_shared"].astype(np.float64) if layer.Ds else None)
    scale = np.einsum("tj,tjn->tn", np.abs(pv), np.abs(r["d"].astype(np.float64)))
    if layer.Ds:
        scale += np.abs(r["d_shared"])
    assert np.all(np.abs(r["y"] - y_ref) <= (k + 2) * 2.0 ** -24 * scale + 1e-30)
    # end to end against the all-float64 layer
    ye, ae = oracle.moe_layer_ref(X, ids, p, layer.W, layer.Wsh(), n_experts=layer.n, with_scale=True)
    e2e = oracle.tol_ratio(r["y"], ye, ae)
    assert e2e <= 1.0, e2e
    return worst, e2e


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("T", [1, 3, 17, 64, 65])
def test_small_moe_stagewise(kind, T):
    layer = Layer("small", kind, 16, 512, 256, 256)
    g = synth.rng("gpu-moe", "route", kind, T)
    ids, p = synth.gen_router(g, T, 16, 4, 1.1)
    X = synth.gen_x(g, T, 512)
    r = layer.run(X, ids, p)
    assert r["err"] == 0
    print(_check_stages(layer, X, ids, p, r))


def test_no_shared_expert_and_k1():
    layer = Layer("noshared", "q4_1", 8, 256, 256, 0)
    g = synth.rng("gpu-moe", "route-ns")
    ids, p = synth.gen_router(g, 5, 8, 1, 1.1)
    X = synth.gen_x(g, 5, 256)
    r = layer.run(X, ids, p)
    _check_stages(layer, X, ids, p, r)


def test_out_of_range_ids_flagged_and_skipped():
    layer = Layer("badid", "q4_1", 16, 512, 256, 256)
    g = synth.rng("gpu-moe", "route-bad")
    ids, p = synth.gen_router(g, 6, 16, 4, 1.1)
    X = synth.gen_x(g, 6, 512)
    bad = ids.copy()
    bad[1, 2] = -1
    bad[4, 0] = 16 + 5
    r = layer.run(X, bad, p)
    assert r["err"] & 1
    # the same call with those slots routed to a valid expert at weight 0 gives the same bits
    alt, palt = ids.copy(), p.copy()
    alt[1, 2], alt[4, 0] = 0, 0
    palt[1, 2], palt[4, 0] = 0.0, 0.0
    r2 = layer.run(X, alt, palt)
    assert r2["err"] == 0
    np.testing.assert_array_equal(r["y"].view(np.uint32), r2["y"].view(np.uint32))
    _check_stages(layer, X, bad, p, r)


@pytest.mark.parametrize("case", ["repeat", "bad"])
def test_block_routing_with_repeated_or_bad_ids(case):
    """A 20-token block (routed through the route kernel) where one token names
    the same expert in two slots, or where ids are out of range: the same
    results as the oracle's slot-by-slot sum, and for bad ids the error flag."""
    layer = Layer("blockroute", "q4_1", 16, 512, 256, 256)
    g = synth.rng("gpu-moe", "route-block", case)
    ids, p = synth.gen_router(g, 20, 16, 4, 1.1)
    X = synth.gen_x(g, 20, 512)
    ids = ids.copy()
    if case == "repeat":
        ids[3, 1] = ids[3, 0]
        ids[11, 3] = ids[11, 2]
    else:
        ids[2, 1] = -3
        ids[17, 0] = 16
    r = layer.run(X, ids, p)
    assert r["err"] == (1 if case == "bad" else 0)
    _check_stages(layer, X, ids, p, r)


def test_token_result_does_not_depend_on_its_batch():
    """With the matrix-core path off (the default), a token alone (T=1) and
    inside a 64-token block get the same bits."""
    layer = Layer("batch", "q4_1", 16, 512, 256, 256)
    g = synth.rng("gpu-moe", "route-batch")
    ids, p = synth.gen_router(g, 64, 16, 4, 1.1)
    X = synth.gen_x(g, 64, 512)
    full = layer.run(X, ids, p, dbg=False)
    for t in (0, 13, 63):
        one = layer.run(X[t:t + 1], ids[t:t + 1], p[t:t + 1], dbg=False)
        np.testing.assert_array_equal(one["y"][0].view(np.uint32), full["y"][t].view(np.uint32))


def _weights(g, T, k):
    p = g.random((T, k)).astype(np.float32) + np.float32(0.05)
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("per_expert", [1, 2])
def test_block_of_one_or_two_tokens_per_expert(kind, per_expert):
    """An 80-pair block (routed through the route kernel) where every expert is
    picked by exactly one token (all routed batches in the one-token launch) or
    by exactly two (none there): against the oracle stage by stage, and each
    sampled token's bits equal to the same token routed alone."""
    T, k = 20, 4
    n = T * k // per_expert
    layer = Layer(f"pertok{per_expert}", kind, n, 512, 256, 256)
    g = synth.rng("gpu-moe", "per-expert", kind, per_expert)
    if per_expert == 1:
        ids = g.permutation(n).astype(np.int32).reshape(T, k)
    else:   # tokens 2i and 2i + 1 share experts 4i .. 4i + 3
        ids = np.array([[4 * (t // 2) + j for j in range(k)] for t in range(T)], np.int32)
    p = _weights(g, T, k)
    X = synth.gen_x(g, T, 512)
    r = layer.run(X, ids, p)
    assert r["err"] == 0
    print(_check_stages(layer, X, ids, p, r))
    for t in (0, 7, T - 1):
        one = layer.run(X[t:t + 1], ids[t:t + 1], p[t:t + 1], dbg=False)
        np.testing.assert_array_equal(one["y"][0].view(np.uint32), r["y"][t].view(np.uint32))


def test_repeat_bit_identical():
    layer = Layer("rep", "q4_k", 16, 512, 256, 256)
    g = synth.rng("gpu-moe", "route-rep")
    ids, p = synth.gen_router(g, 33, 16, 4, 1.1)
    X = synth.gen_x(g, 33, 512)
    a = layer.run(X, ids, p, dbg=False)
    b = layer.run(X, ids, p, dbg=False)
    np.testing.assert_array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32))


@pytest.mark.parametrize("T", [1, 64])
def test_moe_512x10_layer_full_size(T):
    """512 experts of 512x2048 / 2048x512 plus a 1024-wide shared expert, top-10."""
    ids, p = synth.moe_router(0, T)
    layer = Layer("full", "q4_1", synth.MOE_EXPERTS, synth.MOE_D_MODEL, synth.MOE_D_EXPERT,
                  synth.MOE_D_SHARED, experts_needed=ids.ravel().tolist())
    X = synth.gen_x(synth.rng("moe_512x10", 0, "X", T), T, synth.MOE_D_MODEL)
    r = layer.run(X, ids, p)
    assert r["err"] == 0
    sel = [0] if T == 1 else [0, 31, 63]
    sub = {name: (v[sel] if name not in ("err",) else v) for name, v in r.items()}
    _check_stages(layer, X[sel], ids[sel], p[sel], sub)


@pytest.mark.parametrize("T,k", [(1024, 4), (4096, 1)])
def test_maximum_pairs(T, k):
    """T * k at its limit of 4096 pairs (the sort in one workgroup's LDS): every
    token's output against the oracle's slot-by-slot sum on a sample of tokens,
    and a token's bits equal to the same token routed alone."""
    layer = Layer("maxpairs", "q4_1", 16, 512, 256, 256)
    g = synth.rng("gpu-moe", "maxpairs", T, k)
    ids, p = synth.gen_router(g, T, 16, k, 1.1)
    X = synth.gen_x(g, T, 512)
    sel = [0, 1, T // 2, T - 1]
    for hot in (1, 0):   # every expert on the matrix cores, then none
        layer.L.hot_tokens = hot
        r = layer.run(X, ids, p)
        assert r["err"] == 0
        sub = {name: (v[sel] if name != "err" else v) for name, v in r.items()}
        _check_stages(layer, X[sel], ids[sel], p[sel], sub)
    for t in (0, T - 1):
        one = layer.run(X[t:t + 1], ids[t:t + 1], p[t:t + 1], dbg=False)
        np.testing.assert_array_equal(one["y"][0].view(np.uint32), r["y"][t].view(np.uint32))


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("hot", [1, 9, -1])
def test_matrix_core_experts(kind, hot):
    """hot_tokens 1: every expert of a prompt block (and the shared expert) on
    the matrix cores; 9: the popular ones only; -1: none (as 0, the default).  Stage-wise and end
    to end against the oracle each time, with 70 tokens (two 64-row blocks for
    the shared expert and the most popular experts) and a d_model of 768
    (an odd number of tile columns)."""
    layer = Layer("hot", kind, 24, 768, 256, 512, hot_tokens=hot)
    g = synth.rng("gpu-moe", "hot", kind)
    ids, p = synth.gen_router(g, 70, 24, 6, 1.1)
    X = synth.gen_x(g, 70, 768)
    r = layer.run(X, ids, p)
    assert r["err"] == 0
    counts = np.bincount(ids.ravel(), minlength=24)
    assert counts.max() > 64 and (counts < 9).any() and (counts >= 9).any()
    print(_check_stages(layer, X, ids, p, r))


@pytest.mark.parametrize("hot", [5, 8])
def test_matrix_core_experts_full_size_block(hot):
    """The 512-expert layer's 64-token block with experts of `hot` or more pairs
    on the matrix cores, and the same call with that path off: every sampled
    output within the bar of the oracle's scale."""
    T = 64
    ids, p = synth.moe_router(0, T)
    layer = Layer("full", "q4_1", synth.MOE_EXPERTS, synth.MOE_D_MODEL, synth.MOE_D_EXPERT,
                  synth.MOE_D_SHARED, experts_needed=ids.ravel().tolist(), hot_tokens=hot)
    X = synth.gen_x(synth.rng("moe_512x10", 0, "X", T), T, synth.MOE_D_MODEL)
    counts = np.bincount(ids.ravel(), minlength=synth.MOE_EXPERTS)
    assert (counts >= hot).sum() >= 5
    a = layer.run(X, ids, p, dbg=False)
    layer.L.hot_tokens = 0
    b = layer.run(X, ids, p, dbg=False)
    sel = [0, 17, 40, 63]
    ye, ae = oracle.moe_layer_ref(X[sel], ids[sel], p[sel], layer.W, layer.Wsh(), n_experts=layer.n,
                                  with_scale=True)
    assert oracle.tol_ratio(a["y"][sel], ye, ae) <= 1.0
    assert oracle.tol_ratio(b["y"][sel], ye, ae) <= 1.0
    assert not np.array_equal(a["y"], b["y"])   # the two paths did run
