"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test ties the oracle to something fixed independently: the chunk sizes
and decode formulas of the 1bit engine docs (page "NPU engine", section
"Q4NX chunks"), hand-worked chunks under tests/golden, exact rational
arithmetic, a per-weight brute-force decoder, closed forms (the Q4_0 mapping
zero = -8*scale of section "From a GGUF", one-hot activations), and
invariants (the two Q8 layouts of one tensor, the Q4_K -> q4_1 repack bound).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle.decode import decode_fields, scalar_decode_chunk, weights_exact, weights_f32


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def _golden_cases():
    here = os.path.join(os.path.dirname(__file__), "golden", "chunks_hand.json")
    with open(here) as f:
        return json.load(f)["cases"]


def _chunk_from_writes(kind, writes):
    b = bytearray(oracle.KIND_BYTES[kind])
    for off, hexs in writes:
        data = bytes.fromhex(hexs)
        b[off:off + len(data)] = data
    return bytes(b)


def _rne_f32(q: Fraction) -> float:
    """Round an exact rational to the nearest float32 (ties to even), from scratch."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    qexp = max(e, -126) - 23                 # quantum of the binade (subnormals: 2^-149)
    scaled = q / (Fraction(2) ** qexp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n) * Fraction(2) ** qexp)


def _finite_bf16(g, n):
    """Random bf16 bit patterns over the whole exponent range short of overflow
    (|v| < 2^113, so products with a code or a u8 stay finite in float32)."""
    b = g.integers(0, 1 << 16, n, dtype=np.uint16)
    exp = np.minimum((b >> 7) & 0xFF, 0xF0).astype(np.uint16)
    return (b & np.uint16(0x807F)) | (exp << np.uint16(7))


def _bf16_fraction(bits: int) -> Fraction:
    return Fraction(float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]))


# ----------------------------------------------------------------------------
# sizes and layouts
# ----------------------------------------------------------------------------
def test_chunk_byte_budgets_are_the_pages_sizes():
    tile = 32 * 256
    # q4_1: 4-bit codes + (bf16 scale, bf16 zero) per 32 columns of each row
    assert tile // 2 + (tile // 32) * 4 == 5120 == oracle.KIND_BYTES["q4_1"]
    # Q4_K: 4-bit codes + (u8 scale, u8 min) per 32 columns + (bf16 S, bf16 M) per row
    assert tile // 2 + (tile // 32) * 2 + 32 * 4 == 4736 == oracle.KIND_BYTES["q4_k"]
    # Q8: int8 codes + bf16 scale per 32 columns
    assert tile + (tile // 32) * 2 == 8704 == oracle.KIND_BYTES["q8"]


@pytest.mark.parametrize("layout", ["A", "B"])
def test_q8_layout_formulas_are_bijections(layout):
    r = np.arange(32)[:, None]
    k = np.arange(256)[None, :]
    if layout == "A":
        off = k * 32 + r
    else:
        off = (r // 16) * 4096 + (k // 32) * 512 + (k % 32) * 16 + r % 16
    assert np.array_equal(np.sort(off.ravel()), np.arange(8192))


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_hand_chunks(case):
    kind, layout = case["kind"], case.get("layout")
    chunk = _chunk_from_writes(kind, case["writes"])
    W = weights_exact(np.frombuffer(chunk, np.uint8), kind, 32, 256, layout)
    S = scalar_decode_chunk(chunk, kind, layout)
    for r, k, v in case["expect"]:
        assert W[r, k] == v, (r, k, W[r, k], v)
        assert S[r][k] == v, (r, k, S[r][k], v)


def test_q8_needs_a_layout():
    ch = np.zeros(8704, np.uint8)
    with pytest.raises(ValueError):
        decode_fields(ch, "q8", 32, 256, None)


def test_unknown_kind_and_short_tensor_refused():
    with pytest.raises(ValueError):
        decode_fields(np.zeros(5000, np.uint8), "q5", 32, 256)
    with pytest.raises(ValueError):
        decode_fields(np.zeros(5119, np.uint8), "q4_1", 32, 256)
    with pytest.raises(ValueError):
        decode_fields(np.zeros(5120 * 2, np.uint8), "q4_1", 48, 256)


# ----------------------------------------------------------------------------
# brute force and round trips
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind,layout", [("q4_1", None), ("q4_k", None), ("q8", "A"), ("q8", "B")])
@pytest.mark.parametrize("TR,TC", [(1, 1), (2, 3)])
def test_vectorised_decoder_matches_brute_force(kind, layout, TR, TC):
    g = synth.rng("pin", "brute", kind, layout or "-", TR, TC)
    raw = np.frombuffer(g.bytes(TR * TC * oracle.KIND_BYTES[kind]), np.uint8).reshape(TR, TC, -1)
    W = weights_exact(raw, kind, 32 * TR, 256 * TC, layout)
    for tr in range(TR):
        for tc in range(TC):
            ref = np.array(scalar_decode_chunk(raw[tr, tc].tobytes(), kind, layout))
            got = W[32 * tr:32 * tr + 32, 256 * tc:256 * tc + 256]
            np.testing.assert_array_equal(got, ref)


def test_pack_decode_round_trip_q4_1():
    g = synth.rng("pin", "rt", "q4_1")
    N, K = 64, 512
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    sb = g.integers(0, 1 << 16, (N, K // 32), dtype=np.uint16)
    zb = g.integers(0, 1 << 16, (N, K // 32), dtype=np.uint16)
    f = decode_fields(synth.pack_q4_1(codes, sb, zb), "q4_1", N, K)
    assert np.array_equal(f["codes"], codes)
    assert np.array_equal(f["scale"], sb) and np.array_equal(f["zero"], zb)


def test_pack_decode_round_trip_q4_k():
    g = synth.rng("pin", "rt", "q4_k")
    N, K = 64, 512
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    sc = g.integers(0, 256, (N, K // 32), dtype=np.uint8)
    mn = g.integers(0, 256, (N, K // 32), dtype=np.uint8)
    S = g.integers(0, 1 << 16, (N, K // 256), dtype=np.uint16)
    M = g.integers(0, 1 << 16, (N, K // 256), dtype=np.uint16)
    f = decode_fields(synth.pack_q4_k(codes, sc, mn, S, M), "q4_k", N, K)
    for name, v in (("codes", codes), ("sc", sc), ("mn", mn), ("S", S), ("M", M)):
        assert np.array_equal(f[name], v), name


@pytest.mark.parametrize("layout", ["A", "B"])
def test_pack_decode_round_trip_q8(layout):
    g = synth.rng("pin", "rt", "q8", layout)
    N, K = 64, 512
    codes = g.integers(-128, 128, (N, K), dtype=np.int8)
    d = g.integers(0, 1 << 16, (N, K // 32), dtype=np.uint16)
    f = decode_fields(synth.pack_q8(codes, d, layout), "q8", N, K, layout)
    assert np.array_equal(f["codes"], codes) and np.array_equal(f["d"], d)


def test_q8_layouts_of_one_tensor_decode_identically():
    g = synth.rng("pin", "q8ab")
    N, K = 96, 768
    A = synth.gen_q8(g, N, K, "A")
    B = synth.q8_relayout(A, "A", "B")
    assert not np.array_equal(A, B)
    np.testing.assert_array_equal(weights_exact(A, "q8", N, K, "A"), weights_exact(B, "q8", N, K, "B"))
    np.testing.assert_array_equal(synth.q8_relayout(B, "B", "A"), A)
    x = synth.gen_x(g, 2, K)
    ya, _ = oracle.gemv_ref(weights_exact(A, "q8", N, K, "A"), x)
    yb, _ = oracle.gemv_ref(weights_exact(B, "q8", N, K, "B"), x)
    np.testing.assert_array_equal(ya, yb)


# ----------------------------------------------------------------------------
# exact values and closed forms
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind,layout", [("q4_1", None), ("q4_k", None), ("q8", "B")])
def test_float32_decode_is_one_rounding_of_the_exact_value(kind, layout):
    g = synth.rng("pin", "exact", kind)
    raw = np.frombuffer(g.bytes(oracle.KIND_BYTES[kind]), np.uint8).copy()
    if kind == "q4_1":   # keep metadata finite, include subnormal and huge magnitudes
        meta = _finite_bf16(g, 512)
        meta[::7] &= 0x807F          # subnormals
        raw[4096:] = meta.view(np.uint8)
    elif kind == "q4_k":
        sm = _finite_bf16(g, 64)
        sm[::5] &= 0x807F
        raw[4608:] = sm.view(np.uint8)
    else:
        raw[8192:] = _finite_bf16(g, 256).view(np.uint8)
    f = decode_fields(raw, kind, 32, 256, layout)
    W32 = weights_f32(raw, kind, 32, 256, layout)
    for idx in g.integers(0, 32 * 256, 600):
        r, k = divmod(int(idx), 256)
        grp = k // 32
        c = int(f["codes"][r, k])
        if kind == "q4_1":
            q = c * _bf16_fraction(int(f["scale"][r, grp])) + _bf16_fraction(int(f["zero"][r, grp]))
        elif kind == "q4_k":
            q = (_bf16_fraction(int(f["S"][r, 0])) * int(f["sc"][r, grp]) * c
                 + _bf16_fraction(int(f["M"][r, 0])) * int(f["mn"][r, grp]))
        else:
            q = _bf16_fraction(int(f["d"][r, grp])) * c
        assert float(W32[r, k]) == _rne_f32(q), (r, k)


def test_q4_0_mapping_closed_form():
    """zero = -8*scale (the Q4_0 row of the GGUF table) gives w = scale*(code-8) exactly."""
    g = synth.rng("pin", "q40")
    N, K = 64, 512
    ch = synth.gen_q4_1(g, N, K, zero="minus8")
    f = decode_fields(ch, "q4_1", N, K)
    s = np.repeat((f["scale"].astype(np.uint32) << 16).view(np.float32).astype(np.float64), 32, axis=1)
    centred = f["codes"].astype(np.int64) - 8
    np.testing.assert_array_equal(weights_exact(ch, "q4_1", N, K), s * centred)
    # and the GEMV is sum over groups of scale * sum (code-8) x, evaluated exactly
    x = synth.gen_x(g, 1, K)
    xf = [Fraction(float(v)) for v in (x[0].astype(np.uint32) << 16).view(np.float32)]
    y, _ = oracle.gemv_ref(weights_exact(ch, "q4_1", N, K), x)
    for n in range(0, N, 7):
        exact = Fraction(0)
        for grp in range(K // 32):
            inner = sum(int(centred[n, grp * 32 + j]) * xf[grp * 32 + j] for j in range(32))
            exact += Fraction(float(s[n, grp * 32])) * inner
        assert abs(y[0, n] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


@pytest.mark.parametrize("kind,layout", [("q4_1", None), ("q4_k", None), ("q8", "A")])
def test_one_hot_activation_returns_a_column(kind, layout):
    g = synth.rng("pin", "onehot", kind)
    N, K = 64, 512
    ch = {"q4_1": lambda: synth.gen_q4_1(g, N, K, zero="normal"),
          "q4_k": lambda: synth.gen_q4_k(g, N, K),
          "q8": lambda: synth.gen_q8(g, N, K, "A")}[kind]()
    W = weights_exact(ch, kind, N, K, layout)
    for k in (0, 31, 32, 255, 256, 511):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80                     # 1.0
        y, a = oracle.gemv_ref(W, x)
        np.testing.assert_array_equal(y[0], W[:, k])
        np.testing.assert_array_equal(a[0], np.abs(W[:, k]))


def test_gemv_ref_matches_brute_force_sum():
    g = synth.rng("pin", "fsum")
    ch = synth.gen_q4_1(g, 32, 256, zero="normal")
    x = synth.gen_x(g, 2, 256)
    W_brute = np.array(scalar_decode_chunk(ch[0, 0].tobytes(), "q4_1"))
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y, a = oracle.gemv_ref(weights_exact(ch, "q4_1", 32, 256), x)
    for m in range(2):
        for n in range(32):
            exact = math.fsum((W_brute[n] * xv[m]).tolist())
            assert abs(y[m, n] - exact) <= 1e-13 * a[m, n]
            assert a[m, n] == pytest.approx(math.fsum(np.abs(W_brute[n] * xv[m]).tolist()), rel=1e-14)
    y2, a2 = oracle.gemv_ref(weights_exact(ch, "q4_1", 32, 256), x, exact_sum=True)
    np.testing.assert_allclose(y2, y, rtol=0, atol=1e-12 * a.max())


# ----------------------------------------------------------------------------
# repack
# ----------------------------------------------------------------------------
def test_q4k_to_q41_repack_codes_and_rounding():
    g = synth.rng("pin", "repack")
    N, K = 64, 512
    ch = synth.gen_q4_k(g, N, K)
    codes, sb, zb = oracle.repack_q4k_to_q41(ch, N, K)
    f = decode_fields(ch, "q4_k", N, K)
    assert np.array_equal(codes, f["codes"])
    for n in range(0, N, 5):
        for grp in range(0, K // 32, 3):
            S = _bf16_fraction(int(f["S"][n, grp // 8]))
            M = _bf16_fraction(int(f["M"][n, grp // 8]))
            want_s = _rne_bf16(S * int(f["sc"][n, grp]))
            want_z = _rne_bf16(M * int(f["mn"][n, grp]))
            assert int(sb[n, grp]) == want_s and int(zb[n, grp]) == want_z
    w41 = weights_exact(synth.pack_q4_1(codes, sb, zb), "q4_1", N, K)
    w4k = weights_exact(ch, "q4_k", N, K)
    bound = oracle.repack_bound(ch, N, K)
    diff = np.abs(w41 - w4k)
    assert np.all(diff <= bound)
    assert diff.max() > 0                       # the repack is not exact in general


def _rne_bf16(q: Fraction) -> int:
    """Nearest-even bf16 bits of an exact rational that is exact in float32."""
    f = np.float32(float(q))
    assert Fraction(float(f)) == q
    u = int(f.view(np.uint32))
    lower = u >> 16
    rest = u & 0xFFFF
    if rest > 0x8000 or (rest == 0x8000 and lower & 1):
        lower += 1
    return lower


# ----------------------------------------------------------------------------
# tolerance rule, SwiGLU, MoE
# ----------------------------------------------------------------------------
def test_tolerance_rule():
    y_ref = np.array([1.0, 0.0, -2.0])
    a = np.array([10.0, 0.0, 4.0])
    assert oracle.tol_ratio(y_ref, y_ref, a) == 0.0
    assert oracle.check_tol(y_ref + np.array([0.019, 0, 0]), y_ref, a)
    assert not oracle.check_tol(y_ref + np.array([0.021, 0, 0]), y_ref, a)
    assert not oracle.check_tol(y_ref + np.array([0, 1e-30, 0]), y_ref, a)   # a = 0 demands exact
    assert not oracle.check_tol(np.array([np.nan, 0, -2.0]), y_ref, a)


def test_silu_identities():
    z = np.linspace(-30, 30, 601)
    s = oracle.silu(z)
    np.testing.assert_allclose(s - oracle.silu(-z), z, rtol=1e-12, atol=1e-12)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-15
    np.testing.assert_allclose(oracle.silu(np.array([1.0])), [1.0 / (1.0 + math.exp(-1.0))])


def _tiny_moe(seed_tag, n_exp=4, D=256, De=256, Ds=256):
    g = synth.rng("pin", "moe", seed_tag)
    ex = {e: tuple(synth.gen_q4_1(g, *shp, zero="normal") for shp in ((De, D), (De, D), (D, De)))
          for e in range(n_exp)}
    sh = tuple(synth.gen_q4_1(g, *shp, zero="normal") for shp in ((Ds, D), (Ds, D), (D, Ds)))

    def W(e):
        G, U, Dn = ex[e]
        return (weights_exact(G, "q4_1", De, D), weights_exact(U, "q4_1", De, D),
                weights_exact(Dn, "q4_1", D, De))
    Wsh = (weights_exact(sh[0], "q4_1", Ds, D), weights_exact(sh[1], "q4_1", Ds, D),
           weights_exact(sh[2], "q4_1", D, Ds))
    return g, W, Wsh


def test_moe_one_hot_routing_is_a_dense_ffn_plus_shared():
    g, W, Wsh = _tiny_moe("onehot")
    X = synth.gen_x(g, 3, 256)
    ids = np.array([[2, 0], [1, 3], [3, 2]], np.int32)
    p = np.array([[1.0, 0.0], [1.0, 0.0], [1.0, 0.0]], np.float32)
    y = oracle.moe_layer_ref(X, ids, p, W, Wsh, n_experts=4)
    xv = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for t in range(3):
        G, U, Dn = W(int(ids[t, 0]))
        g_, u_ = G @ xv[t], U @ xv[t]
        dense = Dn @ (g_ * u_ / (1.0 + np.exp(-g_)))
        gs, us = Wsh[0] @ xv[t], Wsh[1] @ xv[t]
        dense += Wsh[2] @ (gs * us / (1.0 + np.exp(-gs)))
        np.testing.assert_allclose(y[t], dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


def test_moe_stagewise_pieces_compose_to_the_layer():
    g, W, Wsh = _tiny_moe("stage")
    T, k = 4, 3
    X = synth.gen_x(g, T, 256)
    ids = np.array([[0, 1, 2], [3, 3 - 1, 0], [1, 0, 3], [2, 3, 1]], np.int32)
    p = g.random((T, k)).astype(np.float32)
    y = oracle.moe_layer_ref(X, ids, p, W, Wsh, n_experts=4)
    d = np.zeros((T, k, 256))
    ds = np.zeros((T, 256))
    for t in range(T):
        for j in range(k):
            G, U, Dn = W(int(ids[t, j]))
            gg, _ = oracle.gemv_ref(G, X[t:t + 1])
            uu, _ = oracle.gemv_ref(U, X[t:t + 1])
            d[t, j] = Dn @ oracle.swiglu(gg[0], uu[0])
        gg, _ = oracle.gemv_ref(Wsh[0], X[t:t + 1])
        uu, _ = oracle.gemv_ref(Wsh[1], X[t:t + 1])
        ds[t] = Wsh[2] @ oracle.swiglu(gg[0], uu[0])
    yc, _ = oracle.moe_combine_ref(d, p, ds)
    np.testing.assert_allclose(yc, y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_moe_out_of_range_ids_contribute_nothing():
    g, W, Wsh = _tiny_moe("badid")
    X = synth.gen_x(g, 2, 256)
    ids = np.array([[0, 7], [-1, 1]], np.int32)
    p = np.array([[0.5, 0.5], [0.5, 0.5]], np.float32)
    y = oracle.moe_layer_ref(X, ids, p, W, None, n_experts=4)
    ids_ok = np.array([[0, 0], [1, 1]], np.int32)
    p_ok = np.array([[0.5, 0.0], [0.0, 0.5]], np.float32)
    np.testing.assert_allclose(y, oracle.moe_layer_ref(X, ids_ok, p_ok, W, None, n_experts=4),
                               rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------
# router (top-k of the softmax, renormalised)
# ----------------------------------------------------------------------------
def test_router_topk_brute_force_and_invariants():
    """Brute force on a tiny router: every k-subset is scored by its smallest
    logit (then by ids), the best subset must be the oracle's, and the weights
    must be the subset's softmax mass rescaled to one."""
    import itertools
    g = np.random.default_rng(3)
    E, k = 7, 3
    for trial in range(20):
        z = g.integers(-3, 4, E).astype(np.float32) * 0.5     # many ties
        ids, p = oracle.router_topk(z[None, :], k)
        best = None
        for sub in itertools.combinations(range(E), k):
            key = (sorted((-float(z[e]), e) for e in sub))
            if best is None or key < best[0]:
                best = (key, sub)
        want_order = [e for _, e in best[0]]
        assert list(ids[0]) == want_order, (z, ids, want_order)
        ex = [math.exp(float(v) - float(z.max())) for v in z]
        tot = math.fsum(ex)
        mass = [ex[e] / tot for e in want_order]
        assert np.allclose(p[0], np.array(mass) / math.fsum(mass), rtol=1e-14, atol=0)
        ids2, p2 = oracle.router_topk(z[None, :], k, renormalize=False)
        assert list(ids2[0]) == want_order and np.allclose(p2[0], mass, rtol=1e-14, atol=0)
        assert abs(math.fsum(p[0]) - 1.0) < 1e-14


def test_router_logits_one_hot_column():
    """One-hot activation picks one column of the router matrix exactly."""
    g = synth.rng("pin", "router-onehot")
    E, D = 16, 64
    R = synth.bf16_bits(g.standard_normal((E, D)).astype(np.float32))
    X = np.zeros((1, D), dtype=np.uint16)
    X[0, 13] = 0x3F80   # 1.0
    z, a = oracle.router_logits_ref(R, X)
    np.testing.assert_array_equal(z[0], synth.bf16_to_f32(R[:, 13]).astype(np.float64))
    np.testing.assert_array_equal(a[0], np.abs(z[0]))


def test_head_topk_hand_worked_and_brute_force():
    """The head's pick: hand-worked rows with ties, signed zeros and NaNs, then
    brute force (repeated argmax over what is left, a different method) on
    random rows with many repeated values."""
    nan = float("nan")
    y = np.array([[1.0, 3.0, 3.0, -0.0, 0.0, nan, 2.0],
                  [nan, nan, -1.0, nan, -1.0, -2.0, -0.0]], dtype=np.float32)
    ids = oracle.head_topk(y, 5)
    np.testing.assert_array_equal(ids[0], [1, 2, 6, 0, 3])     # 3, 3 (lower index first), 2, 1, then -0 (index 3) ahead of +0
    np.testing.assert_array_equal(ids[1], [6, 2, 4, 5, -1])    # -0, -1, -1, -2, then nothing (NaNs never picked)
    rng = np.random.default_rng(7)
    for trial in range(20):
        M, N, k = 2, int(rng.integers(1, 40)), int(rng.integers(1, 9))
        v = rng.integers(-4, 5, (M, N)).astype(np.float32)
        v[rng.random((M, N)) < 0.1] = np.nan
        got = oracle.head_topk(v, k)
        for m in range(M):
            left = [i for i in range(N) if not np.isnan(v[m, i])]
            want = []
            for _ in range(k):
                if not left:
                    want.append(-1)
                    continue
                best = left[0]
                for i in left[1:]:
                    if v[m, i] > v[m, best]:
                        best = i
                want.append(best)
                left.remove(best)
            np.testing.assert_array_equal(got[m], want)


# ----------------------------------------------------------------------------
# described in-chunk layouts
# ----------------------------------------------------------------------------
def test_layout_hand_worked_block_chunk(golden_dir):
    """A q4_1 chunk in a 20-byte-record layout, weights worked out by hand."""
    import json
    import os
    doc = json.load(open(os.path.join(golden_dir, "layout_blocks_hand.json")))
    ch = np.zeros(5120, np.uint8)
    for off, v in doc["bytes"].items():
        ch[int(off)] = v
    W = oracle.weights_exact_layout(ch, "q4_1", 32, 256, doc["layout"])
    for e in doc["expected"]:
        assert W[e["r"], e["k"]] == e["w"], e


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
def test_layout_default_description_reads_like_the_fixed_decoder(kind):
    g = synth.rng("pin-layout", kind)
    N, K = 64, 512
    ch = synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)
    a = oracle.decode_fields(ch, kind, N, K)
    b = oracle.decode_fields_layout(ch, kind, N, K, oracle.default_layout(kind))
    for name in a:
        np.testing.assert_array_equal(a[name], b[name])


LAYOUTS = {
    "q4_1": {
        "blocks": dict(code_off=4, code_row=160, code_group=20, code_step=1, code_pairing=1, code_high_first=0,
                       f0_off=0, f0_row=160, f0_group=20, f1_off=2, f1_row=160, f1_group=20),
        "columns": dict(code_off=0, code_row=1, code_group=512, code_step=32, code_pairing=0, code_high_first=1,
                        f0_off=4096, f0_row=2, f0_group=64, f1_off=4608, f1_row=2, f1_group=64),
    },
    "q4_k": {
        "blocks": dict(code_off=2, code_row=144, code_group=18, code_step=1, code_pairing=1, code_high_first=0,
                       f0_off=0, f0_row=144, f0_group=18, f1_off=1, f1_row=144, f1_group=18,
                       s_off=4608, s_row=4, m_off=4610, m_row=4),
        "columns": dict(code_off=0, code_row=1, code_group=512, code_step=32, code_pairing=0, code_high_first=1,
                        f0_off=4096, f0_row=1, f0_group=32, f1_off=4352, f1_row=1, f1_group=32,
                        s_off=4608, s_row=2, m_off=4672, m_row=2),
    },
}


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("name", ["blocks", "columns"])
def test_layout_pack_and_decode_round_trip(kind, name):
    """Fields packed by the input generator in a described layout come back from
    the oracle's decode of that layout unchanged (two independent readings of
    the same description), and the weights equal those of the same fields in
    the project's own layout."""
    g = synth.rng("pin-layout-rt", kind, name)
    N, K = 64, 512
    ch = synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)
    f = oracle.decode_fields(ch, kind, N, K)
    L = LAYOUTS[kind][name]
    other = synth.pack_q4_layout(kind, f, L)
    assert not np.array_equal(other, ch)
    back = oracle.decode_fields_layout(other, kind, N, K, L)
    for key in f:
        np.testing.assert_array_equal(back[key], f[key])
    np.testing.assert_array_equal(oracle.weights_exact_layout(other, kind, N, K, L),
                                  oracle.weights_exact(ch, kind, N, K))
