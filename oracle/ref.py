"""Float64 reference products and checks (test infrastructure only).

* GEMV / block GEMM: y[m, n] = sum_k w[n, k] * x[m, k] with the decoded
  weights (the method reaches exactly this product; see the 1bit engine docs,
  page "NPU engine", section "Q4NX chunks" for the decode, and the Strata
  article, section 1 "Introduction", for why decode is a weight-read-bound
  matrix-vector product).  The error scale is a[m, n] = sum_k |w x|.
* Tolerance: every output finite and |y - y_ref| <= 2e-3 * a, per element.
* MoE layer (Strata article, section 2 "target model", MoE paragraph: 512
  routed experts, the router's top 10, a shared expert every token, then the
  sum): y_t = sum_j p[t,j] * D_e (silu(G_e x) * (U_e x)) + D_s (silu(G_s x) * (U_s x)),
  with silu(z) = z / (1 + exp(-z)).
* Q4_K -> q4_1 repack (NPU engine page, "Q4NX chunks" and "From a GGUF"):
  codes unchanged, scale' = bf16(S * scale), zero' = bf16(M * min), exact apart
  from those two roundings.
"""
from __future__ import annotations

import math

import numpy as np

from .decode import decode_fields

TOL = 2e-3


def _x64(x_bits) -> np.ndarray:
    b = np.asarray(x_bits, dtype=np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def gemv_ref(W64: np.ndarray, x, x_is_bits: bool = True, exact_sum: bool = False):
    """y = X W^T and a = |X| |W|^T in float64.

    W64 [N, K] float64 weights; x [M, K] bf16 bits (or float values when
    ``x_is_bits`` is False).  ``exact_sum`` uses math.fsum per output (tiny sizes).
    """
    X = _x64(x) if x_is_bits else np.asarray(x, dtype=np.float64)
    X = np.atleast_2d(X)
    if exact_sum:
        M, N = X.shape[0], W64.shape[0]
        y = np.empty((M, N))
        a = np.empty((M, N))
        for m in range(M):
            for n in range(N):
                prods = W64[n] * X[m]
                y[m, n] = math.fsum(prods.tolist())
                a[m, n] = math.fsum(np.abs(prods).tolist())
        return y, a
    return X @ W64.T, np.abs(X) @ np.abs(W64).T


def tol_ratio(y, y_ref, a, rel: float = TOL) -> float:
    """max |y - y_ref| / (rel * a) over all outputs (inf when a output is not finite,
    or when a = 0 and y differs from y_ref)."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return math.inf
    err = np.abs(y - y_ref)
    bound = rel * np.asarray(a, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(r.max(initial=0.0))


def check_tol(y, y_ref, a, rel: float = TOL) -> bool:
    return tol_ratio(y, y_ref, a, rel) <= 1.0


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(g, u):
    """h = silu(g) * u, in float64."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def moe_combine_ref(d, p, d_shared=None, a_d=None, a_shared=None):
    """y_t = sum_j p[t,j] d[t,j] (+ d_shared[t]); returns (y, a) with
    a = sum_j |p| a_d (+ a_shared) when the error scales are given."""
    d = np.asarray(d, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    y = np.einsum("tj,tjn->tn", p, d)
    a = None
    if a_d is not None:
        a = np.einsum("tj,tjn->tn", np.abs(p), np.asarray(a_d, dtype=np.float64))
    if d_shared is not None:
        y = y + np.asarray(d_shared, dtype=np.float64)
        if a is not None and a_shared is not None:
            a = a + np.asarray(a_shared, dtype=np.float64)
    return y, a


def moe_layer_ref(X_bits, ids, p, expert_w, shared_w=None, n_experts: int | None = None,
                  with_scale: bool = False):
    """The whole MoE layer in float64.

    X_bits [T, D] bf16 bits; ids [T, k] int; p [T, k] float; expert_w(e) returns
    (G, U, Dn) float64 weights of expert e; shared_w is (G, U, Dn) or None.
    Slots whose id is outside [0, n_experts) contribute nothing.
    Returns y [T, D] float64, and with ``with_scale`` also the layer's error
    scale a = sum_j |p| (|Dn_e| |h_e|) + |Dn_s| |h_s| (the combine's scale with
    each down projection's sum |w h|).
    """
    X = _x64(X_bits)
    T = X.shape[0]
    y = np.zeros((T, X.shape[1]))
    a = np.zeros((T, X.shape[1]))
    cache = {}
    for t in range(T):
        acc = np.zeros(X.shape[1])
        sc = np.zeros(X.shape[1])
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if n_experts is not None and not (0 <= e < n_experts):
                continue
            if e not in cache:
                cache[e] = expert_w(e)
            G, U, Dn = cache[e]
            h = swiglu(G @ X[t], U @ X[t])
            acc += float(p[t, j]) * (Dn @ h)
            sc += abs(float(p[t, j])) * (np.abs(Dn) @ np.abs(h))
        if shared_w is not None:
            G, U, Dn = shared_w
            h = swiglu(G @ X[t], U @ X[t])
            acc += Dn @ h
            sc += np.abs(Dn) @ np.abs(h)
        y[t] = acc
        a[t] = sc
    return (y, a) if with_scale else y


# ----------------------------------------------------------------------------
# Q4_K -> q4_1 repack
# ----------------------------------------------------------------------------
def _f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round values that are exact in float32 to bf16, nearest-even."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(v, dtype=np.float64)):
        raise ValueError("repack inputs must be exact in float32")
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def repack_q4k_to_q41(chunks, N: int, K: int):
    """Q4_K chunks -> logical q4_1 fields (codes, scale bits, zero bits).

    scale' = bf16(S * sc) and zero' = bf16(M * mn) per (row, 32 columns); codes unchanged.
    """
    f = decode_fields(chunks, "q4_k", N, K)
    S = np.repeat(_x64(f["S"]), 8, axis=1)
    M = np.repeat(_x64(f["M"]), 8, axis=1)
    scale = _f64_to_bf16_bits(S * f["sc"].astype(np.float64))
    zero = _f64_to_bf16_bits(M * f["mn"].astype(np.float64))
    return f["codes"], scale, zero


def repack_bound(chunks, N: int, K: int) -> np.ndarray:
    """Per-weight bound on |w_q4_1 - w_q4_k| after the repack:
    2^-8 * (code * |S*sc| + |M*mn|).  A bf16 carries 8 significant bits, so
    rounding to nearest moves a value by at most 2^-8 of its magnitude."""
    f = decode_fields(chunks, "q4_k", N, K)
    S = np.repeat(_x64(f["S"]), 256, axis=1)
    M = np.repeat(_x64(f["M"]), 256, axis=1)
    sc = np.repeat(f["sc"].astype(np.float64), 32, axis=1)
    mn = np.repeat(f["mn"].astype(np.float64), 32, axis=1)
    return 2.0 ** -8 * (f["codes"] * np.abs(S * sc) + np.abs(M * mn))


def router_topk(logits, k: int, renormalize: bool = True):
    """Top-k routing from router logits (Strata article, section 2: the router
    picks 10 of 512 experts per token; the weights are the softmax
    probabilities of the picked experts, rescaled to sum to one unless the
    tail-skip variant of section 4.3 keeps them as they are).

    logits [T, E] (any float dtype; the ranking is taken on these values as
    given).  Returns ids [T, k] int32 in decreasing logit order, the lower id
    first among equal logits, and p [T, k] float64 (softmax in float64).
    """
    L = np.asarray(logits)
    T, E = L.shape
    ids = np.zeros((T, k), dtype=np.int32)
    p = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        row = L[t]
        order = sorted(range(E), key=lambda e: (-float(row[e]), e))[:k]
        ids[t] = order
        z = row.astype(np.float64)
        w = np.exp(z - z.max())
        prob = w / w.sum()
        sel = prob[order]
        p[t] = sel / sel.sum() if renormalize else sel
    return ids, p


def router_logits_ref(R_bits, X_bits):
    """Router logits z[t, e] = sum_d R[e, d] * X[t, d] in float64 from bf16 bits,
    with the error scale a[t, e] = sum_d |R[e, d] X[t, d]|."""
    R = _x64(R_bits)
    X = _x64(X_bits)
    return X @ R.T, np.abs(X) @ np.abs(R).T


def head_topk(y, k: int):
    """The greedy / top-k pick from the lm_head's logits (NPU engine page, "Q4NX
    chunks": the tied Q8 embedding / lm_head; onw technical notes, the host
    work of one step picks the next token from the head's outputs).

    y [M, N] (taken as given, in its own precision).  Returns ids [M, k] int32:
    per row the indices of the k largest values in decreasing order, the lower
    index first among equal values (-0 and +0 are equal); NaNs are never
    picked, and past the last number the ids are -1.
    """
    Y = np.atleast_2d(np.asarray(y))
    M, N = Y.shape
    out = np.full((M, k), -1, dtype=np.int32)
    for m in range(M):
        row = Y[m]
        order = sorted((i for i in range(N) if not math.isnan(float(row[i]))),
                       key=lambda i: (-float(row[i]), i))
        for j, i in enumerate(order[:k]):
            out[m, j] = i
    return out
