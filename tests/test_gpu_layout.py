"""Chunks in another in-chunk layout (q4nx_chunk_layout, q4nx_relayout).

The NPU engine page ("Q4NX chunks") leaves the byte order inside a q4_1 or
Q4_K chunk to an unpublished header.  A tensor packed in a described layout
(20- or 18-byte records with codes j and j+16 sharing a byte, or a
column-major code plane with high nibbles first and planar metadata) is
converted on the device to the library's layout bit for bit (every byte equal
to the same fields packed in the library's layout), decodes bit-exactly to the
oracle's decode of the described layout, and multiplies within the GEMV bar.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_u8, gemv, have_gpu, host, q, torch, weight
from test_oracle_pins import LAYOUTS

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _fields(kind, N, K, tag):
    g = synth.rng("gpu-layout", tag, kind, N, K)
    ch = synth.gen_q4_1(g, N, K, zero="normal") if kind == "q4_1" else synth.gen_q4_k(g, N, K)
    return oracle.decode_fields(ch, kind, N, K), ch


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
@pytest.mark.parametrize("name", ["blocks", "columns"])
@pytest.mark.parametrize("N,K", [(32, 256), (160, 1280), (4096, 2560)])
def test_relayout_bit_exact_then_decode_and_gemv(kind, name, N, K):
    f, own = _fields(kind, N, K, name)
    Ld = LAYOUTS[kind][name]
    other = synth.pack_q4_layout(kind, f, Ld)
    L = q().chunk_layout(chunk_bytes=oracle.KIND_BYTES[kind], **Ld)
    assert q().chunk_layout_check(L) == 0
    src = dev_u8(other)
    out = torch.zeros(own.size, dtype=torch.uint8, device="cuda")
    q().relayout(L, weight(src, N, K, kind), out)
    np.testing.assert_array_equal(host(out).reshape(own.shape), own)
    # decode of the converted tensor = the oracle's decode of the described layout
    dec = torch.empty((N, K), dtype=torch.float32, device="cuda")
    q().decode(weight(out, N, K, kind), dec)
    W = oracle.weights_exact_layout(other, kind, N, K, Ld)
    np.testing.assert_array_equal(host(dec).view(np.uint32), W.astype(np.float32).view(np.uint32))
    x = synth.gen_x(synth.rng("gpu-layout", "x", name, N, K), 2, K)
    y = gemv(out, N, K, kind, x)
    yr, a = oracle.gemv_ref(W, x)
    assert oracle.tol_ratio(y, yr, a) <= 1.0


def test_relayout_of_the_default_layout_is_a_copy():
    N, K = 96, 768
    for kind in ("q4_1", "q4_k"):
        _, own = _fields(kind, N, K, "default")
        src = dev_u8(own)
        out = torch.zeros(own.size, dtype=torch.uint8, device="cuda")
        q().relayout(q().chunk_layout_default(kind), weight(src, N, K, kind), out)
        np.testing.assert_array_equal(host(out).reshape(own.shape), own)
