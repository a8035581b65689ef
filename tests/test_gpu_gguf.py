"""GPU GGUF -> q4_1 conversion (q4nx_gguf_to_q41) vs the oracle, bit for bit.

The oracle's conversion (oracle/gguf.py) is pinned in test_oracle_gguf.py to
hand-worked GGUF blocks and to the exactness and rounding bound of the mapping
table; here the device's chunks are decoded back into fields and every code and
every (scale, zero) bit pattern must match.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.decode import decode_fields, weights_exact

from _gpu import dev_bf16, dev_u8, gemv, have_gpu, host, q, torch

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

TYPES = [oracle.GGUF_Q4_0, oracle.GGUF_Q4_1, oracle.GGUF_Q4_K]


def _convert(src_dev, gtype, N, K):
    tiles = (N // 32) * (K // 256)
    out = torch.zeros(tiles * 5120, dtype=torch.uint8, device="cuda")
    q().gguf_to_q41(gtype, src_dev, N, K, out)
    return out


def _check(got_chunks, src, gtype, N, K):
    got = decode_fields(got_chunks, "q4_1", N, K)
    codes, sb, zb = oracle.gguf_to_q41(src, gtype, N, K)
    np.testing.assert_array_equal(got["codes"], codes)
    np.testing.assert_array_equal(got["scale"], sb)
    np.testing.assert_array_equal(got["zero"], zb)


@pytest.mark.parametrize("gtype", TYPES)
@pytest.mark.parametrize("N,K", [(32, 256), (96, 768), (64, 2560)])
def test_conversion_matches_oracle(gtype, N, K):
    src = synth.gen_gguf(synth.rng("gpu-gguf", gtype, N, K), gtype, N, K)
    out = _convert(dev_u8(src), gtype, N, K)
    _check(host(out).reshape(-1, 5120), src, gtype, N, K)


@pytest.mark.parametrize("gtype", TYPES)
def test_special_fp16_fields(gtype):
    """Zeros of both signs, the smallest and largest subnormals, the largest
    finite values and negative fields; Q4_K with sc, mn at 63."""
    N, K = 32, 512
    src = synth.gen_gguf(synth.rng("gpu-gguf-special", gtype), gtype, N, K).copy()
    bb = oracle.gguf.BLOCK_BYTES[gtype]
    blk = src.reshape(-1, bb)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x7BFF, 0xFBFF, 0x8001, 0x3C00, 0xBC00],
                        dtype=np.uint16)
    nf = 1 if gtype == oracle.GGUF_Q4_0 else 2
    for i in range(blk.shape[0]):
        for f in range(nf):
            v = specials[(i + 3 * f) % len(specials)]
            blk[i, 2 * f], blk[i, 2 * f + 1] = v & 0xFF, v >> 8
    if gtype == oracle.GGUF_Q4_K:
        blk[::2, 4:16] = 0xFF        # every sc and mn 63
    out = _convert(dev_u8(src), gtype, N, K)
    _check(host(out).reshape(-1, 5120), src, gtype, N, K)


@pytest.mark.parametrize("gtype", TYPES)
def test_full_size_8b_gate_up_sampled(gtype):
    """28672 x 4096 (the 8B block's gate|up rows); tile rows sampled, each
    checked against the oracle on the same 32 rows of the GGUF tensor."""
    N, K = 28672, 4096
    src = synth.gen_gguf(synth.rng("gpu-gguf-full", gtype), gtype, N, K)
    out = host(_convert(dev_u8(src), gtype, N, K)).reshape(N // 32, K // 256 * 5120)
    row_bytes = oracle.gguf_bytes(gtype, 1, K)
    for tr in (0, 1, 377, N // 32 - 1):
        band = src[tr * 32 * row_bytes:(tr + 1) * 32 * row_bytes]
        _check(out[tr].reshape(-1, 5120), band, gtype, 32, K)


def test_converted_weight_runs_in_the_gemv():
    """The converted chunks are an ordinary q4_1 weight: the GEMV on them matches
    the oracle's product with the converted weights."""
    gtype, N, K = oracle.GGUF_Q4_K, 512, 2048
    src = synth.gen_gguf(synth.rng("gpu-gguf-gemv"), gtype, N, K)
    out = _convert(dev_u8(src), gtype, N, K)
    x = synth.gen_x(synth.rng("gpu-gguf-gemv", "x"), 2, K)
    y = gemv(out, N, K, "q4_1", x)
    codes, sb, zb = oracle.gguf_to_q41(src, gtype, N, K)
    yr, a = oracle.gemv_ref(weights_exact(synth.pack_q4_1(codes, sb, zb), "q4_1", N, K), x)
    assert oracle.tol_ratio(y, yr, a) <= 1.0
