"""GPU Q4_K -> q4_1 repack (q4nx_repack_q4k_to_q41) vs the oracle, bit for bit.

The oracle's repack (oracle.repack_q4k_to_q41) is pinned in
test_oracle_pins.py to the rational products S*sc, M*mn rounded to nearest
even; here the device's chunk bytes are decoded back into fields and every
code and every (scale', zero') bit pattern must match.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.decode import decode_fields

from _gpu import dev_u8, have_gpu, host, q, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _repack(ch, N, K):
    w = weight(dev_u8(ch), N, K, "q4_k")
    tiles = (N // 32) * (K // 256)
    out = torch.zeros(tiles * 5120, dtype=torch.uint8, device="cuda")
    q().repack_q4k_to_q41(w, out)
    return host(out).reshape(tiles, 5120)


def _check(ch, N, K):
    got = decode_fields(_repack(ch, N, K), "q4_1", N, K)
    codes, sb, zb = oracle.repack_q4k_to_q41(ch, N, K)
    np.testing.assert_array_equal(got["codes"], codes)
    np.testing.assert_array_equal(got["scale"], sb)
    np.testing.assert_array_equal(got["zero"], zb)


@pytest.mark.parametrize("N,K", [(32, 256), (96, 1280), (2560, 2560)])
def test_repack_matches_oracle(N, K):
    _check(synth.gen_q4_k(synth.rng("gpu-repack", N, K), N, K), N, K)


def test_repack_edge_values():
    """Zero scales and mins, subnormal and large S / M, ties in the rounding."""
    N, K = 64, 512
    g = synth.rng("gpu-repack", "edge")
    ch = synth.gen_q4_k(g, N, K).copy()
    tiles = ch.reshape(-1, 4736)
    sm = tiles[:, 4608:4736].view(np.uint16).reshape(-1, 32, 2)
    # row patterns for S and M: subnormal bf16, smallest normal, 1.0 with a
    # 7-bit mantissa (products need rounding), large but finite under x255
    pats = np.array([0x0001, 0x0080, 0x3FFF, 0x7B00, 0x8001, 0xBF81, 0x0000, 0x4B7F], dtype=np.uint16)
    sm[:, :, 0] = pats[np.arange(32) % 8]
    sm[:, :, 1] = pats[(np.arange(32) + 3) % 8]
    scmn = tiles[:, 4096:4608].reshape(-1, 32, 8, 2)
    scmn[:, ::5, :, 0] = 0
    scmn[:, 1::7, :, 1] = 255
    _check(ch, N, K)
