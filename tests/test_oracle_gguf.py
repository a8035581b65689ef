"""Pins of the oracle's GGUF -> q4_1 conversion (oracle/gguf.py).

The GGUF block layouts are pinned by blocks worked by hand (byte values chosen
here, weights computed by hand and written as literals), the conversion by the
mapping table of the 1bit engine docs (page "NPU engine", section "From a
GGUF"): codes unchanged, scale and zero rounded to bf16 as the only error, so
the result is exact whenever d, m (or d*sc, dmin*mn) are bf16 values, and
within the bf16 rounding bound otherwise.  The q4_1 side is read back through
the chunk decoder, which has pins of its own.
"""
import struct

import numpy as np
import pytest

import oracle
import synth
from oracle.decode import weights_exact

Q40, Q41, Q4K = oracle.GGUF_Q4_0, oracle.GGUF_Q4_1, oracle.GGUF_Q4_K


def _h(v: float) -> bytes:
    return struct.pack("<e", v)


def test_q4_0_block_worked_by_hand():
    # d = 0.5; byte j holds code j in its low nibble and 15 - j in its high one
    blk = _h(0.5) + bytes(j | ((15 - j) << 4) for j in range(16))
    w = oracle.gguf_dequant(blk, Q40, 1, 32)[0]
    assert w[0] == -4.0 and w[1] == -3.5 and w[8] == 0.0 and w[15] == 3.5   # low nibbles first
    assert w[16] == 3.5 and w[23] == 0.0 and w[31] == -4.0                  # then the high ones


def test_q4_1_block_worked_by_hand():
    blk = _h(0.25) + _h(-1.0) + bytes([0xA3] + [0x00] * 14 + [0xF1])
    w = oracle.gguf_dequant(blk, Q41, 1, 32)[0]
    assert w[0] == -0.25 and w[16] == 1.5          # 0.25 * 3 - 1 and 0.25 * 10 - 1
    assert w[1] == -1.0 and w[17] == -1.0
    assert w[15] == -0.75 and w[31] == 2.75        # codes 1 and 15


# (sc, mn) of the eight sub-blocks and their 12-byte packing, worked by hand
_SC = [1, 2, 3, 4, 33, 50, 63, 17]
_MN = [5, 6, 7, 8, 40, 20, 0, 63]
_SCALES12 = bytes([0x81, 0xC2, 0xC3, 0x44, 0x85, 0x46, 0x07, 0xC8, 0x81, 0x42, 0x0F, 0xF1])


def _q4k_block(d=1.0, dmin=0.5):
    # qs[32 p + t]: low nibble t & 15, high nibble (t + p) & 15
    qs = bytes((t & 15) | (((t + p) & 15) << 4) for p in range(4) for t in range(32))
    return _h(d) + _h(dmin) + _SCALES12 + qs


def test_q4_k_six_bit_scales_worked_by_hand():
    f = oracle.gguf_fields(_q4k_block(), Q4K, 1, 256)
    assert f["a"][0].tolist() == [float(s) for s in _SC]               # d = 1
    assert f["b"][0].tolist() == [-0.5 * m for m in _MN]               # dmin = 0.5


def test_q4_k_sub_block_nibbles_worked_by_hand():
    w = oracle.gguf_dequant(_q4k_block(), Q4K, 1, 256)[0]
    assert w[32 * 0 + 3] == 0.5       # sub-block 0, low nibble 3:  1 * 3 - 0.5 * 5
    assert w[32 * 1 + 3] == 3.0       # sub-block 1, high nibble 3: 2 * 3 - 0.5 * 6
    assert w[32 * 6 + 20] == 252.0    # sub-block 6, low nibble 4:  63 * 4 - 0
    assert w[32 * 7 + 20] == 87.5     # sub-block 7, high nibble 7: 17 * 7 - 0.5 * 63
    assert w[32 * 4 + 31] == 475.0    # sub-block 4, low nibble 15: 33 * 15 - 0.5 * 40


@pytest.mark.parametrize("gtype", [Q40, Q41, Q4K])
def test_one_block_lands_in_its_row_and_columns(gtype):
    """Brute force over the tensor's block order: one nonzero block at a time."""
    N, K = 3, 512
    bb, bc = oracle.gguf.BLOCK_BYTES[gtype], oracle.gguf.BLOCK_COLS[gtype]
    one = {Q40: _h(1.0) + bytes([0x99] * 16), Q41: _h(1.0) + _h(0.0) + bytes([0x11] * 16),
           Q4K: _h(1.0) + _h(0.0) + bytes([1] * 4 + [0] * 8) + bytes([0x11] * 128)}[gtype]
    for r in range(N):
        for b in range(K // bc):
            src = bytearray(oracle.gguf_bytes(gtype, N, K))
            for i in range(N * (K // bc)):      # every other block: fp16 fields 0, so all weights 0
                src[i * bb:(i + 1) * bb] = bytes(bb)
            off = (r * (K // bc) + b) * bb
            src[off:off + bb] = one
            w = oracle.gguf_dequant(bytes(src), gtype, N, K)
            nz = np.argwhere(w != 0)
            want_cols = np.arange(bc * b, bc * b + (bc if gtype != Q4K else 128))
            assert set(nz[:, 0]) == {r}
            assert np.array_equal(np.unique(nz[:, 1]), want_cols), (r, b)


def _q41_weights(codes, sb, zb, N, K):
    return weights_exact(synth.pack_q4_1(codes, sb, zb), "q4_1", N, K)


@pytest.mark.parametrize("gtype", [Q40, Q41, Q4K])
def test_conversion_within_the_bf16_bound(gtype):
    N, K = 64, 768
    src = synth.gen_gguf(synth.rng("pin", "gguf", gtype), gtype, N, K)
    codes, sb, zb = oracle.gguf_to_q41(src, gtype, N, K)
    diff = np.abs(_q41_weights(codes, sb, zb, N, K) - oracle.gguf_dequant(src, gtype, N, K))
    assert np.all(diff <= oracle.gguf_to_q41_bound(src, gtype, N, K))
    assert diff.max() > 0            # fp16 fields carry more bits than a bf16


@pytest.mark.parametrize("gtype", [Q40, Q41, Q4K])
def test_conversion_exact_on_bf16_fields(gtype):
    """fp16 fields with at most 8 significant bits (and, for Q4_K, every sc and
    mn 0 or 2, so d * sc and dmin * mn keep 8): the q4_1 weights equal the GGUF ones."""
    N, K = 32, 512
    src = synth.gen_gguf(synth.rng("pin", "gguf-exact", gtype), gtype, N, K).copy()
    bb = oracle.gguf.BLOCK_BYTES[gtype]
    blk = src.reshape(-1, bb)
    nf = 1 if gtype == Q40 else 2
    for i in range(nf):          # clear the low 3 mantissa bits of each fp16 field
        u = blk[:, 2 * i].astype(np.uint16) | (blk[:, 2 * i + 1].astype(np.uint16) << 8)
        u &= np.uint16(0xFFF8)
        blk[:, 2 * i] = (u & 0xFF).astype(np.uint8)
        blk[:, 2 * i + 1] = (u >> 8).astype(np.uint8)
    if gtype == Q4K:             # every sc, mn 0 or 2: d * sc keeps 8 significant bits
        blk[:, 4:16] &= np.uint8(0x02)
    codes, sb, zb = oracle.gguf_to_q41(src, gtype, N, K)
    assert np.array_equal(_q41_weights(codes, sb, zb, N, K), oracle.gguf_dequant(src, gtype, N, K))


def test_q4_0_zero_is_minus_eight_scale():
    """Q4_0's zero -8 d is the scale with its sign flipped and exponent + 3, bit for bit."""
    N, K = 32, 256
    src = synth.gen_gguf(synth.rng("pin", "gguf-q40"), Q40, N, K)
    _, sb, zb = oracle.gguf_to_q41(src, Q40, N, K)
    normal = ((sb & 0x7F80) != 0) & ((sb & 0x7F80) < (0xFF - 3) << 7)
    assert normal.mean() > 0.99
    assert np.array_equal(zb[normal], (sb[normal] ^ 0x8000) + (3 << 7))
