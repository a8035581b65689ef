"""GGUF 4-bit blocks -> q4_1 chunk fields (test infrastructure only).

What it follows:

* the 1bit engine docs, page "NPU engine", section "From a GGUF", its table of
  GGUF types: Q4_0 and Q4_1 map to q4_1 with their codes unchanged (scale d and
  zero -8d, or scale d and zero m), and Q4_K per 32-column sub-block with scale
  d*sc and zero -dmin*mn, a Q4_K super-block being one tile row's 256 columns;
  the only error is rounding scale and zero to bf16;
* the GGUF block types themselves, which that page names but does not lay out;
  they are taken from the public GGUF format (ggml's block_q4_0, block_q4_1 and
  block_q4_K), little-endian:

  ====  ======  ===========================================================
  type  bytes   fields (weights per block)
  ====  ======  ===========================================================
  Q4_0  18      fp16 d, u8 qs[16] (32): weight j < 16 is the low nibble of
                qs[j], weight j + 16 its high nibble; value d * (q - 8)
  Q4_1  20      fp16 d, fp16 m, u8 qs[16] (32): same nibble order;
                value d * q + m
  Q4_K  144     fp16 d, fp16 dmin, u8 scales[12], u8 qs[128] (256): eight
                sub-blocks of 32 with 6-bit (sc, mn) each; sub-block j takes
                the low (j even) or high (j odd) nibbles of qs[32 (j/2) ..
                32 (j/2) + 31]; value d * sc * q - dmin * mn
  ====  ======  ===========================================================

  The 6-bit (sc, mn) of sub-block j sit in scales[12] as follows: for j < 4,
  sc = scales[j] & 63 and mn = scales[j + 4] & 63; for j >= 4, the low four
  bits come from scales[j + 4] (sc the low nibble, mn the high one) and the
  top two bits from the top two bits of scales[j - 4] (sc) and scales[j] (mn).

A tensor of N rows and K columns stores each row as K/32 (Q4_0, Q4_1) or K/256
(Q4_K) consecutive blocks, rows one after another; block b of a row covers
columns 32 b .. 32 b + 31 (256 b .. for Q4_K).

Every product here is exact in float64; the scale and zero are rounded to bf16
once, to nearest even, as the q4_1 fields.  Non-finite fp16 fields are outside
the conversion's domain.
"""
import numpy as np

GGUF_Q4_0, GGUF_Q4_1, GGUF_Q4_K = 2, 3, 12
BLOCK_BYTES = {GGUF_Q4_0: 18, GGUF_Q4_1: 20, GGUF_Q4_K: 144}
BLOCK_COLS = {GGUF_Q4_0: 32, GGUF_Q4_1: 32, GGUF_Q4_K: 256}


def gguf_bytes(gtype: int, N: int, K: int) -> int:
    """Bytes of an N x K tensor of GGUF type ``gtype``."""
    return N * (K // BLOCK_COLS[gtype]) * BLOCK_BYTES[gtype]


def _f16(b: np.ndarray, off: int) -> np.ndarray:
    """The little-endian fp16 at byte ``off`` of every block row of ``b``, as float64."""
    u = b[..., off].astype(np.uint16) | (b[..., off + 1].astype(np.uint16) << 8)
    return u.view(np.float16).astype(np.float64)


def _blocks(src, gtype: int, N: int, K: int) -> np.ndarray:
    """Raw bytes -> [N, blocks per row, block bytes]."""
    b = np.frombuffer(bytes(src) if not isinstance(src, np.ndarray) else src.tobytes(), dtype=np.uint8)
    if b.size != gguf_bytes(gtype, N, K):
        raise ValueError("GGUF tensor has the wrong size")
    return b.reshape(N, K // BLOCK_COLS[gtype], BLOCK_BYTES[gtype])


def _k4_scale_min(sc12: np.ndarray):
    """Q4_K 6-bit (sc, mn) of the eight sub-blocks: [..., 12] bytes -> two [..., 8] arrays."""
    s = sc12.astype(np.int64)
    sc = np.zeros(s.shape[:-1] + (8,), dtype=np.int64)
    mn = np.zeros_like(sc)
    for j in range(8):
        if j < 4:
            sc[..., j] = s[..., j] & 63
            mn[..., j] = s[..., j + 4] & 63
        else:
            sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
            mn[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, mn


def gguf_fields(src, gtype: int, N: int, K: int) -> dict:
    """Per-weight codes [N, K] and per-32-column (a, b) with weight = a * code + b.

    For Q4_0 a = d, b = -8 d; Q4_1 a = d, b = m; Q4_K a = d * sc, b = -dmin * mn
    (all float64, exact).
    """
    blk = _blocks(src, gtype, N, K)
    nb = blk.shape[1]
    if gtype in (GGUF_Q4_0, GGUF_Q4_1):
        qoff = 2 if gtype == GGUF_Q4_0 else 4
        qs = blk[:, :, qoff:qoff + 16]
        codes = np.concatenate([qs & 15, qs >> 4], axis=2)        # weights 0..15, then 16..31
        d = _f16(blk, 0)
        a = d
        b = -8.0 * d if gtype == GGUF_Q4_0 else _f16(blk, 2)
        return {"codes": codes.reshape(N, K).astype(np.int64), "a": a, "b": b}
    if gtype == GGUF_Q4_K:
        d, dmin = _f16(blk, 0), _f16(blk, 2)
        sc, mn = _k4_scale_min(blk[:, :, 4:16])
        qs = blk[:, :, 16:144]
        codes = np.zeros((N, nb, 8, 32), dtype=np.int64)
        for j in range(8):
            q = qs[:, :, 32 * (j // 2):32 * (j // 2) + 32]
            codes[:, :, j, :] = (q >> 4) if j % 2 else (q & 15)
        a = d[:, :, None] * sc
        b = -dmin[:, :, None] * mn
        return {"codes": codes.reshape(N, K), "a": a.reshape(N, nb * 8), "b": b.reshape(N, nb * 8)}
    raise ValueError(f"GGUF type {gtype} is not a 4-bit type this conversion takes")


def gguf_dequant(src, gtype: int, N: int, K: int) -> np.ndarray:
    """The GGUF tensor's weights [N, K] in float64, from its own definition."""
    f = gguf_fields(src, gtype, N, K)
    return np.repeat(f["a"], 32, axis=1) * f["codes"] + np.repeat(f["b"], 32, axis=1)


def _bf16_rne_bits(v: np.ndarray) -> np.ndarray:
    """float64 values that are exact in float32 -> bf16 bits, nearest-even."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(v, dtype=np.float64)):
        raise ValueError("values must be exact in float32")
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def gguf_to_q41(src, gtype: int, N: int, K: int):
    """The q4_1 fields the conversion must produce: codes [N, K] (unchanged) and
    bf16 bits of scale = a and zero = b per (row, 32 columns), [N, K/32] each."""
    f = gguf_fields(src, gtype, N, K)
    return f["codes"], _bf16_rne_bits(f["a"]), _bf16_rne_bits(f["b"])


def gguf_to_q41_bound(src, gtype: int, N: int, K: int) -> np.ndarray:
    """Per-weight bound on |w_q4_1 - w_gguf|: 2^-8 (code |a| + |b|), the effect of
    rounding a and b to bf16 (8 significant bits, nearest)."""
    f = gguf_fields(src, gtype, N, K)
    return 2.0 ** -8 * (f["codes"] * np.repeat(np.abs(f["a"]), 32, axis=1)
                        + np.repeat(np.abs(f["b"]), 32, axis=1))
