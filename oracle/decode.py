"""Q4NX chunk decoding, written from the definition (test infrastructure only).

Source: 1bit engine docs, page "NPU engine", section "Q4NX chunks":

* a weight of N rows (outputs) x K columns (inputs) is a grid of 32x256 tiles,
  one chunk per tile, row-major over the grid: tile (tr, tc) is chunk
  tr * (K/256) + tc;
* the chunk size names the kind: 5120 B q4_1, 4736 B Q4_K, 8704 B Q8;
* q4_1 weight = code * scale + zero, with a bf16 scale and zero per 32 columns
  of a row;
* Q4_K weight = S * scale * code + M * min, with u8 scale and min per 32
  columns and bf16 S, M per row;
* Q8 weight = d * code, with int8 codes and a bf16 scale per 32 columns; code
  (r, k) of a tile sits at byte k*32 + r (layout A) or at
  (r/16)*4096 + (k/32)*512 + (k%32)*16 + r%16 (layout B).

Readings of what that section leaves to a header that is not published (the
project's written layout; parity against real files is unpinned):

* q4_1 / Q4_K codes at byte r*128 + k/2 of the chunk, the even column in the
  low nibble;
* q4_1 (scale, zero) of row r, group g = k/32 at byte 4096 + 4*(8r + g);
* Q4_K (scale, min) u8 pair at 4096 + 2*(8r + g), (S, M) bf16 pair of row r at
  4608 + 4r, one pair per row of each chunk;
* Q8 d of (r, g) at 8192 + 2*(8r + g);
* little-endian fields; int8 codes in two's complement; the Q4_K formula taken
  as printed, with a plus sign on the M * min term.
"""
from __future__ import annotations

import struct

import numpy as np

KIND_BYTES = {"q4_1": 5120, "q4_k": 4736, "q8": 8704}

_R = np.arange(32)
_K = np.arange(256)


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (a bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _grid(chunks: np.ndarray, kind: str, N: int, K: int) -> np.ndarray:
    if N % 32 or K % 256 or N <= 0 or K <= 0:
        raise ValueError("rows must be a multiple of 32 and columns a multiple of 256")
    TR, TC = N // 32, K // 256
    a = np.asarray(chunks, dtype=np.uint8).reshape(-1)
    need = TR * TC * KIND_BYTES[kind]
    if a.size < need:
        raise ValueError("tensor shorter than its layout needs")
    return a[:need].reshape(TR, TC, KIND_BYTES[kind])


def _u16_at(g: np.ndarray, off: np.ndarray) -> np.ndarray:
    """Little-endian u16 read at byte offsets ``off`` of every chunk of grid ``g``."""
    return g[..., off].astype(np.uint16) | (g[..., off + 1].astype(np.uint16) << np.uint16(8))


def _to_matrix(t: np.ndarray) -> np.ndarray:
    """[TR, TC, 32, cols_per_tile] -> [TR*32, TC*cols_per_tile]."""
    TR, TC, R, C = t.shape
    return t.transpose(0, 2, 1, 3).reshape(TR * R, TC * C)


def _q4_codes(g: np.ndarray) -> np.ndarray:
    off = _R[:, None] * 128 + _K[None, :] // 2                        # [32, 256]
    byte = g[..., off]                                                 # [TR, TC, 32, 256]
    shift = (4 * (_K & 1)).astype(np.uint8)[None, None, None, :]
    return _to_matrix((byte >> shift) & np.uint8(15))


def _q8_codes(g: np.ndarray, layout: str) -> np.ndarray:
    r = _R[:, None]
    k = _K[None, :]
    if layout == "A":
        off = k * 32 + r
    elif layout == "B":
        off = (r // 16) * 4096 + (k // 32) * 512 + (k % 32) * 16 + r % 16
    else:
        raise ValueError("Q8 tensors need their code layout, 'A' or 'B'; it cannot be detected")
    return _to_matrix(g[..., off].view(np.int8))


def _per_group(g: np.ndarray, base: int, stride: int, field: int, u16: bool) -> np.ndarray:
    """Field of each (r, g) record at base + stride*(8r + g) + field -> [N, K/32]."""
    rg = (_R[:, None] * 8 + np.arange(8)[None, :]) * stride + base + field   # [32, 8]
    v = _u16_at(g, rg) if u16 else g[..., rg]
    return _to_matrix(v)


def decode_fields(chunks, kind: str, N: int, K: int, q8_layout: str | None = None) -> dict:
    """Chunk bytes -> logical fields of an N x K weight.

    q4_1: codes [N, K] u8, scale, zero [N, K/32] bf16 bits
    q4_k: codes [N, K] u8, sc, mn [N, K/32] u8, S, M [N, K/256] bf16 bits
    q8:   codes [N, K] int8, d [N, K/32] bf16 bits
    """
    if kind not in KIND_BYTES:
        raise ValueError(f"unknown chunk kind {kind!r}")
    g = _grid(chunks, kind, N, K)
    if kind == "q4_1":
        return {"codes": _q4_codes(g),
                "scale": _per_group(g, 4096, 4, 0, True),
                "zero": _per_group(g, 4096, 4, 2, True)}
    if kind == "q4_k":
        row = _R * 4 + 4608
        return {"codes": _q4_codes(g),
                "sc": _per_group(g, 4096, 2, 0, False),
                "mn": _per_group(g, 4096, 2, 1, False),
                "S": _to_matrix(_u16_at(g, row)[..., None]),
                "M": _to_matrix(_u16_at(g, row + 2)[..., None])}
    return {"codes": _q8_codes(g, q8_layout), "d": _per_group(g, 8192, 2, 0, True)}


def _expand(per_group: np.ndarray, width: int) -> np.ndarray:
    return np.repeat(per_group, width, axis=1)


def weights_exact(chunks, kind: str, N: int, K: int, q8_layout: str | None = None) -> np.ndarray:
    """Decoded weights [N, K] as float64.

    Every term is exact in float64 (a 4-bit code times a bf16 has 12 significant
    bits, S*scale*code 20 bits, M*min and d*code 16 bits), and the one addition
    of q4_1 and Q4_K is rounded once, which makes the float32 rounding of these
    values equal to the float32 rounding of the exact result (53 >= 2*24 + 2).
    """
    f = decode_fields(chunks, kind, N, K, q8_layout)
    c = f["codes"].astype(np.float64)
    if kind == "q4_1":
        s = _expand(_bf16_to_f64(f["scale"]), 32)
        z = _expand(_bf16_to_f64(f["zero"]), 32)
        return c * s + z
    if kind == "q4_k":
        S = _expand(_bf16_to_f64(f["S"]), 256)
        M = _expand(_bf16_to_f64(f["M"]), 256)
        sc = _expand(f["sc"].astype(np.float64), 32)
        mn = _expand(f["mn"].astype(np.float64), 32)
        return (S * sc) * c + M * mn
    d = _expand(_bf16_to_f64(f["d"]), 32)
    return d * c


def weights_f32(chunks, kind: str, N: int, K: int, q8_layout: str | None = None) -> np.ndarray:
    """Decoded weights rounded once to float32: the bit-exact expectation of a decode."""
    return weights_exact(chunks, kind, N, K, q8_layout).astype(np.float32)


def unpack_expected(chunks, kind: str, N: int, K: int, q8_layout: str | None = None) -> dict:
    """Fields in the form the library's unpack call writes them.

    codes [N, K] u8 (Q8: the int8 bit pattern); meta0 [N, K/32] u16 (scale | sc | d);
    meta1 [N, K/32] u16 (zero | mn; zeros for Q8); row_meta [N, K/256, 2] u16
    ((S, M) for Q4_K; zeros otherwise).
    """
    f = decode_fields(chunks, kind, N, K, q8_layout)
    G, C = K // 32, K // 256
    out = {"codes": f["codes"].view(np.uint8) if kind == "q8" else f["codes"],
           "meta1": np.zeros((N, G), np.uint16), "row_meta": np.zeros((N, C, 2), np.uint16)}
    if kind == "q4_1":
        out["meta0"], out["meta1"] = f["scale"], f["zero"]
    elif kind == "q4_k":
        out["meta0"], out["meta1"] = f["sc"].astype(np.uint16), f["mn"].astype(np.uint16)
        out["row_meta"][..., 0], out["row_meta"][..., 1] = f["S"], f["M"]
    else:
        out["meta0"] = f["d"]
    return out


# ----------------------------------------------------------------------------
# brute force: one chunk, one weight at a time, in plain Python
# ----------------------------------------------------------------------------
def _bf16(b: bytes, off: int) -> float:
    return struct.unpack("<f", b"\x00\x00" + b[off:off + 2])[0]


def scalar_decode_chunk(chunk: bytes, kind: str, q8_layout: str | None = None):
    """Decode one chunk into a 32 x 256 list of Python floats (float64 arithmetic).

    Written per weight, straight from the formulas, for cross-checking the
    vectorised decoder on tiny grids.
    """
    b = bytes(chunk)
    if len(b) != KIND_BYTES[kind]:
        raise ValueError("chunk size does not match its kind")
    out = [[0.0] * 256 for _ in range(32)]
    for r in range(32):
        for k in range(256):
            grp = k // 32
            if kind in ("q4_1", "q4_k"):
                byte = b[r * 128 + k // 2]
                code = (byte >> 4) if (k % 2) else (byte & 0x0F)
                if kind == "q4_1":
                    rec = 4096 + 4 * (8 * r + grp)
                    out[r][k] = code * _bf16(b, rec) + _bf16(b, rec + 2)
                else:
                    rec = 4096 + 2 * (8 * r + grp)
                    sc, mn = b[rec], b[rec + 1]
                    S, M = _bf16(b, 4608 + 4 * r), _bf16(b, 4608 + 4 * r + 2)
                    out[r][k] = S * sc * code + M * mn
            else:
                if q8_layout == "A":
                    pos = k * 32 + r
                elif q8_layout == "B":
                    pos = (r // 16) * 4096 + (k // 32) * 512 + (k % 32) * 16 + r % 16
                else:
                    raise ValueError("Q8 layout required")
                code = struct.unpack("<b", b[pos:pos + 1])[0]
                out[r][k] = _bf16(b, 8192 + 2 * (8 * r + grp)) * code
    return out


# ----------------------------------------------------------------------------
# other in-chunk layouts (q4_1 / Q4_K): the byte order inside a chunk is left
# by the NPU engine page ("Q4NX chunks") to an unpublished header, so a layout
# is described field by field (the same description as q4nx_chunk_layout):
#   code (r, g, j): byte code_off + r*code_row + g*code_group + b*code_step,
#     b = j//2 and nibble j%2 (code_pairing 0) or b = j%16 and nibble j//16
#     (code_pairing 1); nibble 0 is the low one unless code_high_first;
#   per (r, g): field 0 / field 1 at f*_off + r*f*_row + g*f*_group
#     (q4_1: bf16 scale / zero; Q4_K: u8 scale / min);
#   per row (Q4_K): bf16 S at s_off + r*s_row, bf16 M at m_off + r*m_row.
# ----------------------------------------------------------------------------
def default_layout(kind: str) -> dict:
    """The project's own layout (the one decode_fields reads) as a description."""
    L = {"code_off": 0, "code_row": 128, "code_group": 16, "code_step": 1, "code_pairing": 0,
         "code_high_first": 0}
    if kind == "q4_1":
        L.update(f0_off=4096, f0_row=32, f0_group=4, f1_off=4098, f1_row=32, f1_group=4)
    elif kind == "q4_k":
        L.update(f0_off=4096, f0_row=16, f0_group=2, f1_off=4097, f1_row=16, f1_group=2,
                 s_off=4608, s_row=4, m_off=4610, m_row=4)
    else:
        raise ValueError("layouts describe q4_1 and Q4_K chunks")
    return L


def decode_fields_layout(chunks, kind: str, N: int, K: int, L: dict) -> dict:
    """decode_fields for chunks stored in the described layout L."""
    if kind not in ("q4_1", "q4_k"):
        raise ValueError("layouts describe q4_1 and Q4_K chunks")
    g = _grid(chunks, kind, N, K)
    r = _R[:, None, None]
    gg = np.arange(8)[None, :, None]
    j = np.arange(32)[None, None, :]
    if L["code_pairing"] == 0:
        b, nib = j // 2, j % 2
    else:
        b, nib = j % 16, j // 16
    if L["code_high_first"]:
        nib = 1 - nib
    off = L["code_off"] + r * L["code_row"] + gg * L["code_group"] + b * L["code_step"]   # [32, 8, 32]
    byte = g[..., off.reshape(32, 256)]                                                  # [TR, TC, 32, 256]
    shift = (4 * np.broadcast_to(nib, (32, 8, 32))).reshape(32, 256).astype(np.uint8)
    codes = _to_matrix((byte >> shift) & np.uint8(15))
    rg0 = L["f0_off"] + _R[:, None] * L["f0_row"] + np.arange(8)[None, :] * L["f0_group"]
    rg1 = L["f1_off"] + _R[:, None] * L["f1_row"] + np.arange(8)[None, :] * L["f1_group"]
    if kind == "q4_1":
        return {"codes": codes, "scale": _to_matrix(_u16_at(g, rg0)), "zero": _to_matrix(_u16_at(g, rg1))}
    srow = L["s_off"] + _R * L["s_row"]
    mrow = L["m_off"] + _R * L["m_row"]
    return {"codes": codes, "sc": _to_matrix(g[..., rg0]), "mn": _to_matrix(g[..., rg1]),
            "S": _to_matrix(_u16_at(g, srow)[..., None]), "M": _to_matrix(_u16_at(g, mrow)[..., None])}


def weights_exact_layout(chunks, kind: str, N: int, K: int, L: dict) -> np.ndarray:
    """weights_exact for chunks stored in the described layout L (same formulas)."""
    f = decode_fields_layout(chunks, kind, N, K, L)
    c = f["codes"].astype(np.float64)
    if kind == "q4_1":
        return c * _expand(_bf16_to_f64(f["scale"]), 32) + _expand(_bf16_to_f64(f["zero"]), 32)
    S = _expand(_bf16_to_f64(f["S"]), 256)
    M = _expand(_bf16_to_f64(f["M"]), 256)
    return (S * _expand(f["sc"].astype(np.float64), 32)) * c + M * _expand(f["mn"].astype(np.float64), 32)
