"""Seeded synthetic inputs for the Q4NX dequant-GEMV / block-GEMM / MoE path.

This module draws random numbers and lays them out as Q4NX chunk bytes and bf16
activation vectors.  It is the one module that both the CPU oracle's tests and
the GPU path's tests and benchmark take their inputs from.  It computes nothing
that the hot path computes: no code is ever turned back into a weight here, and
no product or sum of weights and activations is formed.

Container facts used here (1bit engine docs, page "NPU engine", section
"Q4NX chunks"): a weight is a grid of 32-row x 256-column tiles, one chunk per
tile, row-major over the grid; the chunk size names the kind (5120 B q4_1,
4736 B Q4_K, 8704 B Q8); the two Q8 code layouts are the byte formulas that
section prints.  Where the page defers to a header that is not published (the
order of codes and metadata inside a q4_1 or Q4_K chunk, and where a Q8 chunk
keeps its scales), this module follows the project's written layout, which is:

  q4_1 (5120 B):  codes  byte r*128 + k//2, low nibble = even k      [0, 4096)
                  (scale, zero) bf16 pair of (r, g) at 4096 + 4*(8r+g) [4096, 5120)
  Q4_K (4736 B):  codes  as q4_1                                     [0, 4096)
                  (sc, mn) u8 pair of (r, g) at 4096 + 2*(8r+g)       [4096, 4608)
                  (S, M) bf16 pair of row r at 4608 + 4*r             [4608, 4736)
  Q8   (8704 B):  int8 code (r, k) at k*32 + r (layout A) or at
                  (r//16)*4096 + (k//32)*512 + (k%32)*16 + r%16 (B)  [0, 8192)
                  d bf16 of (r, g) at 8192 + 2*(8r+g)                 [8192, 8704)

with r the row in the tile (0..31), k the column in the tile (0..255) and
g = k // 32 the 32-column group.  All multi-byte fields are little-endian.

Every draw comes from numpy's PCG64 seeded by a SeedSequence with the fixed
entropy 20261202 and a spawn key naming the tensor (workload, layer, tensor),
so any tensor can be regenerated on its own and is identical on every machine.
"""
from __future__ import annotations

import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED = 20261202

Q4_1_BYTES = 5120
Q4_K_BYTES = 4736
Q8_BYTES = 8704
TILE_ROWS = 32
TILE_COLS = 256


# ----------------------------------------------------------------------------
# seeding
# ----------------------------------------------------------------------------
def _key_part(k) -> int:
    if isinstance(k, (int, np.integer)):
        return int(k)
    return zlib.crc32(str(k).encode("utf-8"))


def rng(*key) -> np.random.Generator:
    """A PCG64 generator for the tensor named by ``key`` (ints or strings)."""
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=tuple(_key_part(k) for k in key))))


# ----------------------------------------------------------------------------
# bf16 rounding of drawn values (input preparation only)
# ----------------------------------------------------------------------------
def bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 with round-to-nearest-even; returns uint16 bits.

    The generator draws no NaN or infinity, so no special case is needed for them.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _abs_normal_bf16(g: np.random.Generator, shape, std: float) -> np.ndarray:
    v = np.abs(g.standard_normal(shape, dtype=np.float32)) * np.float32(std)
    return bf16_bits(v)


def _random_bytes(g: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(g.bytes(n), dtype=np.uint8).reshape(shape)


def _check_shape(N: int, K: int) -> tuple[int, int]:
    if N <= 0 or K <= 0 or N % TILE_ROWS or K % TILE_COLS:
        raise ValueError(f"shape {N}x{K} is not a whole number of 32x256 tiles")
    return N // TILE_ROWS, K // TILE_COLS


# ----------------------------------------------------------------------------
# chunk generators (iid draws written straight into chunk order)
# ----------------------------------------------------------------------------
def gen_q4_1(g: np.random.Generator, N: int, K: int, scale_std: float = 0.02,
             zero: str = "minus8", zero_std: float = 0.1) -> np.ndarray:
    """q4_1 chunks [TR, TC, 5120]: codes uniform 0..15, scale bf16 |N(0, scale_std)|.

    zero="minus8": zero = -8*scale (exact in bf16, the Q4_0 mapping);
    zero="normal": zero = bf16(N(-8*scale, zero_std*scale)).
    """
    TR, TC = _check_shape(N, K)
    out = np.empty((TR, TC, Q4_1_BYTES), dtype=np.uint8)
    out[:, :, :4096] = _random_bytes(g, (TR, TC, 4096))
    s_bits = _abs_normal_bf16(g, (TR, TC, 256), scale_std)
    s = bf16_to_f32(s_bits)
    if zero == "minus8":
        z_bits = bf16_bits(np.float32(-8.0) * s)
    elif zero == "normal":
        n = g.standard_normal((TR, TC, 256), dtype=np.float32)
        z_bits = bf16_bits(s * (np.float32(-8.0) + np.float32(zero_std) * n))
    else:
        raise ValueError(zero)
    meta = np.empty((TR, TC, 256, 2), dtype=np.uint16)
    meta[..., 0] = s_bits
    meta[..., 1] = z_bits
    out[:, :, 4096:] = meta.view(np.uint8).reshape(TR, TC, 1024)
    return out


def gen_q4_k(g: np.random.Generator, N: int, K: int, sm_std: float = 1e-3,
             sc_max: int = 63) -> np.ndarray:
    """Q4_K chunks [TR, TC, 4736]: codes uniform 0..15, sc/mn uniform 0..sc_max,
    S and M bf16 |N(0, sm_std)| per row of each chunk."""
    TR, TC = _check_shape(N, K)
    out = np.empty((TR, TC, Q4_K_BYTES), dtype=np.uint8)
    out[:, :, :4096] = _random_bytes(g, (TR, TC, 4096))
    out[:, :, 4096:4608] = g.integers(0, sc_max + 1, size=(TR, TC, 512), dtype=np.uint8)
    sm = _abs_normal_bf16(g, (TR, TC, 64), sm_std)
    out[:, :, 4608:] = sm.view(np.uint8).reshape(TR, TC, 128)
    return out


def gen_q8(g: np.random.Generator, N: int, K: int, layout: str = "A",
           scale_std: float = 0.02, code_max: int = 127) -> np.ndarray:
    """Q8 chunks [TR, TC, 8704]: int8 codes uniform -code_max..code_max, d bf16 |N(0, scale_std)|.

    The codes are iid, so the draw does not depend on the layout; ``layout`` is
    accepted only so a caller can record which layout the bytes are meant as.
    """
    if layout not in ("A", "B"):
        raise ValueError(layout)
    TR, TC = _check_shape(N, K)
    out = np.empty((TR, TC, Q8_BYTES), dtype=np.uint8)
    out[:, :, :8192] = g.integers(-code_max, code_max + 1, size=(TR, TC, 8192),
                                  dtype=np.int8).view(np.uint8)
    d = _abs_normal_bf16(g, (TR, TC, 256), scale_std)
    out[:, :, 8192:] = d.view(np.uint8).reshape(TR, TC, 512)
    return out


def gen_x(g: np.random.Generator, M: int, K: int, std: float = 1.0) -> np.ndarray:
    """bf16 activations [M, K] drawn from N(0, std), as uint16 bits."""
    return bf16_bits(g.standard_normal((M, K), dtype=np.float32) * np.float32(std))


def gen_gguf(g: np.random.Generator, gtype: int, N: int, K: int, d_std: float = 0.02) -> np.ndarray:
    """A GGUF 4-bit tensor [N, K] as raw bytes (uint8): Q4_0 (type 2, 18-byte
    blocks of 32), Q4_1 (3, 20-byte blocks) or Q4_K (12, 144-byte super-blocks
    of 256), each row K/32 (K/256) consecutive blocks, fields little-endian.
    Codes and Q4_K's packed 6-bit scales are uniform random bytes; the fp16
    fields are drawn: Q4_0 d ~ N(0, d_std); Q4_1 d ~ |N(0, d_std)|, m ~ N(-8 d_std,
    d_std); Q4_K d, dmin ~ |N(0, d_std / 16)|."""
    bb, bc = {2: (18, 32), 3: (20, 32), 12: (144, 256)}[gtype]
    if N <= 0 or K <= 0 or K % bc:
        raise ValueError(f"shape {N}x{K} is not a whole number of GGUF blocks")
    nb = N * (K // bc)
    b = _random_bytes(g, (nb, bb)).copy()

    def put_f16(off, v):
        b[:, off:off + 2] = np.asarray(v, dtype=np.float16).view(np.uint8).reshape(nb, 2)

    if gtype == 2:
        put_f16(0, g.standard_normal(nb) * d_std)
    elif gtype == 3:
        put_f16(0, np.abs(g.standard_normal(nb)) * d_std)
        put_f16(2, g.standard_normal(nb) * d_std - 8 * d_std)
    else:
        put_f16(0, np.abs(g.standard_normal(nb)) * d_std / 16)
        put_f16(2, np.abs(g.standard_normal(nb)) * d_std / 16)
    return b.reshape(-1)


# ----------------------------------------------------------------------------
# packers from logical fields (tests build structured cases with these)
# ----------------------------------------------------------------------------
def _tiles(a: np.ndarray, TR: int, TC: int, per_row: int) -> np.ndarray:
    """[N, TC*per_row] -> [TR, TC, 32, per_row]."""
    return a.reshape(TR, TILE_ROWS, TC, per_row).transpose(0, 2, 1, 3)


def pack_q4_codes(codes: np.ndarray) -> np.ndarray:
    """codes [N, K] in 0..15 -> code region [TR, TC, 4096]."""
    N, K = codes.shape
    TR, TC = _check_shape(N, K)
    c = np.asarray(codes, dtype=np.uint8)
    if c.max(initial=0) > 15:
        raise ValueError("4-bit codes must lie in 0..15")
    b = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)          # [N, K/2]
    return np.ascontiguousarray(_tiles(b, TR, TC, 128)).reshape(TR, TC, 4096)


def pack_q4_1(codes, scale_bits, zero_bits) -> np.ndarray:
    """Logical q4_1 fields -> chunks [TR, TC, 5120].

    codes [N, K] u8 0..15; scale_bits, zero_bits [N, K/32] bf16 bits.
    """
    codes = np.asarray(codes)
    N, K = codes.shape
    TR, TC = _check_shape(N, K)
    out = np.empty((TR, TC, Q4_1_BYTES), dtype=np.uint8)
    out[:, :, :4096] = pack_q4_codes(codes)
    meta = np.empty((TR, TC, 32, 8, 2), dtype=np.uint16)
    meta[..., 0] = _tiles(np.asarray(scale_bits, np.uint16), TR, TC, 8)
    meta[..., 1] = _tiles(np.asarray(zero_bits, np.uint16), TR, TC, 8)
    out[:, :, 4096:] = meta.view(np.uint8).reshape(TR, TC, 1024)
    return out


def pack_q4_k(codes, sc, mn, S_bits, M_bits) -> np.ndarray:
    """Logical Q4_K fields -> chunks [TR, TC, 4736].

    codes [N, K] u8 0..15; sc, mn [N, K/32] u8; S_bits, M_bits [N, K/256] bf16 bits
    (one S and one M per row of each chunk).
    """
    codes = np.asarray(codes)
    N, K = codes.shape
    TR, TC = _check_shape(N, K)
    out = np.empty((TR, TC, Q4_K_BYTES), dtype=np.uint8)
    out[:, :, :4096] = pack_q4_codes(codes)
    scm = np.empty((TR, TC, 32, 8, 2), dtype=np.uint8)
    scm[..., 0] = _tiles(np.asarray(sc, np.uint8), TR, TC, 8)
    scm[..., 1] = _tiles(np.asarray(mn, np.uint8), TR, TC, 8)
    out[:, :, 4096:4608] = scm.reshape(TR, TC, 512)
    sm = np.empty((TR, TC, 32, 2), dtype=np.uint16)
    sm[..., 0] = _tiles(np.asarray(S_bits, np.uint16), TR, TC, 1)[..., 0]
    sm[..., 1] = _tiles(np.asarray(M_bits, np.uint16), TR, TC, 1)[..., 0]
    out[:, :, 4608:] = sm.view(np.uint8).reshape(TR, TC, 128)
    return out


def pack_q4_layout(kind: str, fields: dict, L: dict) -> np.ndarray:
    """Logical q4_1 / Q4_K fields -> chunks [TR, TC, CB] in the described in-chunk
    layout L (the keys of q4nx_chunk_layout; every byte of a chunk must belong
    to exactly one field).  fields: codes [N, K]; q4_1 scale, zero [N, K/32]
    bf16 bits; Q4_K sc, mn [N, K/32] u8, S, M [N, K/256] bf16 bits."""
    codes = np.asarray(fields["codes"], dtype=np.uint8)
    N, K = codes.shape
    TR, TC = _check_shape(N, K)
    CB = Q4_1_BYTES if kind == "q4_1" else Q4_K_BYTES
    out = np.zeros((TR, TC, CB), dtype=np.uint8)
    ct = codes.reshape(TR, 32, TC, 8, 32).transpose(0, 2, 1, 3, 4)        # [TR, TC, r, g, j]
    for r in range(32):
        for g in range(8):
            for j in range(32):
                if L["code_pairing"] == 0:
                    b, nib = j // 2, j % 2
                else:
                    b, nib = j % 16, j // 16
                if L["code_high_first"]:
                    nib = 1 - nib
                off = L["code_off"] + r * L["code_row"] + g * L["code_group"] + b * L["code_step"]
                out[:, :, off] |= (ct[:, :, r, g, j] << (4 * nib)).astype(np.uint8)

    def put16(off, bits):              # bits [TR, TC]
        b = np.asarray(bits, dtype=np.uint16)
        out[:, :, off] = (b & 0xFF).astype(np.uint8)
        out[:, :, off + 1] = (b >> 8).astype(np.uint8)

    names = ("scale", "zero") if kind == "q4_1" else ("sc", "mn")
    per = [np.asarray(fields[n]).reshape(TR, 32, TC, 8).transpose(0, 2, 1, 3) for n in names]
    for r in range(32):
        for g in range(8):
            for fi, name in enumerate(("f0", "f1")):
                off = L[name + "_off"] + r * L[name + "_row"] + g * L[name + "_group"]
                if kind == "q4_1":
                    put16(off, per[fi][:, :, r, g])
                else:
                    out[:, :, off] = per[fi][:, :, r, g].astype(np.uint8)
    if kind == "q4_k":
        for name, key in (("S", "s"), ("M", "m")):
            rows = np.asarray(fields[name]).reshape(TR, 32, TC).transpose(0, 2, 1)
            for r in range(32):
                put16(L[key + "_off"] + r * L[key + "_row"], rows[:, :, r])
    return out


def q8_code_region(tile_codes: np.ndarray, layout: str) -> np.ndarray:
    """Tile codes [..., 32 r, 256 k] int8 -> code region [..., 8192] in the named layout."""
    t = np.asarray(tile_codes)
    lead = t.shape[:-2]
    if layout == "A":          # byte k*32 + r
        reg = np.swapaxes(t, -1, -2)                                  # [..., k, r]
    elif layout == "B":        # byte (r//16)*4096 + (k//32)*512 + (k%32)*16 + r%16
        reg = t.reshape(lead + (2, 16, 8, 32))                         # [.., rh, rl, g, kk]
        reg = np.moveaxis(reg, -3, -1)                                 # [.., rh, g, kk, rl]
    else:
        raise ValueError(layout)
    return np.ascontiguousarray(reg).reshape(lead + (8192,)).view(np.uint8)


def pack_q8(codes, d_bits, layout: str) -> np.ndarray:
    """Logical Q8 fields -> chunks [TR, TC, 8704]; codes [N, K] int8, d_bits [N, K/32]."""
    codes = np.asarray(codes, dtype=np.int8)
    N, K = codes.shape
    TR, TC = _check_shape(N, K)
    out = np.empty((TR, TC, Q8_BYTES), dtype=np.uint8)
    tiles = codes.reshape(TR, 32, TC, 256).transpose(0, 2, 1, 3)      # [TR, TC, 32, 256]
    out[:, :, :8192] = q8_code_region(tiles, layout)
    out[:, :, 8192:] = np.ascontiguousarray(
        _tiles(np.asarray(d_bits, np.uint16), TR, TC, 8)).view(np.uint8).reshape(TR, TC, 512)
    return out


def q8_relayout(chunks: np.ndarray, src: str, dst: str) -> np.ndarray:
    """Re-encode Q8 chunks from one code layout to the other (a byte permutation)."""
    if src == dst:
        return chunks.copy()
    ch = np.asarray(chunks, dtype=np.uint8)
    lead = ch.shape[:-1]
    reg = ch[..., :8192]
    if src == "A":
        tile = np.swapaxes(reg.reshape(lead + (256, 32)), -1, -2)    # [.., r, k]
    elif src == "B":
        t = reg.reshape(lead + (2, 8, 32, 16))                         # [.., rh, g, kk, rl]
        tile = np.moveaxis(t, -1, -3).reshape(lead + (32, 256))       # [.., rh, rl, g, kk]
    else:
        raise ValueError(src)
    out = ch.copy()
    out[..., :8192] = q8_code_region(tile.view(np.int8), dst)
    return out


# ----------------------------------------------------------------------------
# routing inputs for the MoE layer
# ----------------------------------------------------------------------------
def gen_router(g: np.random.Generator, T: int, n_experts: int = 512, k: int = 10,
               zipf_s: float = 1.1, renormalize: bool = True):
    """Top-k expert ids and weights per token, with Zipf(zipf_s) expert popularity.

    Steps: a seeded permutation gives each expert a popularity rank r (1 = most
    popular); logit[t, e] = log(r_e ** -zipf_s) + Gumbel noise; softmax over all
    experts; the k largest probabilities (ties to the lower id); the k weights
    rescaled to sum to one (unless ``renormalize`` is False).
    Returns ids int32 [T, k] and weights float32 [T, k].
    """
    rank = g.permutation(n_experts) + 1
    base = -zipf_s * np.log(rank.astype(np.float64))
    gum = g.gumbel(size=(T, n_experts))
    logit = base[None, :] + gum
    logit -= logit.max(axis=1, keepdims=True)
    prob = np.exp(logit)
    prob /= prob.sum(axis=1, keepdims=True)
    order = np.argsort(-prob, axis=1, kind="stable")[:, :k]
    ids = order.astype(np.int32)
    w = np.take_along_axis(prob, order, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w.astype(np.float32)


# ----------------------------------------------------------------------------
# workload shapes (synthetic stand-ins for the pages' model shapes)
# ----------------------------------------------------------------------------
QWEN3_4B_LAYER = (("q", 4096, 2560), ("k", 1024, 2560), ("v", 1024, 2560),
                  ("o", 2560, 4096), ("gate", 9728, 2560), ("up", 9728, 2560),
                  ("down", 2560, 9728))
QWEN3_4B_LAYERS = 36
QWEN3_4B_LM_HEAD = ("lm_head", 151936, 2560)

DENSE_8B_LAYER = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096),
                  ("o", 4096, 4096), ("gate", 14336, 4096), ("up", 14336, 4096),
                  ("down", 4096, 14336))
DENSE_8B_LAYERS = 32

MOE_D_MODEL = 2048
MOE_EXPERTS = 512
MOE_D_EXPERT = 512
MOE_D_SHARED = 1024
MOE_TOP_K = 10
MOE_LAYERS = 48


@dataclass
class TensorSpec:
    """One weight tensor of a workload: its kind, shape and generator key."""
    name: str
    kind: str            # "q4_1" | "q4_k" | "q8"
    N: int
    K: int
    key: tuple
    q8_layout: str = "A"
    opts: dict = field(default_factory=dict)

    @property
    def nbytes(self) -> int:
        per = {"q4_1": Q4_1_BYTES, "q4_k": Q4_K_BYTES, "q8": Q8_BYTES}[self.kind]
        return (self.N // TILE_ROWS) * (self.K // TILE_COLS) * per

    def generate(self) -> np.ndarray:
        g = rng(*self.key)
        if self.kind == "q4_1":
            return gen_q4_1(g, self.N, self.K, **self.opts)
        if self.kind == "q4_k":
            return gen_q4_k(g, self.N, self.K, **self.opts)
        return gen_q8(g, self.N, self.K, self.q8_layout, **self.opts)


def generate_many(specs, threads: int = 8):
    """Generate several tensors in parallel threads (numpy releases the GIL)."""
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return list(ex.map(lambda s: s.generate(), specs))


def single_gemv_spec() -> TensorSpec:
    """The single q4_1 GEMV workload: 1024x1024, zero = -8*scale."""
    return TensorSpec("w", "q4_1", 1024, 1024, ("q4_1_gemv_1024", 0, "w"),
                      opts={"zero": "minus8"})


def qwen3_4b_decode_specs(layers: int = QWEN3_4B_LAYERS, lm_head: bool = True):
    """All-q4_1 Qwen3-4B-shaped decode step: per-layer projections plus lm_head."""
    specs = []
    for l in range(layers):
        for name, N, K in QWEN3_4B_LAYER:
            specs.append(TensorSpec(f"L{l}.{name}", "q4_1", N, K, ("qwen3_4b_decode", l, name),
                                    opts={"zero": "normal"}))
    if lm_head:
        name, N, K = QWEN3_4B_LM_HEAD
        specs.append(TensorSpec(name, "q4_1", N, K, ("qwen3_4b_decode", 10_000, name),
                                opts={"zero": "normal"}))
    return specs


def mixed_decode_specs(layers: int = QWEN3_4B_LAYERS, q8_layout: str = "A"):
    """Q4_K projections of the Qwen3-4B shapes plus a Q8 tied lm_head 151936x2560."""
    specs = []
    for l in range(layers):
        for name, N, K in QWEN3_4B_LAYER:
            specs.append(TensorSpec(f"L{l}.{name}", "q4_k", N, K, ("mixed_decode", l, name)))
    name, N, K = QWEN3_4B_LM_HEAD
    specs.append(TensorSpec(name, "q8", N, K, ("mixed_decode", 10_000, name), q8_layout=q8_layout))
    return specs


def dense_8b_block_specs(layers: int = DENSE_8B_LAYERS):
    """q4_1 8B-dense projections for the 64-token prompt block GEMM."""
    specs = []
    for l in range(layers):
        for name, N, K in DENSE_8B_LAYER:
            specs.append(TensorSpec(f"L{l}.{name}", "q4_1", N, K, ("dense_8b_block", l, name),
                                    opts={"zero": "normal"}))
    return specs


def moe_expert_spec(layer: int, proj: str, expert: int) -> TensorSpec:
    """One routed expert's projection (gate/up 512x2048, down 2048x512), q4_1."""
    N, K = (MOE_D_EXPERT, MOE_D_MODEL) if proj in ("gate", "up") else (MOE_D_MODEL, MOE_D_EXPERT)
    return TensorSpec(f"L{layer}.{proj}.{expert}", "q4_1", N, K, ("moe_512x10", layer, proj, expert),
                      opts={"zero": "normal"})


def moe_shared_spec(layer: int, proj: str) -> TensorSpec:
    """The shared expert's projection (gate/up 1024x2048, down 2048x1024), q4_1."""
    N, K = (MOE_D_SHARED, MOE_D_MODEL) if proj in ("gate", "up") else (MOE_D_MODEL, MOE_D_SHARED)
    return TensorSpec(f"L{layer}.{proj}.shared", "q4_1", N, K, ("moe_512x10", layer, proj, "shared"),
                      opts={"zero": "normal"})


def moe_router(layer: int, T: int, block: int = 0):
    """Routing inputs of one MoE layer for a batch of T tokens."""
    return gen_router(rng("moe_512x10", layer, "router", T, block), T,
                      MOE_EXPERTS, MOE_TOP_K, 1.1)
