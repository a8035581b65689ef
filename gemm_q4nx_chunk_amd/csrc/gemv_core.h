// The dequant-GEMV cores (q4_1 / Q4_K and Q8) shared by the GEMV, plan and MoE kernels.
#pragma once

#include "q4nx_dev.h"

namespace q4nx {

// ===========================================================================
// q4_1 and Q4_K
// ===========================================================================
// Lane l reads, in slice i = 0..3 of a chunk, the 16 bytes at 1024*i + 16*l:
// the 32 codes of tile row r = 8i + l/8 in group g = l%8.  Every slice of every
// chunk gives lane l the same group g, so the lane's 32 activations of a tile
// column are loaded once per chunk.
//
// Unpack: the bf16 with bits 0x4300 | c is exactly 128 + c for a 4-bit c, so
// (w >> 4j) & 0x000F000F | 0x43004300 makes nibbles j and j+4 of a 32-bit code
// word into a bf16 pair, which v_dot2_f32_bf16 multiplies with the pair
// (x[k], x[k+4]).  The same dot chain run with 136 (= 128 + 8) in place of each
// code is subtracted, so with s the scale, z the zero of the 32-column group:
//     sum_k (c s + z) x = s * (D - D136) + (z + 8 s) * sum_k x
// where D - D136 = sum (c - 8) x, bit-exactly 0 when every code is 8 (the
// identical operand bits give identical chain results).  For Q4_K, s = S*scale
// and z = M*min (both products exact in fp32).

// SL slices of a chunk (all 4, or 2 for launches that split a tile's rows
// between workgroups: slices i0 .. i0 + SL - 1 are rows 8 i0 .. 8 (i0 + SL) - 1).
template <int KIND, int SL = 4>
struct Q4Chunk {
  u32x4 q[SL];
  uint32_t meta[SL];   // q4_1: (scale, zero) bf16 pair;  Q4_K: (sc | mn << 8)
  uint32_t rowsm[SL];  // Q4_K: (S, M) bf16 pair of the lane's row
};

template <int KIND>
__device__ __forceinline__ void q4_load(const uint8_t* __restrict__ ck, int lane, Q4Chunk<KIND>& c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) c.q[i] = load_nt16(ck + 1024 * i + 16 * lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // metadata nontemporal too: weights are read once
    if constexpr (KIND == KIND_Q4_1) {
      c.meta[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ck + 4096 + 256 * i + 4 * lane));
      c.rowsm[i] = 0;
    } else {
      c.meta[i] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(ck + 4096 + 128 * i + 2 * lane));
      c.rowsm[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ck + 4608 + 32 * i + 4 * (lane >> 3)));
    }
  }
}

// q4_load through a buffer resource over a run of chunks: off is the chunk's
// byte offset in the run.  Offsets past the run read zero without touching
// memory, so a prefetch past the last chunk needs no branch.
template <int KIND, int SL = 4>
__device__ __forceinline__ void q4_load_rs(__amdgpu_buffer_rsrc_t rs, uint32_t off, int lane,
                                           Q4Chunk<KIND, SL>& c, int i0 = 0) {
  constexpr int kNt = 2;   // nontemporal, codes and metadata alike: weights are read once
#pragma unroll
  for (int i = 0; i < SL; ++i)
    c.q[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024 * (i0 + i) + 16 * lane, 0, kNt));
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const int si = i0 + i;
    if constexpr (KIND == KIND_Q4_1) {
      c.meta[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4096 + 256 * si + 4 * lane, 0, kNt);
      c.rowsm[i] = 0;
    } else {
      c.meta[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 4096 + 128 * si + 2 * lane, 0, kNt);
      c.rowsm[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4608 + 32 * si + 4 * (lane >> 3), 0, kNt);
    }
  }
}

// Q4_K with the metadata fetched whole: the unit's (sc, mn) bytes (128 per
// slice) as one load per lane, 2 SL bytes each, into meta[0..1], and its rows'
// (S, M) pairs into rowsm[0] of lanes 0 .. 8 SL - 1: two small loads per chunk
// instead of 2 SL.  q4k_turn hands each lane its own entries through a
// per-wave LDS slot of 160 SL bytes.
template <int SL>
__device__ __forceinline__ void q4k_load_rs_whole(__amdgpu_buffer_rsrc_t rs, uint32_t off, int lane,
                                                  Q4Chunk<KIND_Q4_K, SL>& c, int i0) {
  constexpr int kNt = 2;
#pragma unroll
  for (int i = 0; i < SL; ++i)
    c.q[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024 * (i0 + i) + 16 * lane, 0, kNt));
  const uint32_t mb = off + 4096 + 128 * i0;
  if constexpr (SL == 4) {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, mb + 8 * lane, 0, kNt));
    c.meta[0] = v.x;
    c.meta[1] = v.y;
  } else if constexpr (SL == 2) {
    c.meta[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, mb + 4 * lane, 0, kNt);
  } else {
    c.meta[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, mb + 2 * lane, 0, kNt);
  }
  c.rowsm[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4608 + 32 * i0 + 4 * (lane & (8 * SL - 1)), 0, kNt);
}

// ts: the wave's slot.  Afterwards c holds, per slice i, the lane's (sc | mn << 8)
// and its row's (S, M), as q4_load_rs leaves them.  The wave's LDS operations
// run in order; the fences keep the compiler from moving them across each other.
template <int SL>
__device__ __forceinline__ void q4k_turn(uint8_t* ts, int lane, Q4Chunk<KIND_Q4_K, SL>& c) {
  if constexpr (SL == 4) *reinterpret_cast<u32x2*>(ts + 8 * lane) = u32x2{c.meta[0], c.meta[1]};
  else if constexpr (SL == 2) *reinterpret_cast<uint32_t*>(ts + 4 * lane) = c.meta[0];
  else *reinterpret_cast<uint16_t*>(ts + 2 * lane) = (uint16_t)c.meta[0];
  if (lane < 8 * SL) *reinterpret_cast<uint32_t*>(ts + 128 * SL + 4 * lane) = c.rowsm[0];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    c.meta[i] = *reinterpret_cast<const uint16_t*>(ts + 128 * i + 2 * lane);
    c.rowsm[i] = *reinterpret_cast<const uint32_t*>(ts + 128 * SL + 32 * i + 4 * (lane >> 3));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // these reads come before
  __builtin_amdgcn_wave_barrier();                          // the next chunk's writes
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Activation pairs (x[k], x[k+4]) of the lane's group for one tile column, in
// the order the code chain uses them, the 136-chain, and sum x taken as that
// chain / 136 (a few fp32 roundings; it is only ever multiplied by z + 8s, and
// it is exact when a single x of the group is nonzero).
template <int M>
struct XPrep {
  uint32_t p[M][16];
  float sum[M];
  float d136[M];
};

// The lane's 32 activations of one tile column, as loaded (bf16 pairs, k order).
template <int M>
struct XRaw {
  u32x4 v[M][4];
};

template <int M>
__device__ __forceinline__ void x_raw(const uint16_t* const (&xrow)[M], int col, XRaw<M>& r) {
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int d = 0; d < 4; ++d) r.v[m][d] = load16(xrow[m] + col + 8 * d);
}

// Coherent variant for activations written by other workgroups of the same
// launch: device-scope (sc1) buffer loads, which read past this XCD's L2.
// xoff[m] is the byte offset of the lane's group in row m; rsrc covers x.
template <int M>
__device__ __forceinline__ void x_raw_coherent(__amdgpu_buffer_rsrc_t rsrc, const int (&xoff)[M],
                                               int col, XRaw<M>& r) {
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int d = 0; d < 4; ++d)
      r.v[m][d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                rsrc, xoff[m] + 2 * (col + 8 * d), 0, kCpolSc1));
}

template <int M>
__device__ __forceinline__ void x_prep_raw(const XRaw<M>& r, XPrep<M>& xp) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4 v = r.v[m][d];   // x[8d .. 8d+7] of the group, bf16 pairs
      // v_perm_b32 byte select: 0..3 pick bytes of the second operand, 4..7 of the first.
      xp.p[m][4 * d + 0] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);   // (x0, x4)
      xp.p[m][4 * d + 1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);   // (x1, x5)
      xp.p[m][4 * d + 2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);   // (x2, x6)
      xp.p[m][4 * d + 3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);   // (x3, x7)
    }
    float e = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) e = dot2bf16(0x43084308u, xp.p[m][t], e);   // (136, 136)
    xp.d136[m] = e;
    xp.sum[m] = e / 136.0f;
  }
}

template <int M>
__device__ __forceinline__ void x_prep(const uint16_t* const (&xrow)[M], int col, XPrep<M>& xp) {
  XRaw<M> r;
  x_raw<M>(xrow, col, r);
  x_prep_raw<M>(r, xp);
}

template <int KIND, int M, int SL = 4>
__device__ __forceinline__ void q4_compute(const Q4Chunk<KIND, SL>& c, const XPrep<M>& xp,
                                           uint32_t kMask, uint32_t kMagic, float (&acc)[SL][M]) {
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    float s, zz;
    if constexpr (KIND == KIND_Q4_1) {
      s = bf16lo(c.meta[i]);
      zz = fmaf(8.f, s, bf16hi(c.meta[i]));
    } else {
      const float S = bf16lo(c.rowsm[i]), Mn = bf16hi(c.rowsm[i]);
      s = S * (float)(c.meta[i] & 0xFFu);
      zz = fmaf(8.f, s, Mn * (float)((c.meta[i] >> 8) & 0xFFu));
    }
    uint32_t cp[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t w = c.q[i][d];
      cp[4 * d + 0] = (w & kMask) | kMagic;
      cp[4 * d + 1] = ((w >> 4) & kMask) | kMagic;
      cp[4 * d + 2] = ((w >> 8) & kMask) | kMagic;
      cp[4 * d + 3] = ((w >> 12) & kMask) | kMagic;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float D = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) D = dot2bf16(cp[t], xp.p[m][t], D);
      acc[i][m] = fmaf(s, D - xp.d136[m], fmaf(zz, xp.sum[m], acc[i][m]));
    }
  }
}

// ===========================================================================
// Q8 (both code layouts)
// ===========================================================================
// A 16-byte piece of Q8 codes is 16 rows of one column in either layout.
// Lane l = 8g + 4h + j takes, in every chunk, the 8 pieces of group g, row half
// h (rows 16h .. 16h+15), columns k = 32g + 8j + i (i = 0..7):
//   layout A (byte k*32 + r):  1024 g + 256 j + 32 i + 16 h
//   layout B ((r/16)*4096 + (k/32)*512 + (k%32)*16 + r%16):  4096 h + 512 g + 128 j + 16 i
// It forms part[rho] = sum_i code(16h+rho, k) * x[k] for its 8 columns, then
// adds d(16h+rho, g) * part[rho]; the 32 lanes of one row half meet at the end.
// Every product of an int8 code and a bf16 is exact in fp32.

template <int KIND>
__device__ __forceinline__ int q8_piece(int lane, int i) {
  const int j = lane & 3, h = (lane >> 2) & 1, g = lane >> 3;
  if constexpr (KIND == KIND_Q8_A) return 1024 * g + 256 * j + 32 * i + 16 * h;
  else return 4096 * h + 512 * g + 128 * j + 16 * i;
}

struct Q8Chunk {
  u32x4 pc[8];     // the lane's 8 pieces: 16 rows x 1 column each
  uint32_t dv[8];  // d(16h + rho, g), two per word
};

__device__ __forceinline__ int q8_dbase(int lane) {
  return 8192 + 256 * ((lane >> 2) & 1) + 2 * (lane >> 3);   // d(16h + rho, g) at dbase + 16*rho
}

template <int KIND>
__device__ __forceinline__ void q8_load(const uint8_t* __restrict__ ck, int lane, Q8Chunk& c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c.pc[i] = load_nt16(ck + q8_piece<KIND>(lane, i));
  const int dbase = q8_dbase(lane);
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const uint32_t lo = *reinterpret_cast<const uint16_t*>(ck + dbase + 32 * rr);
    const uint32_t hi = *reinterpret_cast<const uint16_t*>(ck + dbase + 32 * rr + 16);
    c.dv[rr] = lo | (hi << 16);
  }
}

// q8_load through a buffer resource over a run of chunks (off = the chunk's
// byte offset in the run; past the run every load reads zero, no traffic).
template <int KIND>
__device__ __forceinline__ void q8_load_rs(__amdgpu_buffer_rsrc_t rs, uint32_t off, int lane, Q8Chunk& c) {
  constexpr int kNt = 2;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    c.pc[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + q8_piece<KIND>(lane, i), 0, kNt));
  const uint32_t dbase = off + q8_dbase(lane);
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, dbase + 32 * rr, 0, kNt);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, dbase + 32 * rr + 16, 0, kNt);
    c.dv[rr] = lo | (hi << 16);
  }
}

// The lane's 8 activations of one Q8 chunk (k = 32g + 8j .. +7), as loaded.
template <int M>
struct Q8XRaw {
  u32x4 v[M];
};

__device__ __forceinline__ int q8_xcol(int lane, int c) {
  return 256 * c + 32 * (lane >> 3) + 8 * (lane & 3);
}

// Adds the chunk's products into acc, given the lane's activations.
template <int M>
__device__ __forceinline__ void q8_compute_raw(const Q8Chunk& ch, const Q8XRaw<M>& xr,
                                               float (&acc)[16][M]) {
  float xf[M][8];
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xf[m][2 * t] = bf16lo(xr.v[m][t]);
      xf[m][2 * t + 1] = bf16hi(xr.v[m][t]);
    }
  }
  float part[16][M];
#pragma unroll
  for (int r = 0; r < 16; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) part[r][m] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float cf = (float)(int8_t)(ch.pc[i][r >> 2] >> (8 * (r & 3)));
#pragma unroll
      for (int m = 0; m < M; ++m) part[r][m] = fmaf(cf, xf[m][i], part[r][m]);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float d = (r & 1) ? bf16hi(ch.dv[r >> 1]) : bf16lo(ch.dv[r >> 1]);
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = fmaf(d, part[r][m], acc[r][m]);
  }
}

// Adds chunk (tile column) c of the lane's rows into acc.  x points at
// activation row 0, column 0; ldx is the activation row stride.
template <int M>
__device__ __forceinline__ void q8_compute(const Q8Chunk& ch, const uint16_t* __restrict__ x,
                                           int ldx, int c, int lane, float (&acc)[16][M]) {
  Q8XRaw<M> xr;
#pragma unroll
  for (int m = 0; m < M; ++m) xr.v[m] = load16(x + (size_t)m * ldx + q8_xcol(lane, c));
  q8_compute_raw<M>(ch, xr, acc);
}

// Partial sums of one tile row over chunks [c0, c1): acc[rho][m] of lane l
// belongs to row 16h + rho (h = bit 2 of l), over the lane's 8 columns of each
// chunk; q8_lane_reduce sums the 32 lanes of each row half.
template <int KIND, int M>
__device__ __forceinline__ void q8_row_partial(const uint8_t* __restrict__ row, int c0, int c1,
                                               const uint16_t* __restrict__ x, int ldx, int lane,
                                               float (&acc)[16][M]) {
  constexpr int D = 1;   // a Q8 chunk already holds 40 registers per lane
  const int n = c1 - c0;
  Q8Chunk ring[D];
#pragma unroll
  for (int b = 0; b < D; ++b)
    if (b < n) q8_load<KIND>(row + (size_t)(c0 + b) * 8704, lane, ring[b]);
  for (int i = 0; i < n; i += D) {
#pragma unroll
    for (int b = 0; b < D; ++b) {
      if (i + b < n) {
        q8_compute<M>(ring[b], x, ldx, c0 + i + b, lane, acc);
        if (i + b + D < n) q8_load<KIND>(row + (size_t)(c0 + i + b + D) * 8704, lane, ring[b]);
      }
    }
  }
}

// Sum over the 32 lanes of each row half (lane bits 0, 1, 3, 4, 5).
template <int M>
__device__ __forceinline__ void q8_lane_reduce(float (&acc)[16][M]) {
#pragma unroll
  for (int r = 0; r < 16; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[r][m];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[r][m] = v;
    }
}

// Partial sums of one tile row over chunks [c0, c1) for M activation rows.
// acc[i][m] of lane l belongs to row 8i + l/8, group l%8 (sum over the groups
// with q4_lane_reduce).  xrow[m] points at activation row m, column 0.
template <int KIND, int M>
__device__ __forceinline__ void q4_step(const Q4Chunk<KIND>& ch, const uint16_t* const (&xrow)[M],
                                        int c, uint32_t kMask, uint32_t kMagic, float (&acc)[4][M]) {
  XPrep<M> xp;
  x_prep<M>(xrow, 256 * c, xp);
  q4_compute<KIND, M>(ch, xp, kMask, kMagic, acc);
}

// Chunks kept in flight per wave by q4_row_partial: a ring of this many chunk
// buffers, refilled as each is consumed, so a wave's chunks are not fetched as
// a chain of dependent round trips.
template <int M> struct Q4Depth { static constexpr int value = 2; };

template <int KIND, int M, int D = Q4Depth<M>::value>
__device__ __forceinline__ void q4_row_partial(const uint8_t* __restrict__ row, int c0, int c1,
                                               const uint16_t* const (&xrow_in)[M], int lane,
                                               float (&acc)[4][M]) {
  constexpr int CB = ChunkBytes<KIND>::value;
  const int g = lane & 7;
  const uint16_t* xrow[M];
#pragma unroll
  for (int m = 0; m < M; ++m) xrow[m] = xrow_in[m] + 32 * g;
  // Register operands let the unpack use one v_and_or_b32 (gfx9 VOP3 takes no literal).
  uint32_t kMask = 0x000F000Fu, kMagic = 0x43004300u;
  asm volatile("" : "+s"(kMask));
  asm volatile("" : "+v"(kMagic));
  const int n = c1 - c0;
  Q4Chunk<KIND> ring[D];
#pragma unroll
  for (int b = 0; b < D; ++b)
    if (b < n) q4_load<KIND>(row + (size_t)(c0 + b) * CB, lane, ring[b]);
  for (int i = 0; i < n; i += D) {
#pragma unroll
    for (int b = 0; b < D; ++b) {
      if (i + b < n) {
        q4_step<KIND, M>(ring[b], xrow, c0 + i + b, kMask, kMagic, acc);
        if (i + b + D < n) q4_load<KIND>(row + (size_t)(c0 + i + b + D) * CB, lane, ring[b]);
      }
    }
  }
}

// Sum a lane's partials over the 8 groups; afterwards every lane of the 8
// holds the row sum of rows 8i + lane/8.
template <int M, int SL = 4>
__device__ __forceinline__ void q4_lane_reduce(float (&acc)[SL][M]) {
#pragma unroll
  for (int i = 0; i < SL; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = sum_lanes_xor7(acc[i][m]);
}

}  // namespace q4nx
