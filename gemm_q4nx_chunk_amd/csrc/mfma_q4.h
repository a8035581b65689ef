// Dequantising bf16 matrix-core tiles of Q4NX chunks (gfx950), shared by the
// block GEMM and the MoE kernels for experts with many tokens.
//
// Dequantisation: a 4-bit code c placed in an fp16 mantissa under the exponent
// of 1024 reads as 1024 + c (low nibble) or 1024 + 16c (high nibble of a
// byte), both exact, so one v_and_or makes two weights' codes into an fp16
// pair; one v_pk_add_f16 of -1024 (or one v_pk_fma_f16 by 1/16 with -64) turns
// the pair into the exact codes (c, c'), and one v_fma_mix_f32 per weight forms
// w = c * s + z in fp32: the exact value rounded once, which is the decoded
// weight bit for bit.  v_cvt_pk_bf16_f32 then rounds two weights to the bf16
// pair the MFMA takes (at most 2^-8 of the weight's size).
//
// k-slot assignment: in MFMA step s (16 per tile column) lane (h = lane/32,
// n = lane%32) feeds the 8 products k = 128h + 8s + 0..7 -- for the B operand
// (weights) of output row n, for the A operand (X) of token row n.  A and B
// use the same slots, so the order of k inside a step does not change the sum.
// With this order a lane's weights are one contiguous 64-byte run of its row's
// codes, and their scale records one 16-byte load.
#pragma once

#include "q4nx_dev.h"

namespace q4nx {

constexpr int kXs = 264;   // LDS row stride of an X tile in bf16 (256 + 8: 4-bank skew per row)

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int KIND>
struct GemmChunk {
  u32x4 q[4];   // codes k = 128h + 32q + 0..31 of row n
  u32x4 meta;   // q4_1: (scale, zero) of groups 4h..4h+3; Q4_K: .x,.y = (sc,mn) bytes, .z = (S, M)
};

// Chunk of tile column t of the lane's row: rs covers the row's chunks of this
// workgroup's K part, off = (t - first tile column) * chunk bytes.  Offsets past
// the part read as zero without touching memory, so the prefetch past the last
// tile column needs no branch.
template <int KIND>
__device__ __forceinline__ void gemm_load(__amdgpu_buffer_rsrc_t rs, uint32_t off, int n, int h,
                                          GemmChunk<KIND>& c) {
  constexpr int kNt = 2;   // nontemporal: weights are read once
#pragma unroll
  for (int q = 0; q < 4; ++q)
    c.q[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, off + 128 * n + 64 * h + 16 * q, 0, kNt));
  if constexpr (KIND == KIND_Q4_1) {
    c.meta = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 4096 + 32 * n + 16 * h, 0, kNt));
  } else {
    const u32x2 scmn = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 4096 + 16 * n + 8 * h, 0, kNt));
    c.meta.x = scmn.x;
    c.meta.y = scmn.y;
    c.meta.z = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4608 + 4 * n, 0, kNt);
    c.meta.w = 0;
  }
}

// Scale and offset of group q (0..3) of the lane: w = code * s + z.
template <int KIND>
__device__ __forceinline__ void group_sz(const GemmChunk<KIND>& c, int q, float& s, float& z) {
  if constexpr (KIND == KIND_Q4_1) {
    s = bf16lo(c.meta[q]);
    z = bf16hi(c.meta[q]);
  } else {
    const uint32_t pair = (q < 2 ? c.meta.x : c.meta.y) >> (16 * (q & 1));
    s = bf16lo(c.meta.z) * (float)(pair & 0xFFu);
    z = bf16hi(c.meta.z) * (float)((pair >> 8) & 0xFFu);
  }
}

// Eight weights of one code word (k = 0..7, even k in the low nibble) as bf16.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s, float z, uint32_t kMaskLo,
                                           uint32_t kMaskHi, uint32_t kMagic) {
  const f16x2 m1024 = {(_Float16)-1024.f, (_Float16)-1024.f};
  const f16x2 m64 = {(_Float16)-64.f, (_Float16)-64.f};
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const f16x2 p0 = __builtin_bit_cast(f16x2, (w & kMaskLo) | kMagic) + m1024;    // (c0, c4)
  const f16x2 p1 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w & kMaskHi) | kMagic), sixteenth, m64);    // (c1, c5)
  const f16x2 p2 = __builtin_bit_cast(f16x2, (w8 & kMaskLo) | kMagic) + m1024;   // (c2, c6)
  const f16x2 p3 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w8 & kMaskHi) | kMagic), sixteenth, m64);   // (c3, c7)
  bf16x8 b;
  b[0] = (__bf16)fmaf((float)p0.x, s, z);
  b[1] = (__bf16)fmaf((float)p1.x, s, z);
  b[2] = (__bf16)fmaf((float)p2.x, s, z);
  b[3] = (__bf16)fmaf((float)p3.x, s, z);
  b[4] = (__bf16)fmaf((float)p0.y, s, z);
  b[5] = (__bf16)fmaf((float)p1.y, s, z);
  b[6] = (__bf16)fmaf((float)p2.y, s, z);
  b[7] = (__bf16)fmaf((float)p3.y, s, z);
  return b;
}

// acc0 (token rows 0..31) and acc1 (rows 32..63) += one X tile times the
// chunk's weights, over the 16 MFMA steps of a tile column.  The lane's
// operands of MFMA step s are at xb + 8 s (rows n, k slots as above) and
// xb + off1 + 8 s (rows n + 32).  Software pipelined: the weights of step
// s + 1 are dequantised and its X operands read while the two products of
// step s run, in the order the group barriers fix (reads, VALU, product,
// VALU, product).
template <int KIND>
__device__ __forceinline__ void mfma_tile(const GemmChunk<KIND>& c, const uint16_t* xb, int off1,
                                          f32x16& acc0, f32x16& acc1, uint32_t kMaskLo,
                                          uint32_t kMaskHi, uint32_t kMagic) {
  float s, z;
  group_sz<KIND>(c, 0, s, z);
  bf16x8 B = dequant8(c.q[0][0], s, z, kMaskLo, kMaskHi, kMagic);
  bf16x8 A0 = *reinterpret_cast<const bf16x8*>(xb);
  bf16x8 A1 = *reinterpret_cast<const bf16x8*>(xb + off1);
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    bf16x8 Bn = B, A0n = A0, A1n = A1;
    if (st < 15) {
      const int sn = st + 1;
      if ((sn & 3) == 0) group_sz<KIND>(c, sn >> 2, s, z);
      Bn = dequant8(c.q[sn >> 2][sn & 3], s, z, kMaskLo, kMaskHi, kMagic);
      A0n = *reinterpret_cast<const bf16x8*>(xb + 8 * sn);
      A1n = *reinterpret_cast<const bf16x8*>(xb + off1 + 8 * sn);
    }
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B, acc1, 0, 0, 0);
    B = Bn;
    A0 = A0n;
    A1 = A1n;
    if (st < 15) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);    // DS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);    // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 14, 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
    }
  }
}

// Eight weights as two bf16 parts, hi = bf16(w) and lo = bf16(w - hi), which
// carry each weight to 2^-16 of its size (hi is within 2^-8 of w, lo within
// 2^-8 of w - hi).
__device__ __forceinline__ void dequant8_hl(uint32_t w, float s, float z, uint32_t kMaskLo, uint32_t kMaskHi,
                                            uint32_t kMagic, bf16x8& hi, bf16x8& lo) {
  const f16x2 m1024 = {(_Float16)-1024.f, (_Float16)-1024.f};
  const f16x2 m64 = {(_Float16)-64.f, (_Float16)-64.f};
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const f16x2 p0 = __builtin_bit_cast(f16x2, (w & kMaskLo) | kMagic) + m1024;
  const f16x2 p1 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w & kMaskHi) | kMagic), sixteenth, m64);
  const f16x2 p2 = __builtin_bit_cast(f16x2, (w8 & kMaskLo) | kMagic) + m1024;
  const f16x2 p3 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w8 & kMaskHi) | kMagic), sixteenth, m64);
  float f[8];
  f[0] = fmaf((float)p0.x, s, z);
  f[1] = fmaf((float)p1.x, s, z);
  f[2] = fmaf((float)p2.x, s, z);
  f[3] = fmaf((float)p3.x, s, z);
  f[4] = fmaf((float)p0.y, s, z);
  f[5] = fmaf((float)p1.y, s, z);
  f[6] = fmaf((float)p2.y, s, z);
  f[7] = fmaf((float)p3.y, s, z);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = (__bf16)f[i];
    lo[i] = (__bf16)(f[i] - (float)hi[i]);
  }
}

// acc0 (token rows 0..31) and, when TWO, acc1 (rows 32..63) += one bf16 X
// tile times the chunk's weights as hi + lo parts (two products per MFMA step
// and token tile), operands as in mfma_tile.  The weights' error is then
// 2^-16 of their size, whatever the distribution of X.
template <int KIND, bool TWO>
__device__ __forceinline__ void mfma_tile_w2(const GemmChunk<KIND>& c, const uint16_t* xb, int off1,
                                             f32x16& acc0, f32x16& acc1, uint32_t kMaskLo,
                                             uint32_t kMaskHi, uint32_t kMagic) {
  float s, z;
  group_sz<KIND>(c, 0, s, z);
  bf16x8 Bh, Bl;
  dequant8_hl(c.q[0][0], s, z, kMaskLo, kMaskHi, kMagic, Bh, Bl);
  bf16x8 A0 = *reinterpret_cast<const bf16x8*>(xb);
  bf16x8 A1 = A0;
  if constexpr (TWO) A1 = *reinterpret_cast<const bf16x8*>(xb + off1);
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    bf16x8 Bhn = Bh, Bln = Bl, A0n = A0, A1n = A1;
    if (st < 15) {
      const int sn = st + 1;
      if ((sn & 3) == 0) group_sz<KIND>(c, sn >> 2, s, z);
      dequant8_hl(c.q[sn >> 2][sn & 3], s, z, kMaskLo, kMaskHi, kMagic, Bhn, Bln);
      A0n = *reinterpret_cast<const bf16x8*>(xb + 8 * sn);
      if constexpr (TWO) A1n = *reinterpret_cast<const bf16x8*>(xb + off1 + 8 * sn);
    }
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, Bh, acc0, 0, 0, 0);
    if constexpr (TWO) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, Bh, acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, Bl, acc0, 0, 0, 0);
    if constexpr (TWO) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, Bl, acc1, 0, 0, 0);
    Bh = Bhn;
    Bl = Bln;
    A0 = A0n;
    A1 = A1n;
    if (st < 15) {
      constexpr int NM = TWO ? 4 : 2;   // products per MFMA step
      __builtin_amdgcn_sched_group_barrier(0x100, TWO ? 2 : 1, 0);    // DS reads
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x002, 40 / NM, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
      }
    }
  }
}

// The same for an fp32 operand held as two bf16 tiles, hi = bf16(x) and
// lo = bf16(x - hi), at xb and xb + offl (rows n; rows n + 32 at + off1):
// acc += xhi whi + xhi wlo + xlo whi, three products per MFMA step and token
// tile (the dropped xlo wlo is below 2^-16 of each product).
template <int KIND, bool TWO>
__device__ __forceinline__ void mfma_tile_hl(const GemmChunk<KIND>& c, const uint16_t* xb, int off1,
                                             int offl, f32x16& acc0, f32x16& acc1, uint32_t kMaskLo,
                                             uint32_t kMaskHi, uint32_t kMagic) {
  float s, z;
  group_sz<KIND>(c, 0, s, z);
  bf16x8 Bh, Bl;
  dequant8_hl(c.q[0][0], s, z, kMaskLo, kMaskHi, kMagic, Bh, Bl);
  // A[0], A[1]: hi of rows n, n + 32; A[2], A[3]: lo of rows n, n + 32
  constexpr int NA = TWO ? 4 : 2;
  auto aoff = [&](int i) { return TWO ? (i & 1) * off1 + (i >> 1) * offl : i * offl; };
  bf16x8 A[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) A[i] = *reinterpret_cast<const bf16x8*>(xb + aoff(i));
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    bf16x8 Bhn = Bh, Bln = Bl, An[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) An[i] = A[i];
    if (st < 15) {
      const int sn = st + 1;
      if ((sn & 3) == 0) group_sz<KIND>(c, sn >> 2, s, z);
      dequant8_hl(c.q[sn >> 2][sn & 3], s, z, kMaskLo, kMaskHi, kMagic, Bhn, Bln);
#pragma unroll
      for (int i = 0; i < NA; ++i) An[i] = *reinterpret_cast<const bf16x8*>(xb + aoff(i) + 8 * sn);
    }
    if constexpr (TWO) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[0], Bh, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[1], Bh, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[0], Bl, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[1], Bl, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[2], Bh, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[3], Bh, acc1, 0, 0, 0);
    } else {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[0], Bh, acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[0], Bl, acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[1], Bh, acc0, 0, 0, 0);
    }
    Bh = Bhn;
    Bl = Bln;
#pragma unroll
    for (int i = 0; i < NA; ++i) A[i] = An[i];
    if (st < 15) {
      constexpr int NM = TWO ? 6 : 3;   // products per MFMA step
      __builtin_amdgcn_sched_group_barrier(0x100, NA, 0);    // DS reads
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x002, 42 / NM, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
      }
    }
  }
}

}  // namespace q4nx
