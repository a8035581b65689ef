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
// column are prepared once per chunk.
//
// A group's weights are w_k = s c_k + z (q4_1: scale s, zero z; Q4_K:
// s = S*scale, z = M*min, both products exact in fp32).  With any integer c0,
//     sum_k w_k x_k = s * sum_k (c_k - c0) x_k + (z + c0 s) * sum_k x_k.
// The library takes c0 = clamp(round(-z/s), 0, 15), the code nearest the
// group's zero crossing, so that |z + c0 s| <= |s|/2 whenever the crossing lies
// inside the code range, and z + c0 s has the sign of every s (c_k - c0) term
// otherwise.  Then |s| |c_k - c0| + |z + c0 s| <= 3 |w_k| for every k: the two
// parts of the sum never cancel more than their own terms, so the error of the
// factored sum stays a small multiple of sum |w x| (the bound the oracle
// checks), for any codes and any (s, z).  (Any c0 gives the same exact value;
// the choice only bounds the rounding.)  The pair z + c0 s is exact in fp32
// when the crossing is inside the code range (Sterbenz), so a one-hot x gives
// back fl(s c + z), the decoded weight, bit for bit.
//
// Signed codes: (w & 0x000F000F) | 0x64006400 makes nibbles 0 and 4 of a code
// word into the fp16 pair (1024 + c, 1024 + c'), and (w & 0x00F000F0) | ...
// nibbles 1 and 5 into (1024 + 16 c, 1024 + 16 c'); one v_pk_add_f16 with
// -(1024 + c0) (one v_pk_fma_f16 by 1/16 with -(64 + c0)) then gives the exact
// pair (c - c0, c' - c0).  v_dot2_f32_f16 multiplies it with the activation
// pair (x[k], x[k+4]); every product (5-bit code times 11-bit fp16) is exact.
//
// Activations are fp16 "records": the 32 values of one (row, tile column,
// group), each pair in the chain's order, scaled by 2^sigma so that the
// largest lands in [2^15, 2^16).  A bf16 value is exact in fp16 from 2^-17 up,
// so a record is exact whenever its nonzero values span at most 2^32; the
// record keeps f = 2^-sigma and X = sum x.  A record that is not exact (values
// spanning more, subnormal or huge bf16s) keeps its raw bf16 pairs and f = -1
// instead, and the lanes that own such a record run the same chain in bf16,
// with the signed codes converted to bf16 pairs (exact small integers).

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

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
// instead of 2 SL.  q4k_turn then hands each lane its own entries.
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

// Afterwards c holds, per slice i, the lane's (sc | mn << 8) and its row's
// (S, M), as q4_load_rs leaves them.  Lane l's entry of slice i is the 2 bytes
// at 128 i + 2 l of the unit's (sc, mn) region, its row's pair the one in
// rowsm[0] of lane 8 i + l / 8.
//   SL <= 2: ds_bpermute fetches both from the lanes that hold them (for
//   SL = 2 the entry is in the upper half of lane 32 i + l / 2's word when l
//   is odd; for one slice it is the lane's own): no LDS memory, no barrier.
//   SL = 4: the lanes hold 8 bytes each, and one permute per slice would need
//   two plus a select; instead the wave writes its loads to ts, its slot of
//   160 SL bytes, and reads its entries back.  The wave's LDS operations run
//   in order; the fences keep the compiler from moving them across each other.
// The split follows measurement: at SL = 4 the slot was faster, at SL <= 2
// the permutes.
template <int SL>
__device__ __forceinline__ void q4k_turn(uint8_t* ts, int lane, Q4Chunk<KIND_Q4_K, SL>& c) {
  if constexpr (SL == 4) {
    *reinterpret_cast<u32x2*>(ts + 8 * lane) = u32x2{c.meta[0], c.meta[1]};
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
  } else {
    uint32_t meta[SL], row[SL];
    const uint32_t rs = c.rowsm[0];
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      if constexpr (SL == 2) {
        const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (32 * i + (lane >> 1)), (int)c.meta[0]);
        meta[i] = (v >> (16 * (lane & 1))) & 0xFFFFu;
      } else {
        meta[i] = c.meta[0] & 0xFFFFu;
      }
      row[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (8 * i + (lane >> 3)), (int)rs);
    }
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      c.meta[i] = meta[i];
      c.rowsm[i] = row[i];
    }
  }
}

// --------------------------------------------------------------------------
// activation records
// --------------------------------------------------------------------------
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

// The 16 bf16 pairs of a group in chain order: pair 4d + j is (x[8d + j], x[8d + j + 4]).
__device__ __forceinline__ void bf16_chain_pairs(const u32x4 (&v)[4], uint32_t (&p)[16]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // v_perm_b32 byte select: 0..3 pick bytes of the second operand, 4..7 of the first.
    p[4 * d + 0] = __builtin_amdgcn_perm(v[d].z, v[d].x, 0x05040100u);   // (x0, x4)
    p[4 * d + 1] = __builtin_amdgcn_perm(v[d].z, v[d].x, 0x07060302u);   // (x1, x5)
    p[4 * d + 2] = __builtin_amdgcn_perm(v[d].w, v[d].y, 0x05040100u);   // (x2, x6)
    p[4 * d + 3] = __builtin_amdgcn_perm(v[d].w, v[d].y, 0x07060302u);   // (x3, x7)
  }
}

// sum of the 32 values of a group of bf16 pairs (fixed order, fp32)
__device__ __forceinline__ float bf16_pairs_sum(const uint32_t (&p)[16]) {
  float e = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t) e = dot2bf16(0x3F803F80u, p[t], e);   // (1, 1)
  return e;
}

// Quad reductions: the 4 consecutive lanes of a record meet through DPP
// quad permutations (xor 1, then xor 2), so every lane ends with the result.
// Each permuted value is read once, outside any branch: a DPP read from a lane
// that is switched off in the exec mask does not return its value.
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
}
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = __builtin_elementwise_max(v, quad_xor1(v));
  return __builtin_elementwise_max(v, quad_xor2(v));
}
__device__ __forceinline__ float quad_sum(float v) {
  v += __uint_as_float(quad_xor1(__float_as_uint(v)));
  return v + __uint_as_float(quad_xor2(__float_as_uint(v)));
}

// One quarter of an fp16 record (see above), built by the 4 consecutive lanes
// that share the record: this lane holds v = x[8d .. 8d+7] of the group (d =
// its place in the quad) and gets the chain pairs 4d .. 4d+3, p[j] = (x[8d+j],
// x[8d+j+4]), plus the record's f = 2^-sigma (or -1 for a bf16 record) and
// X = sum of the 32 values.  Every lane of the quad must call it.
__device__ __forceinline__ void x_record_part(const u32x4 v, uint32_t (&p)[4], float& f, float& X) {
  // largest magnitude (as bits) and a lower bound on the smallest nonzero
  // exponent: (b - 1) & 0x7F80 is the exponent field of b, one less when the
  // mantissa is zero (conservative), 0 for a subnormal, and 0x7F80 for a zero
  // (which then never wins the minimum).
  u16x2 mx = {0, 0}, mn = {0x7F80, 0x7F80};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const u16x2 a = __builtin_bit_cast(u16x2, v[t] & 0x7FFF7FFFu);
    mx = __builtin_elementwise_max(mx, a);
    mn = __builtin_elementwise_min(mn, a - u16x2{1, 1});
  }
  const uint32_t top = quad_max_u32(mx.x > mx.y ? mx.x : mx.y);   // bits of max |x|
  // min over the quad through max of the complement
  const uint32_t mnl = (mn.x < mn.y ? mn.x : mn.y) & 0x7F80u;
  const uint32_t low = 0x7F80u - quad_max_u32(0x7F80u - mnl);
  const int E = (int)(top >> 7), Emin = (int)(low >> 7);
  // exact in fp16 after scaling: max in [2^15, 2^16), every nonzero value
  // >= 2^-17 (exponent field >= E - 32); keep 2^sigma within 2^64 either way
  const bool fast = top == 0 || (E >= 78 && E <= 206 && Emin >= E - 32);
  float xs;
  if (fast) {
    const float up = top == 0 ? 1.f : __uint_as_float((uint32_t)(269 - E) << 23);   // 2^sigma, sigma = 142 - E
    f = top == 0 ? 1.f : __uint_as_float((uint32_t)(E - 15) << 23);                // 2^-sigma
    p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16lo(v.x) * up, bf16lo(v.z) * up));
    p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16hi(v.x) * up, bf16hi(v.z) * up));
    p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16lo(v.y) * up, bf16lo(v.w) * up));
    p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16hi(v.y) * up, bf16hi(v.w) * up));
    float e = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) e = dot2f16(0x3C003C00u, p[t], e);   // (1, 1)
    xs = e * f;
  } else {
    // v_perm_b32 byte select: 0..3 pick bytes of the second operand, 4..7 of the first.
    p[0] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);   // (x0, x4)
    p[1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);   // (x1, x5)
    p[2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);   // (x2, x6)
    p[3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);   // (x3, x7)
    f = -1.f;
    float e = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) e = dot2bf16(0x3F803F80u, p[t], e);   // (1, 1)
    xs = e;
  }
  X = quad_sum(xs);
}

// One quarter of an fp16 record of fp32 activations (the MoE intermediate h),
// built by four consecutive lanes: this lane holds a = h[8d .. 8d+3] and
// b = h[8d+4 .. 8d+7].  The values are scaled by 2^sigma (largest in
// [2^14, 2^15), sigma kept within +-64: an fp32 value just under 2^16 would
// round to the fp16 infinity) and rounded to nearest fp16: each moves by at
// most 2^-12 of its size, or, below the fp16 normal range (values under 2^-28
// of the group's largest), by at most 2^-25 scaled units.
// X is the fp32 sum of the 32 unrounded values.
__device__ __forceinline__ void h_record_part(const f32x4 a, const f32x4 b, uint32_t (&p)[4], float& f,
                                              float& X) {
  const float m = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                        fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
  const uint32_t top = quad_max_u32(__float_as_uint(m));   // |values| compare as their bits
  int E = (int)(top >> 23);
  E = E < 77 ? 77 : (E > 205 ? 205 : E);
  const float up = __uint_as_float((uint32_t)(268 - E) << 23);   // 2^sigma, sigma = 141 - E
  f = __uint_as_float((uint32_t)(E - 14) << 23);                // 2^-sigma
  const f16x2 q0 = {(_Float16)(a.x * up), (_Float16)(b.x * up)};   // (h0, h4)
  const f16x2 q1 = {(_Float16)(a.y * up), (_Float16)(b.y * up)};   // (h1, h5)
  const f16x2 q2 = {(_Float16)(a.z * up), (_Float16)(b.z * up)};   // (h2, h6)
  const f16x2 q3 = {(_Float16)(a.w * up), (_Float16)(b.w * up)};   // (h3, h7)
  p[0] = __builtin_bit_cast(uint32_t, q0);
  p[1] = __builtin_bit_cast(uint32_t, q1);
  p[2] = __builtin_bit_cast(uint32_t, q2);
  p[3] = __builtin_bit_cast(uint32_t, q3);
  X = quad_sum(((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w)));
}

// The same record built by one lane from all 32 values (v[d] = x[8d .. 8d+7]).
__device__ __forceinline__ void x_record(const u32x4 (&v)[4], uint32_t (&p)[16], float& f, float& X) {
  u16x2 mx = {0, 0}, mn = {0x7F80, 0x7F80};
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u16x2 a = __builtin_bit_cast(u16x2, v[d][t] & 0x7FFF7FFFu);
      mx = __builtin_elementwise_max(mx, a);
      mn = __builtin_elementwise_min(mn, a - u16x2{1, 1});
    }
  const uint32_t top = mx.x > mx.y ? mx.x : mx.y;
  const int E = (int)(top >> 7);
  const int Emin = (int)(((mn.x < mn.y ? mn.x : mn.y) & 0x7F80u) >> 7);
  const bool fast = top == 0 || (E >= 78 && E <= 206 && Emin >= E - 32);
  if (fast) {
    const float up = top == 0 ? 1.f : __uint_as_float((uint32_t)(269 - E) << 23);
    f = top == 0 ? 1.f : __uint_as_float((uint32_t)(E - 15) << 23);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4 w = v[d];
      p[4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16lo(w.x) * up, bf16lo(w.z) * up));
      p[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16hi(w.x) * up, bf16hi(w.z) * up));
      p[4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16lo(w.y) * up, bf16lo(w.w) * up));
      p[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16hi(w.y) * up, bf16hi(w.w) * up));
    }
    float e = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) e = dot2f16(0x3C003C00u, p[t], e);   // (1, 1)
    X = e * f;
  } else {
    bf16_chain_pairs(v, p);
    f = -1.f;
    X = bf16_pairs_sum(p);
  }
}

// M prepared records of one tile column (one per activation row).
template <int M>
struct XRec {
  uint32_t p[M][16];
  float f[M];
  float X[M];
};

template <int M>
__device__ __forceinline__ void x_records(const XRaw<M>& r, XRec<M>& xp) {
#pragma unroll
  for (int m = 0; m < M; ++m) x_record(r.v[m], xp.p[m], xp.f[m], xp.X[m]);
}

// bf16-only records (the exact fallback form, used where records are built per
// lane and per chunk): raw pairs, f = -1.  PL planes: a fp32 activation is
// carried as the sum of PL bf16 values (plane 0 = bf16(x), plane 1 = bf16(x -
// plane 0)).
template <int M, int PL = 1>
struct XRecB {
  uint32_t p[M][PL][16];
  float X[M];
};

template <int M>
__device__ __forceinline__ void x_records_b(const XRaw<M>& r, XRecB<M>& xp) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    bf16_chain_pairs(r.v[m], xp.p[m][0]);
    xp.X[m] = bf16_pairs_sum(xp.p[m][0]);
  }
}

// --------------------------------------------------------------------------
// products
// --------------------------------------------------------------------------
// A slice's group: scale, zero, center code and its fp16 constants.
struct Q4Group {
  float s, delta;      // delta = z + c0 s
  uint32_t pkl, pkh;   // fp16 pairs -(1024 + c0), -(64 + c0)
};

template <int KIND, int SL>
__device__ __forceinline__ Q4Group q4_group(const Q4Chunk<KIND, SL>& c, int i) {
  float s, z;
  if constexpr (KIND == KIND_Q4_1) {
    s = bf16lo(c.meta[i]);
    z = bf16hi(c.meta[i]);
  } else {
    s = bf16lo(c.rowsm[i]) * (float)(c.meta[i] & 0xFFu);
    z = bf16hi(c.rowsm[i]) * (float)((c.meta[i] >> 8) & 0xFFu);
  }
  // c0 = clamp(round(-z / s), 0, 15); the reciprocal's rounding only moves
  // the choice near half-integers, which keeps |z + c0 s| within 0.5 |s| plus a
  // few ulps.  s = 0 or a NaN lands on 0 or 15: any c0 is exact.
  const float t = fminf(fmaxf(fmaf(-z, __builtin_amdgcn_rcpf(s), 0.5f), 0.f), 15.5f);
  const uint32_t c0 = (uint32_t)t;
  const uint32_t c2 = (c0 << 16) | c0;   // c0 in both halves
  Q4Group gp;
  gp.s = s;
  gp.delta = fmaf((float)c0, s, z);
  gp.pkl = 0xE400E400u | c2;
  gp.pkh = (c2 << 4) | 0xD400D400u;
  return gp;
}

// Unpack constants kept in registers: gfx9 VOP3 instructions take no literal,
// so a mask in an SGPR and the magic in a VGPR let one v_and_or_b32 build a pair.
struct Q4Consts {
  uint32_t mlo, mhi, magic;
};

__device__ __forceinline__ Q4Consts q4_consts() {
  uint32_t a = 0x000F000Fu, b = 0x00F000F0u, c = 0x64006400u;
  asm volatile("" : "+s"(a));
  asm volatile("" : "+s"(b));
  asm volatile("" : "+v"(c));
  return Q4Consts{a, b, c};
}

// The 16 signed code pairs of one 32-code run, in chain order.
__device__ __forceinline__ void q4_signed(const u32x4& q, const Q4Group& gp, const Q4Consts& k,
                                          uint32_t (&cp)[16]) {
  const f16x2 lo = __builtin_bit_cast(f16x2, gp.pkl), hi = __builtin_bit_cast(f16x2, gp.pkh);
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = q[d], w8 = w >> 8;
    const f16x2 a0 = __builtin_bit_cast(f16x2, (w & k.mlo) | k.magic);    // (1024 + c, 1024 + c')
    const f16x2 a1 = __builtin_bit_cast(f16x2, (w & k.mhi) | k.magic);    // (1024 + 16 c, ...)
    const f16x2 a2 = __builtin_bit_cast(f16x2, (w8 & k.mlo) | k.magic);
    const f16x2 a3 = __builtin_bit_cast(f16x2, (w8 & k.mhi) | k.magic);
    cp[4 * d + 0] = __builtin_bit_cast(uint32_t, a0 + lo);
    cp[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(a1, sixteenth, hi));
    cp[4 * d + 2] = __builtin_bit_cast(uint32_t, a2 + lo);
    cp[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(a3, sixteenth, hi));
  }
}

// fp16 signed code pair -> bf16 pair (small integers: exact).
__device__ __forceinline__ uint32_t f16pair_to_bf16(uint32_t c) {
  const f16x2 h = __builtin_bit_cast(f16x2, c);
  const bf16x2 b = {(__bf16)(float)h.x, (__bf16)(float)h.y};
  return __builtin_bit_cast(uint32_t, b);
}

// acc[i][m] += the slices' products with the fp16 records (bf16 records on
// the lanes that hold one).
template <int KIND, int M, int SL = 4>
__device__ __forceinline__ void q4_compute(const Q4Chunk<KIND, SL>& c, const XRec<M>& xp,
                                           const Q4Consts& k, float (&acc)[SL][M]) {
  bool slow = false;
#pragma unroll
  for (int m = 0; m < M; ++m) slow |= xp.f[m] < 0.f;
  const bool wslow = __builtin_amdgcn_ballot_w64(slow) != 0;   // uniform
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const Q4Group gp = q4_group<KIND, SL>(c, i);
    uint32_t cp[16];
    q4_signed(c.q[i], gp, k, cp);
    float D[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float e = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) e = dot2f16(cp[t], xp.p[m][t], e);
      D[m] = e;
    }
    if (wslow) {
      uint32_t cb[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) cb[t] = f16pair_to_bf16(cp[t]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (xp.f[m] < 0.f) {
          float e = 0.f;
#pragma unroll
          for (int t = 0; t < 16; ++t) e = dot2bf16(cb[t], xp.p[m][t], e);
          D[m] = e;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
      acc[i][m] = fmaf(gp.s * fabsf(xp.f[m]), D[m], fmaf(gp.delta, xp.X[m], acc[i][m]));
  }
}

// The same products with bf16-only records of PL planes.
template <int KIND, int M, int PL, int SL = 4>
__device__ __forceinline__ void q4_compute_b(const Q4Chunk<KIND, SL>& c, const XRecB<M, PL>& xp,
                                             const Q4Consts& k, float (&acc)[SL][M]) {
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const Q4Group gp = q4_group<KIND, SL>(c, i);
    uint32_t cp[16];
    q4_signed(c.q[i], gp, k, cp);
#pragma unroll
    for (int t = 0; t < 16; ++t) cp[t] = f16pair_to_bf16(cp[t]);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float e = 0.f;
#pragma unroll
      for (int pl = 0; pl < PL; ++pl)
#pragma unroll
        for (int t = 0; t < 16; ++t) e = dot2bf16(cp[t], xp.p[m][pl][t], e);
      acc[i][m] = fmaf(gp.s, e, fmaf(gp.delta, xp.X[m], acc[i][m]));
    }
  }
}

// The same products for several activation rows on the matrix cores
// (v_mfma_f32_4x4x4_16b_f16: 16 independent 4x4 blocks, 4 products deep).
// The lanes of a wave split a slice as 4-lane blocks: the 4 lanes of block
// l / 4 hold the codes of 4 rows of one group (k_gemv_q4m gives the order),
// and lane l the record of that group for activation row 4 blk + (l & 3)
// (on gfx950, A row i and B column j of a block come from its lane i and j,
// and result D[r][j] sits in register r of lane j).  Block l / 4 multiplies the
// records (4 activation rows x 4 columns of the group) by the codes (4 columns
// x 4 weight rows), and after the group's 8 steps lane l holds, for its own
// weight row, D[t] = sum over the group of code * record for activation rows
// 4 blk + t, t = 0..3.  Step st takes chain pairs 2 st and 2 st + 1 of both
// the record and the codes, so every product pairs the same column.  Products
// of a code and an fp16 are exact and the sum is kept in fp32, as in the dot
// chain; a record kept in bf16 (f < 0) takes the bf16 form of the same step
// (v_mfma_f32_4x4x4_16b_bf16, exact small-integer codes), whose rows for the
// fp16 records are discarded.  fv, Xv: f and X of the records of activation
// rows 4 blk + t in the lane's group.
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int KIND, int M, int NB, int SL>
__device__ __forceinline__ void q4_compute_mfma(const Q4Chunk<KIND, SL>& c, const uint32_t (&pa)[NB][16],
                                                const float (&fv)[NB][4], const float (&Xv)[NB][4],
                                                const Q4Consts& k, float (&acc)[SL][M]) {
  bool slow = false;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (4 * blk + t < M) slow |= fv[blk][t] < 0.f;
  const bool wslow = __builtin_amdgcn_ballot_w64(slow) != 0;   // uniform
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const Q4Group gp = q4_group<KIND, SL>(c, i);
    uint32_t cp[16];
    q4_signed(c.q[i], gp, k, cp);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const f16x4 a = __builtin_bit_cast(f16x4, u32x2{pa[blk][2 * st], pa[blk][2 * st + 1]});
        const f16x4 w = __builtin_bit_cast(f16x4, u32x2{cp[2 * st], cp[2 * st + 1]});
        d = __builtin_amdgcn_mfma_f32_4x4x4f16(a, w, d, 0, 0, 0);
      }
      if (wslow) {
        f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const i16x4 a = __builtin_bit_cast(i16x4, u32x2{pa[blk][2 * st], pa[blk][2 * st + 1]});
          const i16x4 w = __builtin_bit_cast(
              i16x4, u32x2{f16pair_to_bf16(cp[2 * st]), f16pair_to_bf16(cp[2 * st + 1])});
          e = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, w, e, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (fv[blk][t] < 0.f) d[t] = e[t];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = 4 * blk + t;
        if (m < M) acc[i][m] = fmaf(gp.s * fabsf(fv[blk][t]), d[t], fmaf(gp.delta, Xv[blk][t], acc[i][m]));
      }
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
// with q4_lane_reduce).  xrow[m] points at activation row m, column 0.  The
// activations are loaded per lane and chunk, so they are taken as bf16 records.
template <int KIND, int M>
__device__ __forceinline__ void q4_step(const Q4Chunk<KIND>& ch, const uint16_t* const (&xrow)[M],
                                        int c, const Q4Consts& k, float (&acc)[4][M]) {
  XRaw<M> r;
  x_raw<M>(xrow, 256 * c, r);
  XRecB<M> xb;
  x_records_b<M>(r, xb);
  q4_compute_b<KIND, M, 1>(ch, xb, k, acc);
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
  const Q4Consts k = q4_consts();
  const int n = c1 - c0;
  Q4Chunk<KIND> ring[D];
#pragma unroll
  for (int b = 0; b < D; ++b)
    if (b < n) q4_load<KIND>(row + (size_t)(c0 + b) * CB, lane, ring[b]);
  for (int i = 0; i < n; i += D) {
#pragma unroll
    for (int b = 0; b < D; ++b) {
      if (i + b < n) {
        q4_step<KIND, M>(ring[b], xrow, c0 + i + b, k, acc);
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
