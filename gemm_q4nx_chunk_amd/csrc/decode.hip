// Chunk decoders as a test surface (1bit engine docs, page "NPU engine",
// section "Q4NX chunks": the decoders of the three kinds are checked bit for
// bit).  One workgroup per chunk; thread t handles row r = t/8, group g = t%8
// (32 weights) and writes its codes, metadata and fp32 weights in logical
// [rows][cols] order.
//
// fp32 values: q4_1 is one fma (exact product, one rounding); Q8's d*code is
// exact; Q4_K sums two exact fp64 products and rounds (see below).  Each is the
// exact value of the formula rounded once to nearest even.
#include "q4nx_dev.h"

namespace q4nx {

template <int KIND>
__global__ __launch_bounds__(256) void k_unpack(const uint8_t* __restrict__ w, int TR, int TC,
                                                uint8_t* __restrict__ codes,
                                                uint16_t* __restrict__ meta0,
                                                uint16_t* __restrict__ meta1,
                                                uint16_t* __restrict__ row_meta,
                                                float* __restrict__ out) {
  constexpr int CB = ChunkBytes<KIND>::value;
  const int chunk = blockIdx.x, tr = chunk / TC, tc = chunk - tr * TC;
  const int r = threadIdx.x >> 3, g = threadIdx.x & 7;
  const uint8_t* ck = w + (size_t)chunk * CB;
  const int K = TC * 256, G = K / 32;
  const size_t row = (size_t)tr * 32 + r;
  const int col0 = tc * 256 + g * 32;

  uint8_t c8[32];
  uint16_t m0 = 0, m1 = 0, S = 0, Mm = 0;
  float val[32];
  if constexpr (KIND == KIND_Q4_1 || KIND == KIND_Q4_K) {
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(ck + r * 128 + g * 16);
#pragma unroll
    for (int j = 0; j < 32; ++j) c8[j] = (uint8_t)((v0[j >> 3] >> (4 * (j & 7))) & 0xFu);
    if constexpr (KIND == KIND_Q4_1) {
      const uint32_t sz = *reinterpret_cast<const uint32_t*>(ck + 4096 + 4 * (8 * r + g));
      m0 = (uint16_t)(sz & 0xFFFFu);
      m1 = (uint16_t)(sz >> 16);
      const float s = bf16lo(sz), z = bf16hi(sz);
#pragma unroll
      for (int j = 0; j < 32; ++j) val[j] = fmaf((float)c8[j], s, z);
    } else {
      const uint16_t scmn = *reinterpret_cast<const uint16_t*>(ck + 4096 + 2 * (8 * r + g));
      const uint32_t sm = *reinterpret_cast<const uint32_t*>(ck + 4608 + 4 * r);
      m0 = scmn & 0xFFu;
      m1 = scmn >> 8;
      S = (uint16_t)(sm & 0xFFFFu);
      Mm = (uint16_t)(sm >> 16);
      // S*scale*code and M*min are exact in fp64, and their fp64 sum rounded to
      // fp32 is the exact value rounded once (fp64 has more than 2*24+2 bits).
      // fp32 products could overflow where the exact sum does not, so the test
      // surface works in fp64 with explicit, uncontracted roundings.
      const double a = __dmul_rn((double)bf16lo(sm), (double)m0);
      const double b = __dmul_rn((double)bf16hi(sm), (double)m1);
#pragma unroll
      for (int j = 0; j < 32; ++j) val[j] = (float)__dadd_rn(__dmul_rn(a, (double)c8[j]), b);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int k = g * 32 + j;
      const int pos = (KIND == KIND_Q8_A)
                          ? k * 32 + r
                          : (r >> 4) * 4096 + (k >> 5) * 512 + (k & 31) * 16 + (r & 15);
      c8[j] = ck[pos];
    }
    m0 = *reinterpret_cast<const uint16_t*>(ck + 8192 + 2 * (8 * r + g));
    const float d = __uint_as_float((uint32_t)m0 << 16);
#pragma unroll
    for (int j = 0; j < 32; ++j) val[j] = d * (float)(int8_t)c8[j];
  }

  if (codes) {
    uint8_t* dst = codes + row * K + col0;
#pragma unroll
    for (int j = 0; j < 32; ++j) dst[j] = c8[j];
  }
  if (meta0) meta0[row * G + tc * 8 + g] = m0;
  if (meta1) meta1[row * G + tc * 8 + g] = m1;
  if (row_meta && g == 0) {
    row_meta[(row * TC + tc) * 2 + 0] = S;
    row_meta[(row * TC + tc) * 2 + 1] = Mm;
  }
  if (out) {
    float* dst = out + row * K + col0;
#pragma unroll
    for (int j = 0; j < 32; ++j) dst[j] = val[j];
  }
}

template <int KIND>
static void launch_k(const uint8_t* w, int TR, int TC, uint8_t* codes, uint16_t* meta0,
                     uint16_t* meta1, uint16_t* row_meta, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_unpack<KIND>, dim3(TR * TC), dim3(256), 0, s, w, TR, TC, codes, meta0,
                     meta1, row_meta, out);
}

static hipError_t launch_any(int kind, const uint8_t* w, int TR, int TC, uint8_t* codes,
                             uint16_t* meta0, uint16_t* meta1, uint16_t* row_meta, float* out,
                             hipStream_t s) {
  switch (kind) {
    case KIND_Q4_1: launch_k<KIND_Q4_1>(w, TR, TC, codes, meta0, meta1, row_meta, out, s); break;
    case KIND_Q4_K: launch_k<KIND_Q4_K>(w, TR, TC, codes, meta0, meta1, row_meta, out, s); break;
    case KIND_Q8_A: launch_k<KIND_Q8_A>(w, TR, TC, codes, meta0, meta1, row_meta, out, s); break;
    case KIND_Q8_B: launch_k<KIND_Q8_B>(w, TR, TC, codes, meta0, meta1, row_meta, out, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_unpack(int kind, const uint8_t* w, int TR, int TC, uint8_t* codes,
                         uint16_t* meta0, uint16_t* meta1, uint16_t* row_meta, hipStream_t s) {
  return launch_any(kind, w, TR, TC, codes, meta0, meta1, row_meta, nullptr, s);
}

hipError_t launch_decode(int kind, const uint8_t* w, int TR, int TC, float* out, hipStream_t s) {
  return launch_any(kind, w, TR, TC, nullptr, nullptr, nullptr, nullptr, out, s);
}

// ---------------------------------------------------------------------------
// Q4_K -> q4_1 repack (1bit engine docs, page "NPU engine", section "Q4NX
// chunks": Q4_K weights are repacked to q4_1, exactly apart from rounding
// S * scale and M * min to bf16, so a q4_1 kernel serves both kinds).
// One workgroup per chunk: the 4096 code bytes are copied unchanged (256
// threads x 16 bytes) and thread t = 8r + g writes (scale', zero') of row r,
// group g: S * sc and M * mn are exact in fp32 (8 x 8 significant bits) and
// are rounded once, to nearest even, to bf16.  Products outside the fp32
// range are outside the repack's domain.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_repack_q4k(const uint8_t* __restrict__ w, uint8_t* __restrict__ out) {
  const int t = threadIdx.x, r = t >> 3, g = t & 7;
  const uint8_t* ck = w + (size_t)blockIdx.x * 4736;
  uint8_t* oc = out + (size_t)blockIdx.x * 5120;
  *reinterpret_cast<u32x4*>(oc + 16 * t) = *reinterpret_cast<const u32x4*>(ck + 16 * t);
  const uint32_t scmn = *reinterpret_cast<const uint16_t*>(ck + 4096 + 2 * (8 * r + g));
  const uint32_t sm = *reinterpret_cast<const uint32_t*>(ck + 4608 + 4 * r);
  const float s = bf16lo(sm) * (float)(scmn & 0xFFu);
  const float z = bf16hi(sm) * (float)(scmn >> 8);
  const uint32_t sb = __builtin_bit_cast(uint16_t, (__bf16)s);
  const uint32_t zb = __builtin_bit_cast(uint16_t, (__bf16)z);
  *reinterpret_cast<uint32_t*>(oc + 4096 + 4 * (8 * r + g)) = sb | (zb << 16);
}

// ---------------------------------------------------------------------------
// relayout: chunks in a described in-chunk layout -> the library's layout
// ---------------------------------------------------------------------------
// One workgroup per chunk: the source chunk comes into LDS with 16-byte loads,
// then each thread assembles 16 bytes of the output chunk (code bytes r*128 +
// k/2 hold codes k, k+1 of row r; then the metadata records) and stores them.
__device__ __forceinline__ uint32_t rl_code(const uint8_t* c, const ChunkLayout& L, int r, int k) {
  const int g = k >> 5, j = k & 31;
  const int b = L.code_pairing ? (j & 15) : (j >> 1);
  const int n = (L.code_pairing ? (j >> 4) : (j & 1)) ^ (L.code_high_first ? 1 : 0);
  const uint8_t v = c[L.code_off + r * L.code_row + g * L.code_group + b * L.code_step];
  return n ? (uint32_t)(v >> 4) : (uint32_t)(v & 15u);
}

__device__ __forceinline__ uint32_t rl_u16(const uint8_t* c, int off) {
  return (uint32_t)c[off] | ((uint32_t)c[off + 1] << 8);
}

__global__ __launch_bounds__(256) void k_relayout(ChunkLayout L, const uint8_t* __restrict__ src,
                                                  uint8_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t c[5120];
  const int CB = L.chunk_bytes, tid = threadIdx.x;
  const uint8_t* s = src + (size_t)blockIdx.x * CB;
  uint8_t* o = out + (size_t)blockIdx.x * CB;
  for (int p = tid; p < CB / 16; p += 256)
    *reinterpret_cast<u32x4*>(c + 16 * p) = *reinterpret_cast<const u32x4*>(s + 16 * p);
  __syncthreads();
  for (int p = tid; p < CB / 16; p += 256) {
    uint32_t w[4] = {0, 0, 0, 0};
    for (int e = 0; e < 16; ++e) {
      const int ob = 16 * p + e;   // output byte
      uint32_t v;
      if (ob < 4096) {
        const int r = ob >> 7, k = 2 * (ob & 127);
        v = rl_code(c, L, r, k) | (rl_code(c, L, r, k + 1) << 4);
      } else if (CB == 5120) {    // q4_1 (scale, zero) of (r, g) at 4096 + 4 (8r + g)
        const int q = ob - 4096, rg = q >> 2, r = rg >> 3, g = rg & 7, f = q & 3;
        const int off = f < 2 ? L.f0_off + r * L.f0_row + g * L.f0_group : L.f1_off + r * L.f1_row + g * L.f1_group;
        v = c[off + (f & 1)];
      } else if (ob < 4608) {      // Q4_K (scale, min) of (r, g) at 4096 + 2 (8r + g)
        const int q = ob - 4096, rg = q >> 1, r = rg >> 3, g = rg & 7;
        v = (q & 1) ? c[L.f1_off + r * L.f1_row + g * L.f1_group] : c[L.f0_off + r * L.f0_row + g * L.f0_group];
      } else {                     // Q4_K (S, M) of row r at 4608 + 4r
        const int q = ob - 4608, r = q >> 2, f = q & 3;
        v = rl_u16(c, f < 2 ? L.s_off + r * L.s_row : L.m_off + r * L.m_row) >> (8 * (f & 1)) & 0xFFu;
      }
      w[e >> 2] |= (v & 0xFFu) << (8 * (e & 3));
    }
    *reinterpret_cast<u32x4*>(o + 16 * p) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

hipError_t launch_relayout(const ChunkLayout& L, const uint8_t* src, int tiles, uint8_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_relayout, dim3(tiles), dim3(256), 0, s, L, src, out);
  return hipGetLastError();
}

hipError_t launch_repack_q4k(const uint8_t* w, int tiles, uint8_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_repack_q4k, dim3(tiles), dim3(256), 0, s, w, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// GGUF 4-bit tensors -> q4_1 chunks (1bit engine docs, page "NPU engine",
// section "From a GGUF": Q4_0 maps to scale d, zero -8d; Q4_1 to scale d,
// zero m; Q4_K, per 32-column sub-block, to scale d*sc, zero -dmin*mn, a
// super-block being one tile row's 256 columns; codes unchanged, and rounding
// the scale and zero to bf16 the only error).  The GGUF blocks are the public
// format's: Q4_0 = fp16 d + 16 code bytes (18 B, 32 weights), Q4_1 = fp16 d,
// fp16 m + 16 code bytes (20 B), weight j < 16 in the low nibble of byte j and
// weight j + 16 in its high nibble; Q4_K = fp16 d, fp16 dmin, 12 bytes of
// 6-bit (sc, mn) pairs, 128 code bytes (144 B, 256 weights), sub-block j in the
// low (j even) or high (j odd) nibbles of code bytes 32 (j/2) .. 32 (j/2) + 31.
// Each row of the tensor is its K/32 (K/256) blocks in column order.
//
// One workgroup per tile; thread t = 8r + g builds row r, group g: it reads
// the one GGUF block (Q4_K: the sub-block) covering those 32 weights
// (staging a tile's blocks in LDS with whole 16-byte loads measured slower),
// reorders the codes into the chunk's order (even column in the low nibble),
// and writes its 16 code bytes and its (scale, zero) pair.  fp16 -> fp32 and
// the products d*sc, dmin*mn (11 x 6 significant bits) are exact; each field is
// rounded once, to nearest even.  Non-finite fp16 fields are outside the
// conversion's domain.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

// Four codes (one per byte of a and of b, in column order) -> 4 chunk bytes:
// columns 2i in the low nibble, 2i + 1 in the high one.
__device__ __forceinline__ uint32_t pack_code_pairs(uint32_t a, uint32_t b) {
  const uint32_t a2 = a | (a >> 4), b2 = b | (b >> 4);   // bytes 0 and 2 hold the pairs
  return (a2 & 0xFFu) | ((a2 >> 8) & 0xFF00u) | ((b2 & 0xFFu) << 16) | ((b2 << 8) & 0xFF000000u);
}

template <int GT>
__global__ __launch_bounds__(256) void k_gguf_q41(const uint8_t* __restrict__ src, int TC,
                                                  uint8_t* __restrict__ out) {
  const int t = threadIdx.x, r = t >> 3, g = t & 7;
  const int tile = blockIdx.x, tr = tile / TC, tc = tile - tr * TC;
  const size_t R = (size_t)tr * 32 + r;
  uint32_t c[4];
  float scale, zero;
  if constexpr (GT == 12) {   // Q4_K: super-block (R, tc), sub-block g
    const uint8_t* sb = src + (R * TC + tc) * 144;
    const u32x4 h = *reinterpret_cast<const u32x4*>(sb);
    const u32x4 q0 = *reinterpret_cast<const u32x4*>(sb + 16 + 32 * (g >> 1));
    const u32x4 q1 = *reinterpret_cast<const u32x4*>(sb + 32 + 32 * (g >> 1));
    const int sh = 4 * (g & 1);
    const uint32_t q[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int o = 0; o < 4; ++o)
      c[o] = pack_code_pairs((q[2 * o] >> sh) & 0x0F0F0F0Fu, (q[2 * o + 1] >> sh) & 0x0F0F0F0Fu);
    const uint32_t sw[3] = {h.y, h.z, h.w};   // the 12 scale bytes
    auto sbyte = [&](int j) { return (sw[j >> 2] >> (8 * (j & 3))) & 0xFFu; };
    uint32_t sc, mn;
    if (g < 4) {
      sc = sbyte(g) & 63u;
      mn = sbyte(g + 4) & 63u;
    } else {
      sc = (sbyte(g + 4) & 15u) | ((sbyte(g - 4) >> 6) << 4);
      mn = (sbyte(g + 4) >> 4) | ((sbyte(g) >> 6) << 4);
    }
    scale = f16_to_f32(h.x) * (float)sc;
    zero = -(f16_to_f32(h.x >> 16) * (float)mn);
  } else {                    // Q4_0 / Q4_1: block (R, 8 tc + g)
    constexpr int BB = GT == 2 ? 18 : 20;
    const uint8_t* bk = src + (R * TC * 8 + 8 * tc + g) * BB;
    uint32_t d, m = 0, q[4];
    if constexpr (GT == 2) {  // 2-byte aligned
      const uint16_t* h = reinterpret_cast<const uint16_t*>(bk);
      d = h[0];
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = (uint32_t)h[1 + 2 * i] | ((uint32_t)h[2 + 2 * i] << 16);
    } else {                  // 4-byte aligned
      const uint32_t* w = reinterpret_cast<const uint32_t*>(bk);
      d = w[0] & 0xFFFFu;
      m = w[0] >> 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = w[1 + i];
    }
    // low nibbles are columns 0..15, high nibbles 16..31
    c[0] = pack_code_pairs(q[0] & 0x0F0F0F0Fu, q[1] & 0x0F0F0F0Fu);
    c[1] = pack_code_pairs(q[2] & 0x0F0F0F0Fu, q[3] & 0x0F0F0F0Fu);
    c[2] = pack_code_pairs((q[0] >> 4) & 0x0F0F0F0Fu, (q[1] >> 4) & 0x0F0F0F0Fu);
    c[3] = pack_code_pairs((q[2] >> 4) & 0x0F0F0F0Fu, (q[3] >> 4) & 0x0F0F0F0Fu);
    scale = f16_to_f32(d);
    zero = GT == 2 ? -8.f * scale : f16_to_f32(m);
  }
  uint8_t* oc = out + (size_t)tile * 5120;
  *reinterpret_cast<u32x4*>(oc + 16 * t) = u32x4{c[0], c[1], c[2], c[3]};
  const uint32_t sb16 = __builtin_bit_cast(uint16_t, (__bf16)scale);
  const uint32_t zb16 = __builtin_bit_cast(uint16_t, (__bf16)zero);
  *reinterpret_cast<uint32_t*>(oc + 4096 + 4 * t) = sb16 | (zb16 << 16);
}

hipError_t launch_gguf_q41(int gtype, const uint8_t* src, int TR, int TC, uint8_t* out, hipStream_t s) {
  const dim3 grid(TR * TC);
  switch (gtype) {
    case 2: hipLaunchKernelGGL(k_gguf_q41<2>, grid, dim3(256), 0, s, src, TC, out); break;
    case 3: hipLaunchKernelGGL(k_gguf_q41<3>, grid, dim3(256), 0, s, src, TC, out); break;
    case 12: hipLaunchKernelGGL(k_gguf_q41<12>, grid, dim3(256), 0, s, src, TC, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Q8 row gather: rows of a Q8 weight (a tied embedding) decoded to fp32
// (1bit engine docs, page "NPU engine", section "Q4NX chunks": the Q8 kind
// stores the embedding / lm_head, code (r, k) of a tile at byte k*32 + r in
// layout A or (r/16)*4096 + (k/32)*512 + (k%32)*16 + r%16 in layout B).
// One workgroup per requested row; thread k takes column k of every tile
// column.  d * code is exact in fp32.  An id outside [0, rows) gives a row of
// zeros and touches no weight byte.
// ---------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(256) void k_q8_rows(const uint8_t* __restrict__ w, int rows, int TC,
                                                 const int32_t* __restrict__ ids, float* __restrict__ out) {
  const int t = blockIdx.x, k = threadIdx.x;
  const int id = ids[t];
  float* o = out + (size_t)t * TC * 256;
  if (id < 0 || id >= rows) {
    for (int tc = 0; tc < TC; ++tc) o[256 * tc + k] = 0.f;
    return;
  }
  const int tr = id >> 5, r = id & 31, g = k >> 5;
  const int off = KIND == KIND_Q8_A ? k * 32 + r : (r >> 4) * 4096 + (k >> 5) * 512 + (k & 31) * 16 + (r & 15);
  for (int tc = 0; tc < TC; ++tc) {
    const uint8_t* ck = w + ((size_t)tr * TC + tc) * 8704;
    const float c = (float)(int8_t)ck[off];
    const float d = bf16lo(*reinterpret_cast<const uint16_t*>(ck + 8192 + 2 * (8 * r + g)));
    o[256 * tc + k] = d * c;
  }
}

hipError_t launch_q8_rows(int kind, const uint8_t* w, int rows, int TC, const int32_t* ids, int T,
                          float* out, hipStream_t s) {
  if (kind == KIND_Q8_A) hipLaunchKernelGGL((k_q8_rows<KIND_Q8_A>), dim3(T), dim3(256), 0, s, w, rows, TC, ids, out);
  else if (kind == KIND_Q8_B) hipLaunchKernelGGL((k_q8_rows<KIND_Q8_B>), dim3(T), dim3(256), 0, s, w, rows, TC, ids, out);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// argmax over logits (greedy decode after the lm_head GEMV): per row m of
// y [M][n], the largest value and its index, the lowest index among equal
// values; NaNs are skipped (index -1 when a row holds only NaNs).  One
// workgroup per row; each thread scans a strided slice, then a fixed-order
// tree in LDS.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool am_better(float v, int i, float bv, int bi) {
  return bi < 0 || v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void am_take(float v, int i, float& bv, int& bi) {
  if (v == v && am_better(v, i, bv, bi)) { bv = v; bi = i; }
}

// One workgroup per row.  "Larger value, then lower index" is a total order
// on the non-NaN values, so the pick does not depend on which thread saw which
// element.  A 16-byte aligned row is streamed in 16-byte pieces, eight in
// flight per thread (unconditional buffer loads; pieces past the row read zero
// and are not taken); the last n % 4 elements, or the whole of an unaligned
// row, are read one by one.  Waves meet through lane shuffles, then the 16
// wave results in LDS.
__global__ __launch_bounds__(1024) void k_argmax(const float* __restrict__ y, int n, int ldy,
                                                 int32_t* __restrict__ idx, float* __restrict__ val) {
  __shared__ float sv[16];
  __shared__ int si[16];
  constexpr int U = 8;
  const int m = blockIdx.x, t = threadIdx.x;
  const float* row = y + (size_t)m * ldy;
  float bv = 0.f;
  int bi = -1;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0 && n < (1 << 28);
  const int n4 = vec ? n >> 2 : 0;
  if (n4 > 0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (uint32_t)n4 * 16u);
    for (int b = 0; b < n4; b += 1024 * U) {
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs, (uint32_t)(b + 1024 * u + t) * 16u, 0, 0));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pc = b + 1024 * u + t;
        if (pc < n4)
#pragma unroll
          for (int c = 0; c < 4; ++c) am_take(v[u][c], 4 * pc + c, bv, bi);
      }
    }
  }
  for (int i = 4 * n4 + t; i < n; i += 1024) am_take(row[i], i, bv, bi);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (oi >= 0 && am_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if ((t & 63) == 0) { sv[t >> 6] = bv; si[t >> 6] = bi; }
  __syncthreads();
  if (t == 0) {
    bv = sv[0];
    bi = si[0];
    for (int w = 1; w < 16; ++w)
      if (si[w] >= 0 && am_better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    idx[m] = bi;
    if (val) val[m] = bi >= 0 ? bv : __builtin_nanf("");
  }
}

// Split form: a row is cut into slices of kArgmaxSlice values, one 256-thread
// workgroup each (so a logits row streams through many CUs; one CU draws only
// a few tens of GB/s), whose best candidate goes to the workspace as one
// 64-bit key; a second launch takes the largest key of each row.  Key of value
// v at index i: the order-preserving bits of v (zeros of either sign alike) in
// the high word, ~i in the low one, so the larger key is the larger value and,
// among equal values, the lower index; 0 means no candidate (NaN or none).
__device__ __forceinline__ uint64_t am_key(float v, int i) {
  if (v != v) return 0ull;
  const uint32_t b = v == 0.f ? 0u : __float_as_uint(v);
  const uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)k << 32) | (uint32_t)~i;
}

__device__ __forceinline__ uint64_t am_wave_max(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

__global__ __launch_bounds__(256) void k_argmax_part(const float* __restrict__ y, int n, int ldy,
                                                     uint64_t* __restrict__ ws) {
  constexpr int PP = kArgmaxSlice / 4 / 256;   // 16-byte pieces per thread
  __shared__ uint64_t wbest[4];
  const int g = blockIdx.x, m = blockIdx.y, t = threadIdx.x;
  const float* row = y + (size_t)m * ldy;
  uint64_t best = 0;
  const int i0 = g * kArgmaxSlice;
  if ((reinterpret_cast<uintptr_t>(row) & 15) == 0 && n < (1 << 28)) {
    // pieces wholly inside the row; the one that crosses its end is read by value
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (uint32_t)n * 4u);
    f32x4 v[PP];
#pragma unroll
    for (int u = 0; u < PP; ++u)
      v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, (uint32_t)(i0 + 4 * (t + 256 * u)) * 4u, 0, 0));
#pragma unroll
    for (int u = 0; u < PP; ++u) {
      const int e0 = i0 + 4 * (t + 256 * u);
      if (e0 + 3 < n) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint64_t kk = am_key(v[u][c], e0 + c);
          best = kk > best ? kk : best;
        }
      } else {
        for (int e = e0; e < n; ++e) {
          const uint64_t kk = am_key(row[e], e);
          best = kk > best ? kk : best;
        }
      }
    }
  } else {
    const int i1 = min(n, i0 + kArgmaxSlice);
    for (int e = i0 + t; e < i1; e += 256) {
      const uint64_t kk = am_key(row[e], e);
      best = kk > best ? kk : best;
    }
  }
  best = am_wave_max(best);
  if ((t & 63) == 0) wbest[t >> 6] = best;
  __syncthreads();
  if (t == 0) {
    uint64_t b = wbest[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) b = wbest[w] > b ? wbest[w] : b;
    ws[(size_t)m * gridDim.x + g] = b;
  }
}

__global__ __launch_bounds__(64) void k_argmax_final(const float* __restrict__ y, int ldy, int parts,
                                                     const uint64_t* __restrict__ ws,
                                                     int32_t* __restrict__ idx, float* __restrict__ val) {
  const int m = blockIdx.x, lane = threadIdx.x;
  uint64_t best = 0;
  for (int g = lane; g < parts; g += 64) {
    const uint64_t kk = ws[(size_t)m * parts + g];
    best = kk > best ? kk : best;
  }
  best = am_wave_max(best);
  if (lane == 0) {
    const int i = best ? (int)~(uint32_t)best : -1;
    idx[m] = i;
    if (val) val[m] = i >= 0 ? y[(size_t)m * ldy + i] : __builtin_nanf("");
  }
}

hipError_t launch_argmax(const float* y, int n, int ldy, int M, int32_t* idx, float* val, void* ws,
                         hipStream_t s) {
  if (!ws) {
    hipLaunchKernelGGL(k_argmax, dim3(M), dim3(1024), 0, s, y, n, ldy, idx, val);
    return hipGetLastError();
  }
  const int parts = argmax_parts(n);
  hipLaunchKernelGGL(k_argmax_part, dim3(parts, M), dim3(256), 0, s, y, n, ldy, static_cast<uint64_t*>(ws));
  hipLaunchKernelGGL(k_argmax_final, dim3(M), dim3(64), 0, s, y, ldy, parts, static_cast<const uint64_t*>(ws),
                     idx, val);
  return hipGetLastError();
}

}  // namespace q4nx
