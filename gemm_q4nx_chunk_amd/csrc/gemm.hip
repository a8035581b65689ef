// Q4NX block GEMM for gfx950: Y[m] = W X[m] for a prompt block of M <= 64 rows.
//
// At 64 rows each 4-bit weight serves 128 flops, a dense contraction, so the
// products run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation.  Each chunk is read from HBM once and dequantised once, in
// registers, to bf16 (round to nearest even); no bf16 copy of a weight is ever
// written.  All M rows share one pass over the weights: splitting the token
// rows over several passes would read the weights again (Strata article,
// section 5.1, on an overlap attempt that lost speed by reading dense weights
// twice).
//
// Workgroup: 8 waves, one tile row (32 outputs) each, over a range of tile
// columns.  The X columns of the current tile column (M x 256 bf16) sit in
// LDS, double buffered, shared by the 8 waves.  When the tile rows alone give
// too few workgroups to keep every CU's ALUs busy with dequantisation, K is
// split over S workgroups; each writes its fp32 partial tile to the workspace
// and the last of the S to arrive adds the parts in part order (no atomics on
// data, so the result bits do not depend on timing).
//
// Dequantisation: a 4-bit code c placed in an fp16 mantissa under the exponent
// of 1024 reads as 1024 + c (low nibble) or 1024 + 16c (high nibble of a
// byte), both exact, so one v_and_or makes two weights' codes into an fp16
// pair and one v_fma_mix_f32 per weight forms c*s + z in fp32:
//   w = (1024 + c) * s + (z - 1024 s) = (1024 + 16c) * (s/16) + (z - 64 s).
// v_cvt_pk_bf16_f32 then rounds two weights to the bf16 pair the MFMA takes.
// z - 1024 s carries one fp32 rounding (about 2^-24 of 1024 s), far below the
// bf16 rounding of the weight itself (2^-8 of its size).
//
// k-slot assignment: in MFMA step s (16 per tile column) lane (h = lane/32,
// n = lane%32) feeds the 8 products k = 128h + 8s + 0..7 -- for the B operand
// (weights) of output row n, for the A operand (X) of token row n.  A and B
// use the same slots, so the order of k inside a step does not change the sum.
// With this order a lane's weights are one contiguous 64-byte run of its row's
// codes, and their scale records one 16-byte load.
#include "gemm_args.h"
#include "q4nx_dev.h"

namespace q4nx {

constexpr int kXs = 264;   // LDS row stride of the X tile in bf16 (256 + 8: 4-bank skew per row)
constexpr int kGemmWaves = 8;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int KIND>
struct GemmChunk {
  u32x4 q[4];   // codes k = 128h + 32q + 0..31 of row n
  u32x4 meta;   // q4_1: (scale, zero) of groups 4h..4h+3; Q4_K: .x,.y = (sc,mn) bytes, .z = (S, M)
};

template <int KIND>
__device__ __forceinline__ void gemm_load(const uint8_t* __restrict__ ck, int n, int h, GemmChunk<KIND>& c) {
#pragma unroll
  for (int q = 0; q < 4; ++q) c.q[q] = load_nt16(ck + 128 * n + 64 * h + 16 * q);
  if constexpr (KIND == KIND_Q4_1) {
    c.meta = *reinterpret_cast<const u32x4*>(ck + 4096 + 32 * n + 16 * h);
  } else {
    const u32x2 scmn = *reinterpret_cast<const u32x2*>(ck + 4096 + 16 * n + 8 * h);
    c.meta.x = scmn.x;
    c.meta.y = scmn.y;
    c.meta.z = *reinterpret_cast<const uint32_t*>(ck + 4608 + 4 * n);
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
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s, float z_lo, float s16, float z_hi,
                                           uint32_t kMaskLo, uint32_t kMaskHi, uint32_t kMagic) {
  const uint32_t w8 = w >> 8;
  const f16x2 p0 = __builtin_bit_cast(f16x2, (w & kMaskLo) | kMagic);    // (c0, c4)
  const f16x2 p1 = __builtin_bit_cast(f16x2, (w & kMaskHi) | kMagic);    // (16 c1, 16 c5)
  const f16x2 p2 = __builtin_bit_cast(f16x2, (w8 & kMaskLo) | kMagic);   // (c2, c6)
  const f16x2 p3 = __builtin_bit_cast(f16x2, (w8 & kMaskHi) | kMagic);   // (16 c3, 16 c7)
  bf16x8 b;
  b[0] = (__bf16)fmaf((float)p0.x, s, z_lo);
  b[1] = (__bf16)fmaf((float)p1.x, s16, z_hi);
  b[2] = (__bf16)fmaf((float)p2.x, s, z_lo);
  b[3] = (__bf16)fmaf((float)p3.x, s16, z_hi);
  b[4] = (__bf16)fmaf((float)p0.y, s, z_lo);
  b[5] = (__bf16)fmaf((float)p1.y, s16, z_hi);
  b[6] = (__bf16)fmaf((float)p2.y, s, z_lo);
  b[7] = (__bf16)fmaf((float)p3.y, s16, z_hi);
  return b;
}

template <int KIND, bool TWO>
__global__ __launch_bounds__(64 * kGemmWaves) void k_gemm_q4(GemmArgs a) {
  constexpr int CB = ChunkBytes<KIND>::value;
  constexpr int NT = 64 * kGemmWaves;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][64 * kXs];
  __shared__ uint32_t s_old;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, n = lane & 31;
  const int nb = blockIdx.x, part = blockIdx.y;
  const int tr = nb * kGemmWaves + wave;
  const bool active = tr < a.TR;
  const int K = a.TC * 256, N = a.TR * 32, M = a.M;
  const int tc0 = part * a.TC / a.S, tc1 = (part + 1) * a.TC / a.S;
  const uint8_t* rowp = a.w + (size_t)(active ? tr : 0) * a.TC * CB;

  uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  asm volatile("" : "+s"(kMaskLo));
  asm volatile("" : "+s"(kMaskHi));
  asm volatile("" : "+v"(kMagic));

  // X tile loader: 64 rows x 32 pieces of 16 B over NT threads.
  constexpr int XP = 64 * 32 / NT;
  u32x4 xr[XP];
  auto xload = [&](int tc) {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int piece = tid + NT * p, row = piece >> 5, c16 = piece & 31;
      xr[p] = row < M ? load16(a.X + (size_t)row * K + tc * 256 + c16 * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto xstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int piece = tid + NT * p, row = piece >> 5, c16 = piece & 31;
      *reinterpret_cast<u32x4*>(&xs[buf][row * kXs + c16 * 8]) = xr[p];
    }
  };

  f32x16 acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) { acc0[v] = 0.f; acc1[v] = 0.f; }

  GemmChunk<KIND> cur, nxt;
  xload(tc0);
  xstore(0);
  if (active) gemm_load<KIND>(rowp + (size_t)tc0 * CB, n, h, cur);

  for (int tc = tc0; tc < tc1; ++tc) {
    const int buf = (tc - tc0) & 1;
    __syncthreads();                       // X tile tc is in xs[buf]
    const bool more = tc + 1 < tc1;
    if (more) {
      xload(tc + 1);
      if (active) gemm_load<KIND>(rowp + (size_t)(tc + 1) * CB, n, h, nxt);
    }
    if (active) {
      const uint16_t* xb = xs[buf] + n * kXs + 128 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float s, z;
        group_sz<KIND>(cur, q, s, z);
        const float z_lo = fmaf(-1024.f, s, z), s16 = s * 0.0625f, z_hi = fmaf(-64.f, s, z);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int st = 4 * q + e;
          const bf16x8 B = dequant8(cur.q[q][e], s, z_lo, s16, z_hi, kMaskLo, kMaskHi, kMagic);
          const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(xb + 8 * st);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B, acc0, 0, 0, 0);
          if constexpr (TWO) {
            const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(xb + 32 * kXs + 8 * st);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B, acc1, 0, 0, 0);
          }
        }
      }
    }
    if (more) {
      xstore((tc + 1 - tc0) & 1);          // that buffer was last read before this barrier
      cur = nxt;
    }
  }

  // 32x32 accumulator: register v of lane holds token row 8*(v/4) + 4*h + v%4, output column n.
  if (a.S == 1) {
    if (active) {
      float* yc = a.Y + 32 * tr + n;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < M) yc[(size_t)m * N] = acc0[v];
        if (TWO && m + 32 < M) yc[(size_t)(m + 32) * N] = acc1[v];
      }
    }
    return;
  }
  // split K: partial tile [M][8 tile rows x 32] of this part, then the last part adds them
  const int ncol = kGemmWaves * 32;
  float* pt = a.partial + ((size_t)nb * a.S + part) * 64 * ncol;
  {
    float* pc = pt + wave * 32 + n;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * h + (v & 3);
      if (m < M) st_coherent(pc + (size_t)m * ncol, acc0[v]);
      if (TWO && m + 32 < M) st_coherent(pc + (size_t)(m + 32) * ncol, acc1[v]);
    }
  }
  wait_stores();
  __syncthreads();
  if (tid == 0)
    s_old = __hip_atomic_fetch_add(a.cnt + nb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_old != (uint32_t)a.S - 1) return;
  const float* p0 = a.partial + (size_t)nb * a.S * 64 * ncol;
  for (int idx = tid; idx < M * ncol; idx += NT) {
    const int m = idx / ncol, c = idx - m * ncol;
    const int col = nb * ncol + c;
    float v = 0.f;
    for (int p = 0; p < a.S; ++p) v += ld_coherent(p0 + (size_t)p * 64 * ncol + idx);
    if (col < N) a.Y[(size_t)m * N + col] = v;
  }
  if (tid == 0) __hip_atomic_store(a.cnt + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_gemm(int kind, const GemmArgs& a, hipStream_t s) {
  const dim3 grid((a.TR + kGemmWaves - 1) / kGemmWaves, a.S), block(64 * kGemmWaves);
  const bool two = a.M > 32;
  if (kind == KIND_Q4_1) {
    if (two) hipLaunchKernelGGL((k_gemm_q4<KIND_Q4_1, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm_q4<KIND_Q4_1, false>), grid, block, 0, s, a);
  } else if (kind == KIND_Q4_K) {
    if (two) hipLaunchKernelGGL((k_gemm_q4<KIND_Q4_K, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm_q4<KIND_Q4_K, false>), grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace q4nx
