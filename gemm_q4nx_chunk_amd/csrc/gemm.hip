// Q4NX block GEMM for gfx950: Y[m] = W X[m] for a prompt block of M <= 64 rows.
//
// At 64 rows each 4-bit weight serves 128 flops, which is a dense contraction,
// so the products run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) with
// fp32 accumulation.  Each chunk is read from HBM once and dequantised once, in
// registers, to bf16 (round to nearest even) -- no bf16 copy of the weight is
// ever written.  Splitting the token rows over several weight passes would
// re-read the weights (Strata article, section 5.1, on the overlap attempt that
// lost speed by reading dense weights twice), so one pass takes all M rows.
//
// Workgroup: 4 waves, one tile row (32 outputs) each, the whole K.  The X
// columns of the current tile column (M x 256 bf16) sit in LDS, double
// buffered, shared by the 4 waves.
//
// k-slot assignment: in MFMA step s (16 per tile column) lane (h = lane/32,
// n = lane%32) feeds the 8 products k = 128h + 8s + 0..7 -- for the B operand
// (weights) of output row n, for the A operand (X) of token row n.  A and B
// use the same slots, so the order of k inside a step does not change the sum.
// With this order a lane's weights are one contiguous 64-byte run of its row's
// codes, and their (scale, zero) records one 16-byte load.
#include "q4nx_dev.h"

namespace q4nx {

constexpr int kXs = 264;   // LDS row stride of the X tile in bf16 (256 + 8: 4-bank skew per row)

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

__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s, float z) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // codes k = 0, 2, 4, 6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // codes k = 1, 3, 5, 7
  bf16x8 b;
  b[0] = (__bf16)fmaf((float)(lo & 0xFFu), s, z);
  b[1] = (__bf16)fmaf((float)(hi & 0xFFu), s, z);
  b[2] = (__bf16)fmaf((float)((lo >> 8) & 0xFFu), s, z);
  b[3] = (__bf16)fmaf((float)((hi >> 8) & 0xFFu), s, z);
  b[4] = (__bf16)fmaf((float)((lo >> 16) & 0xFFu), s, z);
  b[5] = (__bf16)fmaf((float)((hi >> 16) & 0xFFu), s, z);
  b[6] = (__bf16)fmaf((float)(lo >> 24), s, z);
  b[7] = (__bf16)fmaf((float)(hi >> 24), s, z);
  return b;
}

template <int KIND>
__global__ __launch_bounds__(256) void k_gemm_q4(const uint8_t* __restrict__ w,
                                                 const uint16_t* __restrict__ X,
                                                 float* __restrict__ Y, int TR, int TC, int M) {
  constexpr int CB = ChunkBytes<KIND>::value;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][64 * kXs];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, n = lane & 31;
  const int tr = blockIdx.x * 4 + wave;
  const bool active = tr < TR;
  const int K = TC * 256, N = TR * 32;
  const bool two = M > 32;
  const uint8_t* rowp = w + (size_t)(active ? tr : 0) * TC * CB;

  // X tile loader: 64 rows x 32 pieces of 16 B, 8 pieces per thread.
  u32x4 xr[8];
  auto xload = [&](int tc) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int piece = tid + 256 * p, row = piece >> 5, c16 = piece & 31;
      xr[p] = row < M ? load16(X + (size_t)row * K + tc * 256 + c16 * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto xstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int piece = tid + 256 * p, row = piece >> 5, c16 = piece & 31;
      *reinterpret_cast<u32x4*>(&xs[buf][row * kXs + c16 * 8]) = xr[p];
    }
  };

  f32x16 acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) { acc0[v] = 0.f; acc1[v] = 0.f; }

  GemmChunk<KIND> cur, nxt;
  xload(0);
  xstore(0);
  if (active) gemm_load<KIND>(rowp, n, h, cur);

  for (int tc = 0; tc < TC; ++tc) {
    __syncthreads();                       // X tile tc is in xs[tc & 1]
    const bool more = tc + 1 < TC;
    if (more) {
      xload(tc + 1);
      if (active) gemm_load<KIND>(rowp + (size_t)(tc + 1) * CB, n, h, nxt);
    }
    if (active) {
      const uint16_t* xb = xs[tc & 1] + n * kXs + 128 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float s, z;
        group_sz<KIND>(cur, q, s, z);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int st = 4 * q + e;
          const bf16x8 B = dequant8(cur.q[q][e], s, z);
          const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(xb + 8 * st);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B, acc0, 0, 0, 0);
          if (two) {
            const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(xb + 32 * kXs + 8 * st);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B, acc1, 0, 0, 0);
          }
        }
      }
    }
    if (more) {
      xstore((tc + 1) & 1);                // that buffer was last read before this barrier
      cur = nxt;
    }
  }

  if (active) {
    // 32x32 accumulator: register v of lane holds token row 8*(v/4) + 4*h + v%4, output column n.
    float* yc = Y + 32 * tr + n;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * h + (v & 3);
      if (m < M) yc[(size_t)m * N] = acc0[v];
      if (two && m + 32 < M) yc[(size_t)(m + 32) * N] = acc1[v];
    }
  }
}

hipError_t launch_gemm(int kind, const uint8_t* w, const uint16_t* X, float* Y, int TR, int TC,
                       int M, hipStream_t s) {
  const dim3 grid((TR + 3) / 4), block(256);
  if (kind == KIND_Q4_1)
    hipLaunchKernelGGL(k_gemm_q4<KIND_Q4_1>, grid, block, 0, s, w, X, Y, TR, TC, M);
  else if (kind == KIND_Q4_K)
    hipLaunchKernelGGL(k_gemm_q4<KIND_Q4_K>, grid, block, 0, s, w, X, Y, TR, TC, M);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace q4nx
