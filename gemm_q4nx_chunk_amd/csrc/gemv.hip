// Q4NX dequant-GEMV kernels for gfx950: y[m] = W x[m] for M <= 8 activation rows.
//
// Decode reads every weight once per token and does two flops with it, so the
// kernel is bound by HBM bandwidth (Strata article, section 1: decode speed is
// set by the bytes of weights read per token).  The design keeps the weight
// stream as wide 16-byte nontemporal loads of whole chunks, keeps x in
// registers, unpacks and scales in registers, and leaves the ALU work per
// weight small enough to hide under the stream.
//
// Work split: a workgroup of WAVES waves (4 for launches with many tile rows,
// 16 for small ones, where latency rather than bandwidth sets the time) owns
// WAVES/ks tile rows; the ks waves of one tile row take contiguous runs of its
// chunks, and their partial row sums meet in LDS, where one pass adds them in
// wave order.  No atomics: the result bits do not depend on timing.
#include "gemv_core.h"

namespace q4nx {

template <int KIND, int M, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_q4(const GemvBatch b) {
  constexpr int CB = ChunkBytes<KIND>::value;
  constexpr int D = WAVES == 4 ? Q4Depth<M>::value : (M == 1 ? 2 : 1);
  __shared__ float red[WAVES][32][M];
  const GemvJob& J = b.job[find_job(b, blockIdx.x)];
  const int ks = J.ks, rpw = WAVES / ks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = wave / ks, part = wave % ks;
  const int tr0 = (blockIdx.x - J.wg_begin) * rpw;
  const int tr = tr0 + slot;
  const int g = lane & 7;

  float acc[4][M];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;

  if (tr < J.TR) {
    const int c0 = part * J.TC / ks, c1 = (part + 1) * J.TC / ks;
    const uint16_t* xrow[M];
#pragma unroll
    for (int m = 0; m < M; ++m) xrow[m] = J.x + (size_t)m * J.ldx;
    q4_row_partial<KIND, M, D>(J.w + (size_t)tr * J.TC * CB, c0, c1, xrow, lane, acc);
  }

  q4_lane_reduce<M>(acc);
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave][8 * i + (lane >> 3)][m] = acc[i][m];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < rpw * 32 * M; idx += 64 * WAVES) {
    const int s = idx / (32 * M), rem = idx - s * 32 * M;
    const int r = rem / M, m = rem - r * M;
    const int t = tr0 + s;
    if (t < J.TR) {
      float v = 0.f;
      for (int p = 0; p < ks; ++p) v += red[s * ks + p][r][m];
      J.y[(size_t)m * J.ldy + 32 * t + r] = v;
    }
  }
}

template <int KIND, int M, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_q8(const GemvBatch b) {
  constexpr int CB = 8704;
  __shared__ float red[WAVES][32][M];
  const GemvJob& J = b.job[find_job(b, blockIdx.x)];
  const int ks = J.ks, rpw = WAVES / ks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = wave / ks, part_id = wave % ks;
  const int tr0 = (blockIdx.x - J.wg_begin) * rpw;
  const int tr = tr0 + slot;
  const int h = (lane >> 2) & 1;

  float acc[16][M];
#pragma unroll
  for (int r = 0; r < 16; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  if (tr < J.TR) {
    const int c0 = part_id * J.TC / ks, c1 = (part_id + 1) * J.TC / ks;
    q8_row_partial<KIND, M>(J.w + (size_t)tr * J.TC * CB, c0, c1, J.x, J.ldx, lane, acc);
  }
  q8_lane_reduce<M>(acc);
  if ((lane & ~4) == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave][16 * h + r][m] = acc[r][m];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < rpw * 32 * M; idx += 64 * WAVES) {
    const int s = idx / (32 * M), rem = idx - s * 32 * M;
    const int r = rem / M, m = rem - r * M;
    const int t = tr0 + s;
    if (t < J.TR) {
      float v = 0.f;
      for (int p = 0; p < ks; ++p) v += red[s * ks + p][r][m];
      J.y[(size_t)m * J.ldy + 32 * t + r] = v;
    }
  }
}

// ===========================================================================
// launcher
// ===========================================================================
template <int KIND, int M, int WAVES>
static hipError_t launch_one(const GemvBatch& b, int n_wg, hipStream_t s) {
  if constexpr (KIND == KIND_Q4_1 || KIND == KIND_Q4_K)
    hipLaunchKernelGGL((k_gemv_q4<KIND, M, WAVES>), dim3(n_wg), dim3(64 * WAVES), 0, s, b);
  else
    hipLaunchKernelGGL((k_gemv_q8<KIND, M, WAVES>), dim3(n_wg), dim3(64 * WAVES), 0, s, b);
  return hipGetLastError();
}

template <int KIND, int WAVES>
static hipError_t launch_m(int M, const GemvBatch& b, int n_wg, hipStream_t s) {
  switch (M) {
    case 1: return launch_one<KIND, 1, WAVES>(b, n_wg, s);
    case 2: return launch_one<KIND, 2, WAVES>(b, n_wg, s);
    case 3: return launch_one<KIND, 3, WAVES>(b, n_wg, s);
    case 4: return launch_one<KIND, 4, WAVES>(b, n_wg, s);
    case 5: return launch_one<KIND, 5, WAVES>(b, n_wg, s);
    case 6: return launch_one<KIND, 6, WAVES>(b, n_wg, s);
    case 7: return launch_one<KIND, 7, WAVES>(b, n_wg, s);
    case 8: return launch_one<KIND, 8, WAVES>(b, n_wg, s);
  }
  return hipErrorInvalidValue;
}

template <int WAVES>
static hipError_t launch_w(int kind, int M, const GemvBatch& b, int n_wg, hipStream_t s) {
  switch (kind) {
    case KIND_Q4_1: return launch_m<KIND_Q4_1, WAVES>(M, b, n_wg, s);
    case KIND_Q4_K: return launch_m<KIND_Q4_K, WAVES>(M, b, n_wg, s);
    case KIND_Q8_A: return launch_m<KIND_Q8_A, WAVES>(M, b, n_wg, s);
    case KIND_Q8_B: return launch_m<KIND_Q8_B, WAVES>(M, b, n_wg, s);
  }
  return hipErrorInvalidValue;
}

template <int KIND>
static hipError_t launch_small(int M, const GemvBatch& b, int n_wg, hipStream_t s) {
  if (M == 1) return launch_one<KIND, 1, 16>(b, n_wg, s);
  if (M == 2) return launch_one<KIND, 2, 16>(b, n_wg, s);
  return hipErrorInvalidValue;
}

// 16-wave workgroups hold at most 128 registers per lane, so they are used
// for M <= 2 only.
hipError_t launch_gemv(int kind, int M, int waves, const GemvBatch& b, int n_wg, hipStream_t s) {
  if (waves == 4) return launch_w<4>(kind, M, b, n_wg, s);
  if (waves == 16 && M <= 2) {
    switch (kind) {
      case KIND_Q4_1: return launch_small<KIND_Q4_1>(M, b, n_wg, s);
      case KIND_Q4_K: return launch_small<KIND_Q4_K>(M, b, n_wg, s);
      case KIND_Q8_A: return launch_small<KIND_Q8_A>(M, b, n_wg, s);
      case KIND_Q8_B: return launch_small<KIND_Q8_B>(M, b, n_wg, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace q4nx
