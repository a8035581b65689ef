// MoE router on the GPU: logits, softmax, top-k, weights.
//
// The router (Strata article, section 2 "target model": per token it picks 10
// of the 512 routed experts, weighted by their softmax probabilities, and the
// picked weights are rescaled to sum to one; section 4.3 "tail skip" keeps
// them unrescaled) is the step right before the routed-expert layer.  Here it
// runs on the device, so ids and weights feed q4nx_moe_experts without a
// host round trip.
//
// Two kernels.  Router weights are bf16 [E][D] (row e contiguous); lane l of
// a wave holds columns 512 b + 8 l .. +7 of each 512-column block b, forms
// v_dot2_f32_bf16 products in a fixed order and the 64 lanes meet in a
// fixed-order xor reduction, so a logit's bits depend only on the data.  The
// top-k is then taken per token on those fp32 logits (the larger first, the
// lower id among equals) by k rounds of a fixed-order workgroup reduction;
// the weights are expf(z - max) / sum in fp32.
#include "q4nx_dev.h"

namespace q4nx {

constexpr int kRouterMaxE = 1024;
constexpr int kRouterMaxK = 16;

__device__ __forceinline__ bool rt_better(float v, int i, float bv, int bi) {
  return bi < 0 || v > bv || (v == bv && i < bi);
}

// Logits: workgroup (bx, by) takes router rows 8 bx .. 8 bx + 7 (two per
// wave, held in registers) against tokens 8 by .. 8 by + 7, so the router
// weights stream through many CUs at once (one workgroup per token would
// pull them through a single CU).
template <int DB>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ R,
                                                       const uint16_t* __restrict__ X, int T, int E,
                                                       float* __restrict__ logits) {
  constexpr int D = 512 * DB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = 8 * blockIdx.x + 2 * wave;
  u32x4 ra[DB], rb[DB];
  const int ea = r0 < E ? r0 : E - 1, eb = r0 + 1 < E ? r0 + 1 : E - 1;
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    ra[b] = load16(R + (size_t)ea * D + 512 * b + 8 * lane);
    rb[b] = load16(R + (size_t)eb * D + 512 * b + 8 * lane);
  }
  for (int tk = 0; tk < 8; ++tk) {
    const int t = 8 * blockIdx.y + tk;
    if (t >= T) break;
    u32x4 xv[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) xv[b] = load16(X + (size_t)t * D + 512 * b + 8 * lane);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a0 = dot2bf16(ra[b][i], xv[b][i], a0);
        a1 = dot2bf16(rb[b][i], xv[b][i], a1);
      }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      a0 += __shfl_xor(a0, off);
      a1 += __shfl_xor(a1, off);
    }
    if (lane == 0) {
      if (r0 < E) logits[(size_t)t * E + r0] = a0;
      if (r0 + 1 < E) logits[(size_t)t * E + r0 + 1] = a1;
    }
  }
}

// Picks and weights: one workgroup per token over its E logits.
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int E, int k,
                                                     int renorm, int32_t* __restrict__ ids,
                                                     float* __restrict__ p) {
  __shared__ float lg[kRouterMaxE];
  __shared__ uint8_t taken[kRouterMaxE];
  __shared__ float rv[256];
  __shared__ int ri[256];
  __shared__ int sel[kRouterMaxK];
  const int t = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) {
    lg[e] = logits[(size_t)t * E + e];
    taken[e] = 0;
  }
  __syncthreads();

  // max and sum of expf(z - max), each a fixed-order reduction
  float m = -__builtin_inff();
  for (int e = tid; e < E; e += 256) m = fmaxf(m, lg[e]);
  rv[tid] = m;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) rv[tid] = fmaxf(rv[tid], rv[tid + h]);
    __syncthreads();
  }
  const float mx = rv[0];
  __syncthreads();
  float sacc = 0.f;
  for (int e = tid; e < E; e += 256) sacc += expf(lg[e] - mx);
  rv[tid] = sacc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) rv[tid] += rv[tid + h];
    __syncthreads();
  }
  const float ssum = rv[0];
  __syncthreads();

  // top-k: k rounds of a (value desc, index asc) reduction over untaken experts
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = -1;
    for (int e = tid; e < E; e += 256)
      if (!taken[e] && rt_better(lg[e], e, bv, bi)) { bv = lg[e]; bi = e; }
    rv[tid] = bv;
    ri[tid] = bi;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
      if (tid < h && ri[tid + h] >= 0 && rt_better(rv[tid + h], ri[tid + h], rv[tid], ri[tid])) {
        rv[tid] = rv[tid + h];
        ri[tid] = ri[tid + h];
      }
      __syncthreads();
    }
    if (tid == 0) {
      sel[j] = ri[0];
      taken[ri[0]] = 1;
    }
    __syncthreads();
  }
  if (tid == 0) {
    float w[kRouterMaxK];
    float tot = 0.f;
    for (int j = 0; j < k; ++j) {
      w[j] = expf(lg[sel[j]] - mx) / ssum;
      tot += w[j];
    }
    for (int j = 0; j < k; ++j) {
      ids[(size_t)t * k + j] = sel[j];
      p[(size_t)t * k + j] = renorm ? w[j] / tot : w[j];
    }
  }
}

hipError_t launch_moe_router(const uint16_t* R, const uint16_t* X, int T, int D, int E, int k,
                             int renorm, int32_t* ids, float* p, float* logits, hipStream_t s) {
  const dim3 g((E + 7) / 8, (T + 7) / 8), b(256);
  switch (D / 512) {
    case 1: hipLaunchKernelGGL((k_router_logits<1>), g, b, 0, s, R, X, T, E, logits); break;
    case 2: hipLaunchKernelGGL((k_router_logits<2>), g, b, 0, s, R, X, T, E, logits); break;
    case 4: hipLaunchKernelGGL((k_router_logits<4>), g, b, 0, s, R, X, T, E, logits); break;
    case 8: hipLaunchKernelGGL((k_router_logits<8>), g, b, 0, s, R, X, T, E, logits); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(k_router_topk, dim3(T), b, 0, s, logits, E, k, renorm, ids, p);
  return hipGetLastError();
}

}  // namespace q4nx
