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
// lower id among equals) by k rounds of a wave-wide selection; the weights are
// expf(z - max) / sum in fp32.
#include "q4nx_dev.h"

namespace q4nx {

constexpr int kRouterMaxE = 1024;
constexpr int kRouterMaxK = 16;

__device__ __forceinline__ bool rt_better(float v, int i, float bv, int bi) {
  return bi < 0 || v > bv || (v == bv && i < bi);
}

// Logits: workgroup (bx, by), one wave, takes router rows 2 bx and 2 bx + 1
// (held in registers) against tokens 8 by .. 8 by + 7, so the router weights
// stream through as many CUs as there are row pairs (a CU draws only a few
// tens of GB/s; one workgroup per token would pull them through one CU).
template <int DB>
__global__ __launch_bounds__(64) void k_router_logits(const uint16_t* __restrict__ R,
                                                      const uint16_t* __restrict__ X, int T, int E,
                                                      float* __restrict__ logits) {
  constexpr int D = 512 * DB;
  const int lane = threadIdx.x & 63;
  const int r0 = 2 * blockIdx.x;
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

// Picks and weights: one wave per token (4 tokens per workgroup).  Lane l
// holds logits l + 64 i (i < 16, E <= 1024) in registers; the max, the sum of
// expf(z - max) (each lane's terms in i order, then a fixed xor pattern over
// the lanes) and each of the k picks (the lane's best untaken candidate, then
// an xor-butterfly selection under the (value desc, id asc) order, which picks
// the same expert whatever the pairing) need no LDS and no barrier.
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int T, int E,
                                                     int k, int renorm, int32_t* __restrict__ ids,
                                                     float* __restrict__ p) {
  constexpr int EL = kRouterMaxE / 64;
  const int lane = threadIdx.x & 63;
  const int t = 4 * blockIdx.x + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[EL];
#pragma unroll
  for (int i = 0; i < EL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? logits[(size_t)t * E + e] : 0.f;
  }
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < EL; ++i)
    if (lane + 64 * i < E) m = fmaxf(m, v[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float sacc = 0.f;
#pragma unroll
  for (int i = 0; i < EL; ++i)
    if (lane + 64 * i < E) sacc += expf(v[i] - m);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sacc += __shfl_xor(sacc, off);

  uint32_t taken = 0;   // bit i: expert lane + 64 i already picked
  int my_id = -1;       // lane j < k: the j-th pick
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < EL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && rt_better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi >= 0 && rt_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi >= 0 && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      my_id = bi;
      my_v = bv;
    }
  }
  // weights: lane j < k holds pick j; the renormalising total is a fixed-order
  // sum of the k weights (lanes 0 .. k - 1 in order, via a broadcast loop)
  const float w = lane < k ? expf(my_v - m) / sacc : 0.f;
  float tot = 0.f;
  for (int j = 0; j < k; ++j) tot += __shfl(w, j);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    p[(size_t)t * k + lane] = renorm ? w / tot : w;
  }
}

hipError_t launch_moe_router(const uint16_t* R, const uint16_t* X, int T, int D, int E, int k,
                             int renorm, int32_t* ids, float* p, float* logits, hipStream_t s) {
  const dim3 g((E + 1) / 2, (T + 7) / 8), b(64);
  switch (D / 512) {
    case 1: hipLaunchKernelGGL((k_router_logits<1>), g, b, 0, s, R, X, T, E, logits); break;
    case 2: hipLaunchKernelGGL((k_router_logits<2>), g, b, 0, s, R, X, T, E, logits); break;
    case 4: hipLaunchKernelGGL((k_router_logits<4>), g, b, 0, s, R, X, T, E, logits); break;
    case 8: hipLaunchKernelGGL((k_router_logits<8>), g, b, 0, s, R, X, T, E, logits); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(k_router_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, renorm, ids, p);
  return hipGetLastError();
}

}  // namespace q4nx
