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

// Order-preserving 32-bit key of a logit: larger logits give larger keys;
// NaN maps below every number, so it is never picked before a number.
__device__ __forceinline__ uint32_t rt_key(float v) {
  const uint32_t b = __float_as_uint(v);
  if (v != v) return 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The logit of a key (a NaN for key 0).
__device__ __forceinline__ float rt_logit(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// A candidate as one 64-bit value, key << 32 | ~id: the larger value is the
// better candidate (the larger key, then the lower id), and 0 is "none".
// Takes the larger of the lane's value and its partner's within rows of 16
// lanes, by DPP on both halves.
__device__ __forceinline__ uint64_t rt_max_step(uint64_t v, int ctrl_sel) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  uint32_t olo, ohi;
  switch (ctrl_sel) {   // constant after inlining
    case 0: olo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, false); ohi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: olo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, false); ohi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: olo = __builtin_amdgcn_mov_dpp(lo, 0x141, 0xF, 0xF, false); ohi = __builtin_amdgcn_mov_dpp(hi, 0x141, 0xF, 0xF, false); break; // row_half_mirror
    default: olo = __builtin_amdgcn_mov_dpp(lo, 0x140, 0xF, 0xF, false); ohi = __builtin_amdgcn_mov_dpp(hi, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t rt_readlane(uint64_t v, int l) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((uint32_t)v, l);   // no sign extension
  return ((uint64_t)hi << 32) | lo;
}

// Picks and weights: one wave per token (4 tokens per workgroup).  Lane l
// holds logits l + 64 i (i < EL, E <= 64 EL) in registers.  The max and the
// sum of expf(z - max) (each lane's terms in i order, then a fixed pattern:
// pairs, quads, eights and rows of 16 within a row by DPP, then rows 0..3 in
// order) and each of the k picks (the lane's best untaken candidate, the best
// of each row by DPP, then of the 4 rows) need no LDS and no barrier; a pick
// is a maximum under a total order, so it does not depend on the pairing.
template <int EL>   // logits per lane: E <= 64 EL
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int T, int E,
                                                     int k, int renorm, int32_t* __restrict__ ids,
                                                     float* __restrict__ p) {
  const int lane = threadIdx.x & 63;
  const int t = 4 * blockIdx.x + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  if (t >= T) return;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(logits + (size_t)t * E, (uint32_t)E * 4);
  float v[EL];
#pragma unroll
  for (int i = 0; i < EL; ++i)   // past E: zero, and never a candidate
    v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(lane + 64 * i) * 4, 0, 0));
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < EL; ++i) m = fmaxf(m, lane + 64 * i < E ? v[i] : -__builtin_inff());
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, false)));
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(m), 0x141, 0xF, 0xF, false)));
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(m), 0x140, 0xF, 0xF, false)));
  m = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(m), 0)),
                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(m), 16))),
            fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(m), 32)),
                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(m), 48))));
  float sacc = 0.f;
#pragma unroll
  for (int i = 0; i < EL; ++i) sacc += expf(lane + 64 * i < E ? v[i] - m : -__builtin_inff());   // exp(-inf) = 0
  sacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(sacc), 0xB1, 0xF, 0xF, false));
  sacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(sacc), 0x4E, 0xF, 0xF, false));
  sacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(sacc), 0x141, 0xF, 0xF, false));
  sacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(sacc), 0x140, 0xF, 0xF, false));
  const float ssum = ((__builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(sacc), 0)) +
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(sacc), 16))) +
                      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(sacc), 32))) +
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(sacc), 48));

  uint64_t cand[EL];   // the lane's untaken candidates (0 once taken or past E)
#pragma unroll
  for (int i = 0; i < EL; ++i) {
    const int e = lane + 64 * i;
    cand[i] = e < E ? ((uint64_t)rt_key(v[i]) << 32) | (uint32_t)~e : 0ull;
  }
  int my_id = -1;       // lane j < k: the j-th pick
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EL; ++i) best = cand[i] > best ? cand[i] : best;
#pragma unroll
    for (int c = 0; c < 4; ++c) best = rt_max_step(best, c);
    // rows 0..3: the best of the four row leaders (uniform)
    uint64_t w = rt_readlane(best, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
      const uint64_t o = rt_readlane(best, 16 * r);
      w = o > w ? o : w;
    }
    const int pick = (int)~(uint32_t)w;
    const bool mine = (pick & 63) == lane;
#pragma unroll
    for (int i = 0; i < EL; ++i)
      if (mine && (pick >> 6) == i) cand[i] = 0;
    if (lane == j) {
      my_id = pick;
      my_v = rt_logit((uint32_t)(w >> 32));
    }
  }
  // the weights: lane j < k holds pick j
  const float w = lane < k ? expf(my_v - m) / ssum : 0.f;
  float tot = 0.f;
  for (int j = 0; j < k; ++j) tot += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(w), j));
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
  const dim3 gt((T + 3) / 4), bt(256);
  if (E <= 256) hipLaunchKernelGGL(k_router_topk<4>, gt, bt, 0, s, logits, T, E, k, renorm, ids, p);
  else if (E <= 512) hipLaunchKernelGGL(k_router_topk<8>, gt, bt, 0, s, logits, T, E, k, renorm, ids, p);
  else hipLaunchKernelGGL(k_router_topk<kRouterMaxE / 64>, gt, bt, 0, s, logits, T, E, k, renorm, ids, p);
  return hipGetLastError();
}

}  // namespace q4nx
