// Persistent multi-phase GEMV plan: a whole decode step in one launch.
//
// A decode step is a chain of dependent GEMV groups (per layer: q|k|v, o,
// gate|up, down, then the lm_head).  Launched one group at a time, each short
// kernel pays its start, its first memory latency and its drain, and the
// weight stream stops between kernels.  The Strata article (section 3.2)
// records the same lesson for its own engine, which runs a whole 48-layer pass
// as one captured graph so that no step waits on the driver.
// Here the step is one persistent kernel instead:
//
//  * Work is cut into workgroup units of one tile row (32 outputs) and at most
//    4 x CPW chunks; a tile row whose K needs more chunks is split into S
//    parts, written as fp32 partial rows and added, in part order, by the last
//    part to arrive.
//  * Units are numbered phase by phase and dealt round-robin to a grid sized to
//    stay resident; each workgroup walks its units in increasing order.
//  * A unit issues its weight loads first and only then waits until every
//    tile row of the previous phase is written, so the weight stream of the
//    next phase overlaps the tail of the current one while the dependency is
//    still honoured.  Outputs and partial rows are published with device-scope
//    (sc1) stores, the wave waits for their completion, and only then does one
//    thread move the counter; consumers poll the counter and read activations
//    and partials with device-scope loads.  Nothing here writes back or
//    invalidates a whole L2 (an agent-scope fence would do both, per unit).
//
// The smallest unfinished unit only ever waits on units before it, so the
// schedule cannot deadlock while the grid is resident.  Every wait is also
// bounded: past the spin limit the kernel raises an error flag and moves on
// (later waits return at once), so a misuse ends in an error, never a hang.
// The last workgroup to leave resets the phase counters for the next run.
#include "gemv_core.h"
#include "plan_args.h"

namespace q4nx {

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_at_least(const uint32_t* p, uint32_t need, int limit,
                                              uint32_t* err) {
  if (ld_relaxed(err)) return;
  int it = 0;
  while (ld_relaxed(p) < need) {
    __builtin_amdgcn_s_sleep(2);
    if (++it > limit) {
      __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
}

template <int KIND, int M>
__global__ __launch_bounds__(256) void k_plan(PlanArgs a) {
  constexpr bool kQ8 = KIND == KIND_Q8_A || KIND == KIND_Q8_B;
  constexpr int CB = ChunkBytes<KIND>::value;
  constexpr int CPW = PlanCpw<KIND>::value;
  __shared__ float red[4][32][M];
  __shared__ uint32_t s_old;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const Q4Consts kc = q4_consts();
  int confirmed = 0;   // every phase below this one is known to be finished

  for (int u = blockIdx.x; u < a.n_units; u += gridDim.x) {
    const PlanJob J = a.jobs[a.unit_job[u]];
    const int local = u - J.unit0;
    const int tr = local / J.S, s = local - tr * J.S;
    const int uc0 = s * J.TC / J.S, n = (s + 1) * J.TC / J.S - uc0;
    const int c0 = uc0 + wave * n / 4, nc = uc0 + (wave + 1) * n / 4 - c0;   // nc <= CPW
    const uint8_t* row = J.w + (size_t)tr * J.TC * CB;

    // weight loads first ...
    typename std::conditional<kQ8, Q8Chunk, Q4Chunk<KIND>>::type ch[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      if (i < nc) {
        if constexpr (kQ8) q8_load<KIND>(row + (size_t)(c0 + i) * CB, lane, ch[i]);
        else q4_load<KIND>(row + (size_t)(c0 + i) * CB, lane, ch[i]);
      }
    }
    // ... then the dependency on the previous phase.  Its outputs were stored
    // at device scope before its counters moved; x is read at device scope too.
    if (J.phase > confirmed) {
      if (threadIdx.x == 0)
        wait_at_least(a.done + J.phase - 1, a.need[J.phase - 1], a.spin_limit, a.ctl + 1);
      __syncthreads();
      confirmed = J.phase;
    }
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(J.x, (uint32_t)(2 * M * J.ldx));

    if constexpr (kQ8) {
      float acc[16][M];
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        if (i < nc) {
          Q8XRaw<M> xr;
#pragma unroll
          for (int m = 0; m < M; ++m)
            xr.v[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    xrs, 2 * (m * J.ldx + q8_xcol(lane, c0 + i)), 0,
                                                    kCpolSc1));
          q8_compute_raw<M>(ch[i], xr, acc);
        }
      }
      q8_lane_reduce<M>(acc);
      if ((lane & ~4) == 0) {
        const int h = (lane >> 2) & 1;
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int m = 0; m < M; ++m) red[wave][16 * h + r][m] = acc[r][m];
      }
    } else {
      float acc[4][M];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[i][m] = 0.f;
      const int g = lane & 7;
      int xoff[M];
#pragma unroll
      for (int m = 0; m < M; ++m) xoff[m] = 2 * (m * J.ldx + 32 * g);
      // all of the unit's activation loads at once: one round trip, not one per chunk
      XRaw<M> xr[CPW];
#pragma unroll
      for (int i = 0; i < CPW; ++i)
        x_raw_coherent<M>(xrs, xoff, 256 * (c0 + (i < nc ? i : 0)), xr[i]);
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        if (i < nc) {
          XRecB<M> xp;   // activations per lane and chunk: bf16 records
          x_records_b<M>(xr[i], xp);
          q4_compute_b<KIND, M, 1>(ch[i], xp, kc, acc);
        }
      }
      q4_lane_reduce<M>(acc);
      if (g == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int m = 0; m < M; ++m) red[wave][8 * i + (lane >> 3)][m] = acc[i][m];
      }
    }
    __syncthreads();

    // Publish: device-scope stores, wait for them, then move the counters.
    if (J.S == 1) {
      for (int idx = threadIdx.x; idx < 32 * M; idx += 256) {
        const int r = idx / M, m = idx - r * M;
        st_coherent(J.y + (size_t)m * J.ldy + 32 * tr + r,
                    ((red[0][r][m] + red[1][r][m]) + red[2][r][m]) + red[3][r][m]);
      }
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(a.done + J.phase, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const size_t slot = (size_t)J.slot0 + tr;
      float* pp = a.partial + (slot * a.smax + s) * 32 * M;
      for (int idx = threadIdx.x; idx < 32 * M; idx += 256) {
        const int r = idx / M, m = idx - r * M;
        st_coherent(pp + idx, ((red[0][r][m] + red[1][r][m]) + red[2][r][m]) + red[3][r][m]);
      }
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0)
        s_old = __hip_atomic_fetch_add(a.row_cnt + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (s_old == (uint32_t)J.S - 1) {   // last part of this tile row: add the parts in order
        const float* p0 = a.partial + slot * a.smax * 32 * M;
        for (int idx = threadIdx.x; idx < 32 * M; idx += 256) {
          const int r = idx / M, m = idx - r * M;
          float v = 0.f;
          for (int p = 0; p < J.S; ++p) v += ld_coherent(p0 + (size_t)p * 32 * M + idx);
          st_coherent(J.y + (size_t)m * J.ldy + 32 * tr + r, v);
        }
        wait_stores();
        __syncthreads();
        if (threadIdx.x == 0) {
          __hip_atomic_store(a.row_cnt + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_fetch_add(a.done + J.phase, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();   // red and s_old are reused by the next unit
  }

  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {   // last workgroup out: ready the counters for the next run
      for (int p = 0; p < a.n_phases; ++p)
        __hip_atomic_store(a.done + p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ctl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int KIND, int M>
static const void* plan_fn() {
  return reinterpret_cast<const void*>(&k_plan<KIND, M>);
}

template <int KIND>
static const void* plan_fn_m(int M) {
  switch (M) {
    case 1: return plan_fn<KIND, 1>();
    case 2: return plan_fn<KIND, 2>();
    case 3: return plan_fn<KIND, 3>();
    case 4: return plan_fn<KIND, 4>();
  }
  return nullptr;
}

static const void* plan_kernel(int kind, int M) {
  switch (kind) {
    case KIND_Q4_1: return plan_fn_m<KIND_Q4_1>(M);
    case KIND_Q4_K: return plan_fn_m<KIND_Q4_K>(M);
    case KIND_Q8_A: return plan_fn_m<KIND_Q8_A>(M);
    case KIND_Q8_B: return plan_fn_m<KIND_Q8_B>(M);
  }
  return nullptr;
}

hipError_t plan_resident_blocks(int kind, int M, int* blocks) {
  const void* f = plan_kernel(kind, M);
  if (!f) return hipErrorInvalidValue;
  int per_cu = 0, dev = 0, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, 256, 0);
  if (e != hipSuccess) return e;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  *blocks = per_cu * cus;
  return hipSuccess;
}

hipError_t launch_plan(int kind, int M, const PlanArgs& a, int grid, hipStream_t s) {
  const void* f = plan_kernel(kind, M);
  if (!f) return hipErrorInvalidValue;
  void* args[] = {const_cast<PlanArgs*>(&a)};
  return hipLaunchKernel(f, dim3(grid), dim3(256), args, 0, s);
}

}  // namespace q4nx
