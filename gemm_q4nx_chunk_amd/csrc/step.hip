// A decode step's dependent GEMV phases in one persistent launch, q4 kinds.
//
// A decode step is a chain of GEMV groups that wait on each other (per layer
// q|k|v, o, gate|up, down, then the lm_head).  Launched one group at a time,
// each phase streams only a few MB, so much of its time goes into filling and
// draining the memory pipeline and into the launch itself (the Strata article,
// section 3.2, runs its whole pass as one captured graph for the launch part).
// Here the whole chain is one launch whose weight stream does not stop at a
// phase boundary:
//
//  * One workgroup per CU, all resident (the LDS size makes sure of it), each
//    with a static list of pieces built on the host: a piece is one tile row
//    of one job (cut when longer than kStepPieceCols chunks), and a
//    workgroup's pieces follow the phases in order.  Whole tile rows go to
//    workgroups largest first, to the least loaded one in the phase, so no
//    partial sums cross workgroups.
//  * Eight compute waves (two per SIMD) split each piece's chunks; each
//    streams its share through a ring of LDS slots of its own with direct
//    global-to-LDS loads, several chunks ahead across piece and phase
//    boundaries, so the loads of phase p + 1 are in flight while phase p
//    finishes and while the workgroup waits for it.  The compute waves wait
//    for nothing but their own loads and the workgroup barrier.
//  * A ninth wave does all the ordering: it writes y (device-scope stores),
//    waits for those stores, counts the workgroup out of the phase on its
//    XCD's counter, waits until every XCD's counter shows all of its
//    workgroups out of the previous phase, and stages the next activations in
//    LDS.  Its loads and stores are never queued behind the weight stream.
//  * Activations become fp16 records in LDS (the GEMV's own records, built in
//    place over the staged bf16 values by every wave), once per phase and
//    activation vector.
//
// Measured on the Qwen3-4B-shaped step (145 phases) this runs at 1.77 ms
// against 1.02 ms for the same phases as graph-captured launches: each hand-off
// (publish, count, see every XCD's count, stage x) costs 3-4 us here against
// about 2 us for a kernel boundary, and each phase's dequantisation then runs
// on a few waves per CU with the whole phase's latency exposed.  It is the
// plan's path because it beats the unit-dealing kernel (2.5 ms).
//
// Every wait is bounded: past the spin limit the kernel raises an error flag
// and stops waiting (later waits return at once), so a grid that cannot be
// resident ends in an error, never a hang.  The last workgroup out puts the
// counters back to zero for the next run.
#include "gemv_core.h"
#include "plan_args.h"

namespace q4nx {

namespace {

constexpr size_t kStepMinLds = 84 * 1024;   // two workgroups never share a CU
constexpr int kStage = 16;                   // activation loads in flight per sync-wave lane
constexpr int kSlot = kStepSlot;

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier of the whole workgroup that orders LDS only: the weight loads in
// flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Sync wave: wait until word c[16 x] >= need (lane x < 8 holds XCD x's need).
__device__ void wait_xcds(const uint32_t* c, uint32_t need, int lane, int limit, uint32_t* ctl) {
  if (ld_agent(ctl + 1)) return;   // an earlier wait gave up: no more waiting
  for (int it = 0;; ++it) {
    const bool behind = lane < 8 && ld_agent(c + 16 * lane) < need;
    if (__builtin_amdgcn_ballot_w64(behind) == 0) return;
    if (it >= limit) {
      if (lane == 0) __hip_atomic_fetch_or(ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// A buffer resource built from values every lane holds alike, placed in scalar
// registers: said explicitly, or the compiler may take them for per-lane values
// and serialise every load through them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, uint32_t n) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(n));
}

// Device-scope store through a global-space pointer (a global store, which the
// compiler does not hold back behind this wave's earlier memory operations).
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store((__attribute__((address_space(1))) float*)p, v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at dst + 16 l (dst is the same for the whole wave).
__device__ __forceinline__ void lds_dma16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// Wait until at most `after` chunks of L loads each are still in flight.
template <int L>
__device__ __forceinline__ void wait_landed(int after) {
  static_assert(L * (kStepMaxSlots - 1) <= 63, "vmcnt holds 6 bits");
  switch (after) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * L) : "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * L) : "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * L) : "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * L) : "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * L) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(7 * L) : "memory"); break;
  }
}

}  // namespace

template <int KIND, int M>
__global__ __launch_bounds__(kStepThreads) void k_step(const StepArgs a) {
  constexpr int CB = ChunkBytes<KIND>::value;
  constexpr int kLoads = (CB + 1023) / 1024;   // 16-byte-per-lane loads per chunk
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];   // records (see below)
  constexpr int CW = kStepComputeWaves;
  __shared__ float red[2][CW][32][M];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool syncw = wave == CW;
  const int g = lane & 7;
  const int u0 = ld_const(a.wg_first, blockIdx.x), u1 = ld_const(a.wg_first, blockIdx.x + 1);
  const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7;   // HW_REG_XCC_ID
  uint32_t need = 0;   // sync wave, lane x < 8: workgroups of this launch on XCD x

  if (syncw) {   // count this workgroup in, then learn every XCD's count once all are in
    if (lane == 0) __hip_atomic_fetch_add(a.sync + 16 * xcc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0;; ++it) {
      uint32_t v = lane < 8 ? ld_agent(a.sync + 16 * lane) : 0u;
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      if (__builtin_amdgcn_readfirstlane(v) >= gridDim.x) break;
      if (it >= a.spin_limit) {
        if (lane == 0) __hip_atomic_fetch_or(a.ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    need = lane < 8 ? ld_agent(a.sync + 16 * lane) : 0u;
  }
  uint32_t* arrive = a.sync + 128;   // phase p, XCD x at arrive[16 (8 p + x)]

  // Records, as in the GEMV: record r = (m TC + c) 8 + g holds the 32
  // activations x[m][32 (8c + g) ..] as 16 fp16 (or bf16) pairs at xl[16 r],
  // and (f, X) at xl[16 R + 2 r].  The bf16 values are first staged over the
  // pair area itself: x[m][8q .. 8q + 7] (q = r 4 + d) at xl[4 q], so each
  // lane reads its 16 bytes and writes its record quarter to the same place.
  float* sums = reinterpret_cast<float*>(xl);   // offset 16 R, set per build
  const uint16_t* rec_x = nullptr;
  int rec_ldx = 0, rec_tc = 0;
  int sig = 0;               // phases below this one are counted out
  int cur_phase = -1;
  // sync wave: the last finished tile row whose y is still to be written
  int pend_job = -1, pend_tr = 0, pend_par = 0;

  auto store_pending = [&]() {
    if (pend_job < 0) return;
    // every lane holds the same index: read the job through scalar loads, which
    // never wait behind this wave's earlier stores
    const StepJob P = ld_const(a.jobs, __builtin_amdgcn_readfirstlane(pend_job));
    for (int idx = lane; idx < 32 * M; idx += 64) {
      const int r = idx / M, m = idx - r * M;
      float v = red[pend_par][0][r][m];
#pragma unroll
      for (int w = 1; w < CW; ++w) v += red[pend_par][w][r][m];
      st_agent(P.y + (size_t)m * P.ldy + 32 * __builtin_amdgcn_readfirstlane(pend_tr) + r, v);
    }
    pend_job = -1;
  };

  const Q4Consts kc = q4_consts();
  float acc[4][M];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;

  // Each compute wave streams its chunks through a ring of a.ns slots of its
  // own in LDS, filled by direct global-to-LDS loads (no registers held): the
  // wave walks its share of the pieces in order, keeping up to a.ns chunks in
  // flight, across piece and phase boundaries.  The wave's memory counter
  // counts only these loads, in order, so "chunk t has landed" is "at most
  // (chunks issued after t) x kLoads loads outstanding".
  uint8_t* const ring = reinterpret_cast<uint8_t*>(xl) + a.ring_off + (size_t)(syncw ? 0 : wave) * a.ns * kSlot;
  int issued = 0, consumed = 0;
  int pk = u0, pj = 0, pnw = 0;
  bool pvalid = false;
  const uint8_t* pbase = nullptr;
  auto share = [&](int k, int& cw0, int& nw) {   // the wave's chunk columns of piece k
    const StepUnit U = ld_const(a.units, k);
    const int n = U.c1 - U.c0;
    cw0 = U.c0 + wave * n / CW;
    nw = U.c0 + (wave + 1) * n / CW - cw0;
  };
  auto top_up = [&]() {
    while (issued - consumed < a.ns) {
      if (!pvalid) {
        if (pk >= u1) return;
        int cw0;
        share(pk, cw0, pnw);
        const StepUnit U = ld_const(a.units, pk);
        const StepJob J = ld_const(a.jobs, U.job);
        pbase = J.w + ((size_t)U.tr * J.TC + cw0) * CB;
        pj = 0;
        pvalid = true;
      }
      if (pj >= pnw) {
        ++pk;
        pvalid = false;
        continue;
      }
      uint8_t* dst = ring + (size_t)(issued % a.ns) * kSlot;
      const uint8_t* src = pbase + (size_t)pj * CB + 16 * lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma16(src + 1024 * i, dst + 1024 * i);
      if (CB - 4096 >= 1024 || lane < (CB - 4096) / 16) lds_dma16(src + 4096, dst + 4096);
      ++pj;
      ++issued;
    }
  };

  auto piece = [&](int k) {
    const StepUnit U = ld_const(a.units, k);
    const StepJob J = ld_const(a.jobs, U.job);
    if (!syncw) top_up();   // the next chunks in flight before any wait below
    const bool new_phase = U.phase != cur_phase;
    if (new_phase || J.x != rec_x || J.ldx != rec_ldx || J.TC != rec_tc) {
      const int R = M * J.TC * 8;
      if (syncw) {
        store_pending();
        if (new_phase) {
          wait_stores();   // the finished phase's y is visible before it is counted out
          if (lane == 0)
            for (int p = sig; p < U.phase; ++p)
              __hip_atomic_fetch_add(arrive + 16 * (8 * p + xcc), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          sig = U.phase;
          if (U.phase > 0) wait_xcds(arrive + 128 * (U.phase - 1), need, lane, a.spin_limit, a.ctl);
        }
        // stage x[m][0 .. 256 TC) for m < M: 16 bytes per lane and load, in batches
        const int per_row = 32 * J.TC;   // 16-byte pieces per activation row
        const __amdgpu_buffer_rsrc_t xrs = uniform_rsrc(J.x, (uint32_t)(((M - 1) * J.ldx + J.TC * 256) * 2));
        for (int q0 = 0; q0 < 4 * R; q0 += 64 * kStage) {
          u32x4 v[kStage];
#pragma unroll
          for (int i = 0; i < kStage; ++i) {
            const int q = q0 + 64 * i + lane;
            const int m = q / per_row, off = q - m * per_row;
            v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 xrs, (uint32_t)(m * J.ldx + 8 * off) * 2, 0, kCpolSc1));
          }
#pragma unroll
          for (int i = 0; i < kStage; ++i) {
            const int q = q0 + 64 * i + lane;
            if (q < 4 * R) *reinterpret_cast<u32x4*>(xl + 4 * q) = v[i];
          }
        }
      }
      lds_barrier();
      sums = reinterpret_cast<float*>(xl + 16 * R);
      for (int q = tid; q < 4 * R; q += kStepThreads) {   // whole quads: 4 R and the stride are multiples of 4
        const u32x4 v = *reinterpret_cast<const u32x4*>(xl + 4 * q);
        uint32_t pr[4];
        float f, X;
        x_record_part(v, pr, f, X);
        *reinterpret_cast<u32x4*>(xl + 4 * q) = u32x4{pr[0], pr[1], pr[2], pr[3]};
        if ((q & 3) == 0) {
          sums[2 * (q >> 2)] = f;
          sums[2 * (q >> 2) + 1] = X;
        }
      }
      lds_barrier();
      cur_phase = U.phase;
      rec_x = J.x;
      rec_ldx = J.ldx;
      rec_tc = J.TC;
    }
    if (!syncw) {
      if (U.flags & kStepFirst) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int m = 0; m < M; ++m) acc[i][m] = 0.f;
      }
      int cw0, nw;
      share(k, cw0, nw);
      const int TC = J.TC;
      for (int j = 0; j < nw; ++j) {
        wait_landed<kLoads>(issued - consumed - 1);
        const uint8_t* sl = ring + (size_t)(consumed % a.ns) * kSlot;
        Q4Chunk<KIND, 4> ch;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ch.q[i] = *reinterpret_cast<const u32x4*>(sl + 1024 * i + 16 * lane);
          if constexpr (KIND == KIND_Q4_1) {
            ch.meta[i] = *reinterpret_cast<const uint32_t*>(sl + 4096 + 256 * i + 4 * lane);
            ch.rowsm[i] = 0;
          } else {
            ch.meta[i] = *reinterpret_cast<const uint16_t*>(sl + 4096 + 128 * i + 2 * lane);
            ch.rowsm[i] = *reinterpret_cast<const uint32_t*>(sl + 4608 + 32 * i + 4 * (lane >> 3));
          }
        }
        XRec<M> xp;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const int r = (m * TC + cw0 + j) * 8 + g;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(xl + 16 * r + 4 * d);
            xp.p[m][4 * d] = v.x;
            xp.p[m][4 * d + 1] = v.y;
            xp.p[m][4 * d + 2] = v.z;
            xp.p[m][4 * d + 3] = v.w;
          }
          xp.f[m] = sums[2 * r];
          xp.X[m] = sums[2 * r + 1];
        }
        q4_compute<KIND, M, 4>(ch, xp, kc, acc);
        ++consumed;
        top_up();   // refill the slot just read
      }
      if (U.flags & kStepLast) {
        q4_lane_reduce<M>(acc);
        if (g == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m = 0; m < M; ++m) red[k & 1][wave][8 * i + (lane >> 3)][m] = acc[i][m];
        }
      }
    } else {
      store_pending();   // the previous tile row, while this one is computed
    }
    lds_barrier();
    if (syncw && (U.flags & kStepLast)) {
      pend_job = U.job;
      pend_tr = U.tr;
      pend_par = k & 1;
    }
  };

  for (int k = u0; k < u1; ++k) piece(k);

  if (syncw) {
    store_pending();
    wait_stores();
    if (lane == 0) {
      for (int p = sig; p < a.n_phases; ++p)
        __hip_atomic_fetch_add(arrive + 16 * (8 * p + xcc), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t old = __hip_atomic_fetch_add(a.ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == gridDim.x - 1) {   // last workgroup out: every counter back to zero for the next run
        for (int x = 0; x < 8; ++x) __hip_atomic_store(a.sync + 16 * x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = 0; i < 8 * a.n_phases; ++i)
          __hip_atomic_store(arrive + 16 * i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.ctl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

constexpr size_t kStepLdsLimit = 152 * 1024;   // dynamic LDS; the reduction buffer is static

StepLds step_lds(int M, int max_tc) {
  StepLds L;
  L.rec = ((size_t)M * max_tc * 8 * 72 + 255) & ~(size_t)255;
  L.ns = 0;
  L.total = 0;
  if (L.rec + kStepComputeWaves * 2 * (size_t)kStepSlot > kStepLdsLimit) return L;
  const size_t ns = (kStepLdsLimit - L.rec) / (kStepComputeWaves * (size_t)kStepSlot);
  L.ns = (int)(ns < (size_t)kStepMaxSlots ? ns : (size_t)kStepMaxSlots);
  L.total = L.rec + kStepComputeWaves * (size_t)L.ns * kStepSlot;
  if (L.total < kStepMinLds) L.total = kStepMinLds;
  return L;
}

template <int KIND, int M>
static hipError_t launch_step_t(const StepArgs& a, int grid, size_t lds, hipStream_t s) {
  auto* f = k_step<KIND, M>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kStepLdsLimit);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(f, dim3(grid), dim3(kStepThreads), lds, s, a);
  return hipGetLastError();
}

template <int KIND>
static hipError_t launch_step_m(int M, const StepArgs& a, int grid, size_t lds, hipStream_t s) {
  switch (M) {
    case 1: return launch_step_t<KIND, 1>(a, grid, lds, s);
    case 2: return launch_step_t<KIND, 2>(a, grid, lds, s);
    case 3: return launch_step_t<KIND, 3>(a, grid, lds, s);
    case 4: return launch_step_t<KIND, 4>(a, grid, lds, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_step(int kind, int M, const StepArgs& a, int grid, size_t lds, hipStream_t s) {
  switch (kind) {
    case KIND_Q4_1: return launch_step_m<KIND_Q4_1>(M, a, grid, lds, s);
    case KIND_Q4_K: return launch_step_m<KIND_Q4_K>(M, a, grid, lds, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace q4nx
