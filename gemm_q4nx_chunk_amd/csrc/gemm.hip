// Q4NX block GEMM for gfx950: Y[m] = W X[m] for a prompt block of M <= 64 rows.
//
// At 64 rows each 4-bit weight serves 128 flops, a dense contraction, so the
// products run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation.  Each chunk is read from HBM once and dequantised once, in
// registers, to bf16 (round to nearest even); no bf16 copy of a weight is ever
// written.  All M rows share one pass over the weights: splitting the token
// rows over several passes would read the weights again (Strata article,
// section 3.2, the work split inside one layer: an overlap attempt lost speed
// by reading the dense weights twice).
//
// Workgroup: 8 waves, one tile row (32 outputs) each, over a range of tile
// columns.  The X columns of the current tile column (M x 256 bf16) sit in
// LDS, double buffered, shared by the 8 waves.  When the tile rows alone give
// too few workgroups to keep every CU's ALUs busy with dequantisation, K is
// split over S workgroups; each writes its fp32 partial tile to the workspace
// and the last of the S to arrive adds the parts in part order (no atomics on
// data, so the result bits do not depend on timing).  The dequantisation and
// the order of k inside an MFMA step are described in mfma_q4.h.
#include <atomic>
#include <mutex>

#include "gemm_args.h"
#include "mfma_q4.h"
#include "q4nx_dev.h"

namespace q4nx {

constexpr int kGemmWaves = 8;
#ifndef Q4NX_GEMM_DEPTH
#define Q4NX_GEMM_DEPTH 2
#endif
constexpr int kGemmDepth = Q4NX_GEMM_DEPTH;   // chunk loads in flight per wave
static_assert(kGemmWaves == kGemmRowsPerWg, "one tile row per wave");

// The X columns of the current tile column (XR x 256 bf16) sit in LDS, double
// buffered: the next tile column's X is loaded into registers at the start of
// a step and written to the other buffer at its end.  Chunk loads of tile
// column t run D tile columns ahead of its products, in a ring of D register
// sets.  All loads are unconditional (buffer loads past the end read zero
// without touching memory) and every branch is uniform, so the compiler's
// wait counts stay exact: a step waits only for its own chunk and, at its
// end, for the next X tile.  Waves past the last tile row and X rows past M
// read clamped, in-bounds data whose results are not stored.
#ifndef Q4NX_GEMM_QBARRIER
#define Q4NX_GEMM_QBARRIER 0
#endif
// Waves per SIMD the kernel is compiled for: M > 32 (two accumulator tiles)
// one workgroup per CU, M <= 32 two (at most 128 VGPRs).
#ifndef Q4NX_GEMM_WPE_TWO
#define Q4NX_GEMM_WPE_TWO 2
#endif
#ifndef Q4NX_GEMM_WPE_ONE
#define Q4NX_GEMM_WPE_ONE 4
#endif
// XCD-local placement.  Workgroups are dealt to the 8 XCDs round-robin by
// linear id from a starting XCD that varies between launches (XCD = (id + c)
// mod 8 for one c per launch), so the 8 workgroups of group r = id / 8 land on
// 8 different XCDs, and the workgroup on XCD x takes workgroup row
// nb = 8 (r / S) + x and part r % S: every K part of row nb runs on XCD
// nb % 8, where its partial tiles and arrival counter meet in one L2.
//
// That placement is checked, not assumed: each workgroup claims its XCD's slot
// of its group with an atomic OR.  If the slot is taken (another workgroup of
// the group landed on the same XCD, as concurrent dispatches from other
// streams can cause), it takes the first free slot instead -- 8 workgroups, 8
// slots: each ends with one -- and is "displaced": its unit's home XCD is not
// its own.  A displaced workgroup computes its rows over the whole K range and
// writes Y itself, raises the row's rescue flag and then counts its part in;
// the home parts of that row see the flag and skip their combine.  The last
// claimer of a group clears the group's word for the next call.
struct GemmUnit {
  int nb, part;
  bool displaced;
};

__device__ __forceinline__ GemmUnit gemm_claim(const GemmArgs& a, uint32_t* s_slot) {
  const int r = blockIdx.x >> 3;
  const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7;   // HW_REG_XCC_ID
  if (threadIdx.x == 0) {
    const bool force = a.test_mode == 1 && (r & 1);   // tests: odd groups act displaced
    uint32_t x = xcc, bit = 1u << xcc, old = 0;
    if (!force) old = __hip_atomic_fetch_or(a.claim + r, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (force || (old & bit)) {
      if (!force) __hip_atomic_fetch_add(a.diag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t start = force ? xcc + 1 : 0;
      for (uint32_t i = 0; i < 8; ++i) {
        x = (start + i) & 7;
        bit = 1u << x;
        old = __hip_atomic_fetch_or(a.claim + r, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!(old & bit)) break;
      }
    }
    if ((old | bit) == 0xFFu) __hip_atomic_store(a.claim + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_slot = x;
  }
  __syncthreads();
  const uint32_t x = *s_slot;
  return GemmUnit{8 * (r / a.S) + (int)x, r % a.S, x != xcc};
}

// A displaced workgroup's row is complete in Y: raise the row's rescue flag,
// then count the part in (the flag is out before the count moves); the last
// of the row's parts clears both.
__device__ __forceinline__ void gemm_rescued_part(const GemmArgs& a, int nb) {
  __hip_atomic_store(a.rescued + nb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_stores();
  const uint32_t old = __hip_atomic_fetch_add(a.cnt + nb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old == (uint32_t)a.S - 1) {
    __hip_atomic_store(a.cnt + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.rescued + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int KIND, bool TWO, int D, bool LOCAL>
__global__ __launch_bounds__(64 * kGemmWaves)
__attribute__((amdgpu_waves_per_eu(TWO ? Q4NX_GEMM_WPE_TWO : Q4NX_GEMM_WPE_ONE, TWO ? Q4NX_GEMM_WPE_TWO : Q4NX_GEMM_WPE_ONE)))
void k_gemm_q4(GemmArgs a) {
  constexpr int CB = ChunkBytes<KIND>::value;
  constexpr int NT = 64 * kGemmWaves;
  constexpr int XR = TWO ? 64 : 32;          // token rows staged in LDS
  constexpr int G = TWO ? 8 : 4;             // f32x4 groups of the accumulators
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][XR * kXs];
  __shared__ uint32_t s_old, s_flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave: row data in SGPRs
  const int h = lane >> 5, n = lane & 31;
  // LOCAL: all K parts of a row on one XCD, claimed as gemm_claim describes.
  int nb, part;
  bool displaced = false;
  if constexpr (LOCAL) {
    const GemmUnit u = gemm_claim(a, &s_old);
    nb = u.nb;
    part = u.part;
    displaced = u.displaced;
    if (nb >= a.NB) return;
  } else {
    nb = blockIdx.x;
    part = blockIdx.y;
  }
  int ji = 0;
  for (int i = 1; i < a.n_jobs; ++i)
    if (nb >= a.job[i].nb0) ji = i;
  const GemmJob& job = a.job[ji];
  const int tr_raw = (nb - job.nb0) * kGemmWaves + wave;
  const bool active = tr_raw < job.TR;
  const int tr = active ? tr_raw : job.TR - 1;
  const int K = a.TC * 256, N = job.TR * 32, M = a.M;
  // a displaced workgroup takes its rows' whole K range
  const int tc0 = displaced ? 0 : part * a.TC / a.S, tc1 = displaced ? a.TC : (part + 1) * a.TC / a.S;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(job.w + ((size_t)tr * a.TC + tc0) * CB, (uint32_t)((tc1 - tc0) * CB));

  uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  asm volatile("" : "+s"(kMaskLo));
  asm volatile("" : "+s"(kMaskHi));
  asm volatile("" : "+v"(kMagic));

  // X tile loader: XR rows x 32 pieces of 16 B over NT threads (row clamped to
  // M - 1).  Past the last tile column of X the loads read zeros or the next
  // row; that tile is never used.
  constexpr int XP = XR * 32 / NT;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.X, (uint32_t)(M * K * 2));
  uint32_t xoff[XP];
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    const int piece = tid + NT * p, row = piece >> 5, c16 = piece & 31;
    xoff[p] = (uint32_t)((row < M ? row : M - 1) * K + c16 * 8) * 2;
  }
  // X tiles are loaded two tile columns ahead: xr[b] holds the tile whose
  // column has parity b (relative to tc0) until it is written to xs[b].
  u32x4 xr[2][XP];
  auto xload = [&](int b, int tc) {
#pragma unroll
    for (int p = 0; p < XP; ++p)
      xr[b][p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[p] + tc * 512, 0, 0));
  };
  auto xstore = [&](int b) {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int piece = tid + NT * p, row = piece >> 5, c16 = piece & 31;
      *reinterpret_cast<u32x4*>(&xs[b][row * kXs + c16 * 8]) = xr[b][p];
    }
  };

  f32x16 acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) { acc0[v] = 0.f; acc1[v] = 0.f; }

  GemmChunk<KIND> c[D];
  xload(0, tc0);
#pragma unroll
  for (int j = 0; j < D; ++j) gemm_load<KIND>(wrs, j * CB, n, h, c[j]);
  xstore(0);
  xload(1, tc0 + 1);

  // One tile column t (parity j relative to tc0): its X tile is in xs[j], its
  // chunk in c[j]; the tile of t + 1 is in flight in xr[j ^ 1].
  static_assert(D % 2 == 0, "the X double buffer follows the chunk ring's parity");
  auto step = [&](int j, int t) {
    __syncthreads();                       // X tile t is in xs[j]; xs[j ^ 1] is free
    xload(j, t + 2);                       // xr[j] went to LDS at the end of step t - 1
    __builtin_amdgcn_sched_barrier(0);     // issue the X loads before the products
    const uint16_t* xb = xs[j] + n * kXs + 128 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#if Q4NX_GEMM_QBARRIER
      __builtin_amdgcn_sched_barrier(0);   // bound how far operand reads are hoisted (registers)
#endif
      float s, z;
      group_sz<KIND>(c[j], q, s, z);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int st = 4 * q + e;
        const bf16x8 B = dequant8(c[j].q[q][e], s, z, kMaskLo, kMaskHi, kMagic);
        const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(xb + 8 * st);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B, acc0, 0, 0, 0);
        if constexpr (TWO) {
          const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(xb + 32 * kXs + 8 * st);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B, acc1, 0, 0, 0);
        }
      }
    }
    gemm_load<KIND>(wrs, (uint32_t)(t + D - tc0) * CB, n, h, c[j]);
    xstore(j ^ 1);                         // tile t + 1, loaded during step t - 1
  };
  // Full groups of D tile columns, then the last (tc1 - tc0) % D: no branch
  // inside a group, so every wait is for the chunk D tile columns back.
  int base = tc0;
  for (; base + D <= tc1; base += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) step(j, base + j);
  }
#pragma unroll
  for (int j = 0; j + 1 < D; ++j)
    if (base + j < tc1) step(j, base + j);

  // 32x32 accumulator: register v of lane holds token row 8*(v/4) + 4*h + v%4, output column n.
  auto store_y = [&](const f32x4* r) {
    float* yc = job.Y + 32 * tr + n;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 32 * (g >> 2) + 8 * (g & 3) + 4 * h + i;
        if (m < M) yc[(size_t)m * N] = r[g][i];
      }
  };
  f32x4 mine[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) mine[g][i] = g < 4 ? acc0[4 * g + i] : acc1[4 * (g - 4) + i];
  if (a.S == 1 || displaced) {
    if (active) store_y(mine);
    if (displaced) {
      wait_stores();
      __syncthreads();
      if (tid == 0) gemm_rescued_part(a, nb);
    }
    return;
  }

  // Split K: each part stores its accumulators in register order (16 B per
  // lane and group), and the last part of the block to arrive adds all parts,
  // its own read back too, in part order (unless a displaced workgroup has
  // already written the row whole).  Loads past the last part fall outside the
  // buffer resource and read zero.
  constexpr size_t kPartBytes = (size_t)kGemmWaves * 8 * 64 * 16;
  const uint32_t part_bytes = (uint32_t)(kPartBytes * a.S);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.partial + (size_t)nb * a.S * (kPartBytes / 4), part_bytes);
  const uint32_t lane_off = (uint32_t)(wave * 8 * 64 + lane) * 16;
  // LOCAL: plain stores (they complete in this XCD's L2) and L2 atomics;
  // otherwise device-scope (sc1) stores, loads and atomics.
  constexpr int kStPol = LOCAL ? 0 : kCpolSc1;
  constexpr int kLdPol = LOCAL ? 1 : kCpolSc1;   // sc0: past this CU's L1
#pragma unroll
  for (int g = 0; g < G; ++g)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, mine[g]), rs,
                                           lane_off + part * (uint32_t)kPartBytes + g * 1024, 0, kStPol);
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    s_old = __hip_atomic_fetch_add(a.cnt + nb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag = 0;
    if (s_old == (uint32_t)a.S - 1) {
      s_flag = __hip_atomic_load(a.rescued + nb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (s_flag) {   // the row is already whole in Y: clear for the next call
        __hip_atomic_store(a.cnt + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.rescued + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __syncthreads();
  if (s_old != (uint32_t)a.S - 1 || s_flag) return;

  constexpr int PB = 16 / G;                 // parts loaded per round trip (64 registers)
  f32x4 sum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) sum[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < a.S; p0 += PB) {
    f32x4 in[PB][G];
#pragma unroll
    for (int j = 0; j < PB; ++j)
#pragma unroll
      for (int g = 0; g < G; ++g)
        in[j][g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, lane_off + (p0 + j) * (uint32_t)kPartBytes + g * 1024, 0, kLdPol));
#pragma unroll
    for (int j = 0; j < PB; ++j)
      if (p0 + j < a.S)
#pragma unroll
        for (int g = 0; g < G; ++g) sum[g] += in[j][g];
  }
  if (active) store_y(sum);
  if (tid == 0) __hip_atomic_store(a.cnt + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The M > 32 variant: 8 waves = 4 tile rows x 2 halves of the workgroup's K
// range.  Wave (row rho, half pi) multiplies tile row rho's chunks of its
// half; the halves meet in LDS at the end (fixed order: first + second).  A
// workgroup covers 4 tile rows, so twice as many workgroups fill the chip
// before K has to be split across workgroups, whose fp32 partial tiles (64
// tokens x 32 outputs per row) cost as many bytes as a few tile columns of
// weights.  The X columns of both halves' current tile columns (2 x 64 x 256
// bf16) sit in LDS, double buffered: the next step's tiles are loaded into
// registers at the start of a step and written to the other buffer at its
// end.  Chunk loads run D steps ahead in a ring of D register sets; as above,
// every load is unconditional and every branch uniform.  Inside a step the
// dequantisation of the next MFMA step's weights and the reads of its X
// operands are interleaved with the current products.
template <int KIND, int D, bool LOCAL>
__global__ __launch_bounds__(64 * kGemmWaves)
__attribute__((amdgpu_waves_per_eu(Q4NX_GEMM_WPE_TWO, Q4NX_GEMM_WPE_TWO)))
void k_gemm_q4h(GemmArgs a) {
  constexpr int CB = ChunkBytes<KIND>::value;
  constexpr int XR = 64, G = 8, R = kGemmRowsHalves;
  constexpr int NH = 64 * kGemmWaves / 2;    // threads of one half
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][2][XR * kXs];   // [buffer][half]
  __shared__ uint32_t s_old, s_flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave: row data in SGPRs
  const int rho = wave & (R - 1), pi = wave / R;
  const int h = lane >> 5, n = lane & 31;
  int nb, part;   // workgroup row and K part, laid out as in k_gemm_q4
  bool displaced = false;
  if constexpr (LOCAL) {
    const GemmUnit u = gemm_claim(a, &s_old);
    nb = u.nb;
    part = u.part;
    displaced = u.displaced;
    if (nb >= a.NB) return;
  } else {
    nb = blockIdx.x;
    part = blockIdx.y;
  }
  int ji = 0;
  for (int i = 1; i < a.n_jobs; ++i)
    if (nb >= a.job[i].nb0) ji = i;
  const GemmJob& job = a.job[ji];
  const int tr_raw = (nb - job.nb0) * R + rho;
  const bool active = tr_raw < job.TR;
  const int tr = active ? tr_raw : job.TR - 1;
  const int K = a.TC * 256, N = job.TR * 32, M = a.M;
  // the workgroup's K part [tc0, tc1) (all of K when displaced), cut into
  // halves [tc0, mid) and [mid, tc1)
  const int tc0 = displaced ? 0 : part * a.TC / a.S, tc1 = displaced ? a.TC : (part + 1) * a.TC / a.S;
  const int mid = tc0 + (tc1 - tc0 + 1) / 2;
  const int nsteps = mid - tc0;                          // steps of the first (longer) half
  const int hc0 = pi ? mid : tc0, hc1 = pi ? tc1 : mid;  // this wave's half
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(job.w + ((size_t)tr * a.TC + hc0) * CB, (uint32_t)((hc1 - hc0) * CB));

  uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  asm volatile("" : "+s"(kMaskLo));
  asm volatile("" : "+s"(kMaskHi));
  asm volatile("" : "+v"(kMagic));

  // X tile loader: the threads of half pi load that half's tile, 64 rows x 32
  // pieces of 16 B; thread th takes rows th / 32 + 8 p.  Rows past M fall
  // outside the buffer resource and read zero; past the end of the half the
  // loads read other columns of X or zeros.  Those values are never stored.
  constexpr int XP = XR * 32 / NH;
  const int th = tid - pi * NH;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.X, (uint32_t)(M * K * 2));
  const uint32_t xoff = (uint32_t)((th >> 5) * K + (th & 31) * 8) * 2;
  const uint32_t xrow8 = (uint32_t)(8 * K * 2);          // 8 rows of X, bytes
  u32x4 xr[XP];
  auto xload = [&](int t) {   // t: step index (tile column hc0 + t)
    const uint32_t col = (uint32_t)(hc0 + t) * 512;
#pragma unroll
    for (int p = 0; p < XP; ++p)
      xr[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff + col, p * xrow8, 0));
  };
  auto xstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int piece = th + NH * p, row = piece >> 5, c16 = piece & 31;
      *reinterpret_cast<u32x4*>(&xs[buf][pi][row * kXs + c16 * 8]) = xr[p];
    }
  };

  f32x16 acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) { acc0[v] = 0.f; acc1[v] = 0.f; }

  GemmChunk<KIND> c[D];
  xload(0);
#pragma unroll
  for (int j = 0; j < D; ++j) gemm_load<KIND>(wrs, j * CB, n, h, c[j]);
  xstore(0);

  // Step t: this half's X tile is in xs[t & 1][pi], its chunk in c[jc]
  // (jc = t mod D).  The tiles of step t + 1 are loaded at the top of the
  // step and stored to the other buffer at its end (one register set: the
  // products cover their latency).  The second half may have one step fewer:
  // its waves skip the products of that step.
  auto step = [&](int jc, int t) {
    const int j = t & 1;
    __syncthreads();                       // the tiles of step t are in xs[j]; xs[j ^ 1] is free
    xload(t + 1);
    __builtin_amdgcn_sched_barrier(0);     // issue the X loads before the products
    if (hc0 + t < hc1)
      mfma_tile<KIND>(c[jc], xs[j][pi] + n * kXs + 128 * h, 32 * kXs, acc0, acc1, kMaskLo, kMaskHi, kMagic);
    gemm_load<KIND>(wrs, (uint32_t)(t + D) * CB, n, h, c[jc]);
    xstore(j ^ 1);                         // tiles of step t + 1
  };
  int base = 0;
  for (; base + D <= nsteps; base += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) step(j, base + j);
  }
#pragma unroll
  for (int j = 0; j + 1 < D; ++j)
    if (base + j < nsteps) step(j, base + j);

  // 32x32 accumulator: register v of lane holds token row 8*(v/4) + 4*h + v%4, output column n.
  f32x4 mine[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) mine[g][i] = g < 4 ? acc0[4 * g + i] : acc1[4 * (g - 4) + i];

  // The halves meet in LDS: the second half's waves leave their sums in the
  // X buffers, the first half's add them (first + second).
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(&xs[0][0][0]);   // [R rows][G][64 lanes]
  static_assert(sizeof(xs) >= sizeof(f32x4) * R * G * 64, "LDS for the halves' sums");
  if (pi == 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) red[(rho * G + g) * 64 + lane] = mine[g];
  }
  __syncthreads();
  if (pi == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) mine[g] += red[(rho * G + g) * 64 + lane];
  }

  auto store_y = [&](const f32x4* r) {
    float* yc = job.Y + 32 * tr + n;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 32 * (g >> 2) + 8 * (g & 3) + 4 * h + i;
        if (m < M) yc[(size_t)m * N] = r[g][i];
      }
  };
  if (a.S == 1 || displaced) {
    if (pi == 0 && active) store_y(mine);
    if (displaced) {
      wait_stores();
      __syncthreads();
      if (tid == 0) gemm_rescued_part(a, nb);
    }
    return;
  }

  // Split K as in k_gemm_q4, over R rows per workgroup row: the first half's
  // waves hold the sums; the second half's only take part in the barriers.
  constexpr size_t kPartBytes = (size_t)R * 8 * 64 * 16;
  const uint32_t part_bytes = (uint32_t)(kPartBytes * a.S);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.partial + (size_t)nb * a.S * (kPartBytes / 4), part_bytes);
  const uint32_t lane_off = (uint32_t)(rho * 8 * 64 + lane) * 16;
  constexpr int kStPol = LOCAL ? 0 : kCpolSc1;
  constexpr int kLdPol = LOCAL ? 1 : kCpolSc1;   // sc0: past this CU's L1
  if (pi == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, mine[g]), rs,
                                             lane_off + part * (uint32_t)kPartBytes + g * 1024, 0, kStPol);
  }
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    s_old = __hip_atomic_fetch_add(a.cnt + nb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag = 0;
    if (s_old == (uint32_t)a.S - 1) {
      s_flag = __hip_atomic_load(a.rescued + nb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (s_flag) {   // the row is already whole in Y: clear for the next call
        __hip_atomic_store(a.cnt + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.rescued + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __syncthreads();
  if (s_old != (uint32_t)a.S - 1 || s_flag || pi == 1) return;

  constexpr int PB = 2;                      // parts loaded per round trip (64 registers)
  f32x4 sum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) sum[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < a.S; p0 += PB) {
    f32x4 in[PB][G];
#pragma unroll
    for (int jj = 0; jj < PB; ++jj)
#pragma unroll
      for (int g = 0; g < G; ++g)
        in[jj][g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs, lane_off + (p0 + jj) * (uint32_t)kPartBytes + g * 1024, 0, kLdPol));
#pragma unroll
    for (int jj = 0; jj < PB; ++jj)
      if (p0 + jj < a.S)
#pragma unroll
        for (int g = 0; g < G; ++g) sum[g] += in[jj][g];
  }
  if (active) store_y(sum);
  if (tid == 0) __hip_atomic_store(a.cnt + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int KIND, bool TWO>
static hipError_t launch_kind(const GemmArgs& a, bool local, hipStream_t s) {
  const dim3 block(64 * kGemmWaves);
  const bool lc = local && a.S > 1;
  const dim3 grid = lc ? dim3(8 * ((a.NB + 7) / 8) * a.S) : dim3(a.NB, a.S);
  if constexpr (TWO) {
    if (lc) hipLaunchKernelGGL((k_gemm_q4h<KIND, kGemmDepth, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm_q4h<KIND, kGemmDepth, false>), grid, block, 0, s, a);
  } else {
    if (lc) hipLaunchKernelGGL((k_gemm_q4<KIND, false, kGemmDepth, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm_q4<KIND, false, kGemmDepth, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int kind, const GemmArgs& a, bool local, hipStream_t s) {
  const bool two = a.M > 32;
  if (kind == KIND_Q4_1) return two ? launch_kind<KIND_Q4_1, true>(a, local, s) : launch_kind<KIND_Q4_1, false>(a, local, s);
  if (kind == KIND_Q4_K) return two ? launch_kind<KIND_Q4_K, true>(a, local, s) : launch_kind<KIND_Q4_K, false>(a, local, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// XCD placement probe
// ---------------------------------------------------------------------------
constexpr int kProbeWgs = 64;
__device__ uint32_t g_xcc_probe[kProbeWgs];

__global__ void k_xcc_probe() {
  if (threadIdx.x == 0) g_xcc_probe[blockIdx.x] = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15;
}

// 1 when a 64-workgroup launch lands as XCD = (id + c) mod 8 for one c.  The
// probe runs once per device, on a non-blocking stream of the library's own,
// and its copy back is asynchronous on that stream: the caller's stream is
// never waited on.  While the caller's stream is being captured into a graph
// nothing is launched (the answer is 0 until the probe has run).
static std::once_flag g_probe_once[64];
static std::atomic<int> g_probe_result[64];

static int run_xcc_probe() {
  hipStream_t ps = nullptr;
  if (hipStreamCreateWithFlags(&ps, hipStreamNonBlocking) != hipSuccess) return 0;
  uint32_t* dev_ids = nullptr;
  int ok = 0;
  uint32_t ids[kProbeWgs];
  hipLaunchKernelGGL(k_xcc_probe, dim3(kProbeWgs), dim3(64), 0, ps);
  if (hipGetLastError() == hipSuccess && hipGetSymbolAddress((void**)&dev_ids, HIP_SYMBOL(g_xcc_probe)) == hipSuccess &&
      hipMemcpyAsync(ids, dev_ids, sizeof ids, hipMemcpyDeviceToHost, ps) == hipSuccess &&
      hipStreamSynchronize(ps) == hipSuccess) {
    ok = ids[0] < 8;
    for (int i = 0; i < kProbeWgs; ++i) ok &= ids[i] == (ids[0] + (uint32_t)i) % 8;
  }
  (void)hipStreamDestroy(ps);
  return ok;
}

int xcd_round_robin_known() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  return g_probe_result[dev].load() == 1 ? 1 : 0;
}

int xcd_round_robin(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return g_probe_result[dev].load() == 1 ? 1 : 0;
  std::call_once(g_probe_once[dev], [dev] { g_probe_result[dev].store(run_xcc_probe() ? 1 : 2); });
  return g_probe_result[dev].load() == 1 ? 1 : 0;
}

}  // namespace q4nx
