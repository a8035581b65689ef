// Q4NX dequant-GEMV kernels for gfx950: y[m] = W x[m] for M <= 8 activation rows.
//
// Decode reads every weight once per token and does two flops with it, so the
// kernel is bound by HBM bandwidth (Strata article, section 1: decode speed is
// set by the bytes of weights read per token).  The design keeps the weight
// stream as wide 16-byte nontemporal loads of whole chunks (metadata included),
// keeps x in registers (k_gemv_q4) or prepared once per workgroup in LDS (the
// default k_gemv_q4x / k_gemv_q8x), unpacks and scales in registers, leaves
// the ALU work per weight small enough to hide under the stream, and writes y
// with nontemporal stores (it is read by a later launch, never by this one).
//
// Work split: a workgroup of WAVES waves (4 for launches with many tile rows,
// 16 for small ones, where latency rather than bandwidth sets the time) owns
// WAVES/ks tile rows; the ks waves of one tile row take contiguous runs of its
// chunks, and their partial row sums meet in LDS, where one pass adds them in
// wave order.  No atomics: the result bits do not depend on timing.
#include "gemv_core.h"
#include "topk.h"

namespace q4nx {

template <int KIND, int M, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_q4(const GemvBatch b) {
  constexpr int CB = ChunkBytes<KIND>::value;
  constexpr int D = WAVES == 4 ? Q4Depth<M>::value : (M == 1 ? 2 : 1);
  __shared__ float red[WAVES][32][M];
  const GemvJob J = gemv_job(b);
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
      __builtin_nontemporal_store(v, &J.y[(size_t)m * J.ldy + 32 * t + r]);   // written once
    }
  }
}

// The same GEMV with the workgroup's activations prepared once in LDS.
//
// Per (activation row m, tile column c, group g) the record the dot chain takes
// (16 fp16 pairs, the scale f and sum x; gemv_core.h) is built once per
// workgroup instead of once per lane and chunk, and a wave's loop then reads
// it from LDS (lgkmcnt) while its chunk loads are counted alone on vmcnt.
// The activation loads are issued before the first chunk loads, so waiting for
// them never waits for a chunk; chunk loads are unconditional buffer loads
// (past the wave's run they read zero without memory traffic) running D chunks
// ahead of the products, and there is no branch inside a group of D steps, so
// every wait is for the chunk D steps back.  The host uses this kernel when
// the prepared records (M * TC * 8 per job, 72 bytes each) fit the LDS budget;
// otherwise k_gemv_q4.
//
// SL = 2 (or 1) splits each tile's 32 rows into two units of 16 (chunk slices
// 0-1 and 2-3: 2 KB of codes and 512 B of scales each), or four of 8, so a
// launch of few tile rows spreads over more compute units with no partial
// sums to combine.  (One CU draws only a few tens of GB/s from HBM, so a 2560-row
// projection, 80 tile rows, otherwise streams from 80 CUs.)
template <int KIND, int M, int WAVES, int D, int SL = 4, bool TOPK = false>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_q4x(const GemvBatch b) {
  constexpr int NT = 64 * WAVES;
  constexpr int XRP = 2;
  constexpr int CB = ChunkBytes<KIND>::value;
  constexpr int PARTS = 4 / SL;       // units per tile row
  constexpr int UR = 8 * SL;          // output rows per unit
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];
  __shared__ float red[WAVES][UR][M];
  constexpr bool kTurn = KIND == KIND_Q4_K;   // Q4_K metadata fetched whole, then handed out to the lanes
  constexpr bool kSlot = kTurn && SL == 4;    // the hand-out at 4 slices goes through an LDS slot per wave
  __shared__ __attribute__((aligned(16))) uint8_t tsl[kSlot ? WAVES : 1][kSlot ? 160 * SL : 16];
  const GemvJob J = gemv_job(b);
  const int ks = J.ks, rpw = WAVES / ks;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave / ks, part = wave % ks;
  const int NU = J.TR * PARTS;        // units of the job
  const int u0 = (blockIdx.x - J.wg_begin) * rpw;
  const int u = u0 + slot < NU ? u0 + slot : NU - 1;          // spare waves redo the last unit, unstored
  const int tr = u / PARTS, i0 = (u - tr * PARTS) * SL;
  const int TC = J.TC, g = lane & 7;
  const int c0 = part * TC / ks, c1 = (part + 1) * TC / ks;
  const int R = M * TC * 8;

  // 1. activations: record r = (m * TC + c) * 8 + g holds the 32 bf16 at
  // x[m][32 * (8c + g)]; four consecutive lanes build it, part d = q & 3 of
  // part index q taking x[m][32 * (8c + g) + 8d .. + 7] (16 bytes)
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(J.x, (uint32_t)(((M - 1) * J.ldx + TC * 256) * 2));
  auto xpart_off = [&](int q) {
    const int r = q >> 2, m = r / (TC * 8), rem = r - m * TC * 8;
    return (uint32_t)(m * J.ldx + 32 * rem + 8 * (q & 3)) * 2;   // q >= 4R: m >= M, past the resource
  };
  u32x4 xr[XRP];
#pragma unroll
  for (int i = 0; i < XRP; ++i)
    xr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xpart_off(tid + NT * i), 0, 0));
  // 2. the first D chunks of the wave's run
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(J.w + ((size_t)tr * TC + c0) * CB, (uint32_t)((c1 - c0) * CB));
  Q4Chunk<KIND, SL> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if constexpr (kTurn) q4k_load_rs_whole<SL>(wrs, j * CB, lane, ring[j], i0);
    else q4_load_rs<KIND>(wrs, j * CB, lane, ring[j], i0);
  }
  // 3. records to LDS: pairs at xl[16 r], (f, X) at xl[16 R + 2 r]
  float* sums = reinterpret_cast<float*>(xl + 16 * R);
  auto put = [&](int q, const u32x4 v) {   // the four lanes of a record come together
    uint32_t pr[4];
    float f, X;
    x_record_part(v, pr, f, X);
    const int r = q >> 2;
    if (r < R) {
      *reinterpret_cast<u32x4*>(xl + 16 * r + 4 * (q & 3)) = u32x4{pr[0], pr[1], pr[2], pr[3]};
      if ((q & 3) == 0) {
        sums[2 * r] = f;
        sums[2 * r + 1] = X;
      }
    }
  };
#pragma unroll
  for (int i = 0; i < XRP; ++i) put(tid + NT * i, xr[i]);
  // long-K launches: the parts past the first XRP per thread, loaded and built
  // in turn; NS at a time for three or more rows (whose staging is long enough
  // for the round trips to add up; at one or two rows the registers cost more)
  constexpr int NS = M >= 3 ? 4 : 1;
  for (int q0 = tid + NT * XRP; q0 < 4 * R; q0 += NS * NT) {
    u32x4 v[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i)
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xpart_off(q0 + NT * i), 0, 0));
#pragma unroll
    for (int i = 0; i < NS; ++i) put(q0 + NT * i, v[i]);
  }
  __syncthreads();

  const Q4Consts k = q4_consts();
  float acc[SL][M];
#pragma unroll
  for (int i = 0; i < SL; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;
  auto step = [&](int j, int c) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kTurn) q4k_turn<SL>(tsl[kSlot ? wave : 0], lane, ring[j]);
    XRec<M> xp;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int r = (m * TC + c) * 8 + g;
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
    q4_compute<KIND, M, SL>(ring[j], xp, k, acc);
    if constexpr (kTurn) q4k_load_rs_whole<SL>(wrs, (uint32_t)(c + D - c0) * CB, lane, ring[j], i0);
    else q4_load_rs<KIND>(wrs, (uint32_t)(c + D - c0) * CB, lane, ring[j], i0);
  };
  int base = c0;
  for (; base + D <= c1; base += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) step(j, base + j);
  }
#pragma unroll
  for (int j = 0; j + 1 < D; ++j)
    if (base + j < c1) step(j, base + j);

  q4_lane_reduce<M>(acc);
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < SL; ++i)
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave][8 * i + (lane >> 3)][m] = acc[i][m];
  }
  __syncthreads();
  __shared__ float tv[TOPK ? M : 1][TOPK ? kTopkRows : 1];
  for (int idx = tid; idx < rpw * UR * M; idx += NT) {
    const int s = idx / (UR * M), rem = idx - s * UR * M;
    const int r = rem / M, m = rem - r * M;
    const int t = u0 + s;   // unit: tile row t / PARTS, rows UR * (t % PARTS) + r of it
    if (t < NU) {
      float v = 0.f;
      for (int p = 0; p < ks; ++p) v += red[s * ks + p][r][m];
      if constexpr (TOPK) {
        tv[m][s * UR + r] = v;
        if (J.y) J.y[(size_t)m * J.ldy + UR * t + r] = v;
      } else {
        __builtin_nontemporal_store(v, &J.y[(size_t)m * J.ldy + UR * t + r]);   // written once
      }
    }
  }
  if constexpr (TOPK) {
    __shared__ uint32_t s_flag;
    __syncthreads();
    const int nr = (NU - u0 < rpw ? NU - u0 : rpw) * UR;
    topk_epilogue<M, WAVES>(b.tk, tv, nr, (uint32_t)(UR * u0), &s_flag);
  }
}

// k_gemv_q4x for M = 2 .. 8 activation rows with the products on the matrix
// cores (q4_compute_mfma).  The dot chain's work grows with M (16 dot2 per
// group and row); here a group's products for four activation rows are 8
// small MFMAs, so the vector work per chunk stays that of one row: signed code
// pairs, and per group and row two FMAs.  Each lane reads one record per block
// of four rows instead of M, which also frees the registers the dot chain held
// for them.  Records, staging, chunk ring and units are those of k_gemv_q4x;
// only the lanes' places in a slice differ (lane l holds row
// (l & 3) + 4 ((l >> 4) & 1) and group ((l >> 2) & 3) + 4 (l >> 5) instead of
// row l >> 3 and group l & 7), so its chunk loads are those of k_gemv_q4x's
// lane 8 row + group, and the 8 lanes of one row (one per group) meet through
// xor-shuffles over lane bits 2, 3 and 5.  At M = 1 the dot chain is faster
// (decode step 1.08 against 1.045 ms, Q4_K lm_head 4.9 against 5.4 TB/s).
template <int KIND, int M, int WAVES, int D, int SL, bool TOPK = false>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_q4m(const GemvBatch b) {
  constexpr int NT = 64 * WAVES;
  constexpr int XRP = 4;   // staging parts per thread loaded before the first chunks
  constexpr int CB = ChunkBytes<KIND>::value;
  constexpr int PARTS = 4 / SL;       // units per tile row
  constexpr int UR = 8 * SL;          // output rows per unit
  constexpr int NB = (M + 3) / 4;     // blocks of four activation rows
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];
  __shared__ float red[WAVES][UR][M];
  const GemvJob J = gemv_job(b);
  const int ks = J.ks, rpw = WAVES / ks;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave / ks, part = wave % ks;
  const int NU = J.TR * PARTS;
  const int u0 = (blockIdx.x - J.wg_begin) * rpw;
  const int u = u0 + slot < NU ? u0 + slot : NU - 1;          // spare waves redo the last unit, unstored
  const int tr = u / PARTS, i0 = (u - tr * PARTS) * SL;
  const int TC = J.TC;
  const int c0 = part * TC / ks, c1 = (part + 1) * TC / ks;
  const int R = M * TC * 8;
  // A quarter-wave (16 lanes, four blocks) takes rows 4 h .. 4 h + 3 and groups
  // 4 v .. 4 v + 3 of a slice, h = bit 4 and v = bit 5 of the lane: four
  // 64-byte runs, one per row, for each 16-byte load instruction.
  const int col = lane & 3;                             // the lane's activation row in a block
  const int lrow = col + 4 * ((lane >> 4) & 1);         // its weight row in a slice
  const int gg = ((lane >> 2) & 3) + 4 * (lane >> 5);   // its group in a tile column
  const int lidx = 8 * lrow + gg;                       // k_gemv_q4x's lane for that (row, group)

  // 1.-3. activations staged as records, as in k_gemv_q4x, with more of the
  // staging loads in flight (this kernel has the registers): 4 parts per
  // thread ahead of the chunk loads, then 4 at a time.  8B block against 2
  // and 1 (at M = 2): M = 2 1.355 -> 1.295 ms, M = 4 1.71 -> 1.60 ms.
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(J.x, (uint32_t)(((M - 1) * J.ldx + TC * 256) * 2));
  auto xpart_off = [&](int q) {
    const int r = q >> 2, m = r / (TC * 8), rem = r - m * TC * 8;
    return (uint32_t)(m * J.ldx + 32 * rem + 8 * (q & 3)) * 2;   // q >= 4R: m >= M, past the resource
  };
  u32x4 xr[XRP];
#pragma unroll
  for (int i = 0; i < XRP; ++i)
    xr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xpart_off(tid + NT * i), 0, 0));
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(J.w + ((size_t)tr * TC + c0) * CB, (uint32_t)((c1 - c0) * CB));
  Q4Chunk<KIND, SL> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) q4_load_rs<KIND>(wrs, j * CB, lidx, ring[j], i0);
  float* sums = reinterpret_cast<float*>(xl + 16 * R);
  auto put = [&](int q, const u32x4 v) {
    uint32_t pr[4];
    float f, X;
    x_record_part(v, pr, f, X);
    const int r = q >> 2;
    if (r < R) {
      *reinterpret_cast<u32x4*>(xl + 16 * r + 4 * (q & 3)) = u32x4{pr[0], pr[1], pr[2], pr[3]};
      if ((q & 3) == 0) {
        sums[2 * r] = f;
        sums[2 * r + 1] = X;
      }
    }
  };
#pragma unroll
  for (int i = 0; i < XRP; ++i) put(tid + NT * i, xr[i]);
  constexpr int NS = 4;
  for (int q0 = tid + NT * XRP; q0 < 4 * R; q0 += NS * NT) {
    u32x4 v[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i)
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xpart_off(q0 + NT * i), 0, 0));
#pragma unroll
    for (int i = 0; i < NS; ++i) put(q0 + NT * i, v[i]);
  }
  __syncthreads();

  const Q4Consts k = q4_consts();
  float acc[SL][M];
#pragma unroll
  for (int i = 0; i < SL; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;
  auto step = [&](int j, int c) {
    __builtin_amdgcn_sched_barrier(0);
    uint32_t pa[NB][16];
    float fv[NB][4], Xv[NB][4];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      // rows past M repeat row M - 1 (in bounds); their results are dropped
      const int ma = 4 * blk + col < M ? 4 * blk + col : M - 1;
      const int ra = (ma * TC + c) * 8 + gg;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xl + 16 * ra + 4 * d);
        pa[blk][4 * d] = v.x;
        pa[blk][4 * d + 1] = v.y;
        pa[blk][4 * d + 2] = v.z;
        pa[blk][4 * d + 3] = v.w;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int mt = 4 * blk + t < M ? 4 * blk + t : M - 1;
        const int rt = (mt * TC + c) * 8 + gg;
        const u32x2 fx = *reinterpret_cast<const u32x2*>(sums + 2 * rt);
        fv[blk][t] = __uint_as_float(fx.x);
        Xv[blk][t] = __uint_as_float(fx.y);
      }
    }
    q4_compute_mfma<KIND, M, NB, SL>(ring[j], pa, fv, Xv, k, acc);
    q4_load_rs<KIND>(wrs, (uint32_t)(c + D - c0) * CB, lidx, ring[j], i0);
  };
  int base = c0;
  for (; base + D <= c1; base += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) step(j, base + j);
  }
#pragma unroll
  for (int j = 0; j + 1 < D; ++j)
    if (base + j < c1) step(j, base + j);

  // the 8 groups of a row: the lanes that differ in bits 2, 3 and 5
#pragma unroll
  for (int i = 0; i < SL; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[i][m];
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 32);
      acc[i][m] = v;
    }
  if (gg == 0) {
#pragma unroll
    for (int i = 0; i < SL; ++i)
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave][8 * i + lrow][m] = acc[i][m];
  }
  __syncthreads();
  __shared__ float tv[TOPK ? M : 1][TOPK ? kTopkRows : 1];
  for (int idx = tid; idx < rpw * UR * M; idx += NT) {
    const int s = idx / (UR * M), rem = idx - s * UR * M;
    const int r = rem / M, m = rem - r * M;
    const int t = u0 + s;   // unit: tile row t / PARTS, rows UR * (t % PARTS) + r of it
    if (t < NU) {
      float v = 0.f;
      for (int p = 0; p < ks; ++p) v += red[s * ks + p][r][m];
      if constexpr (TOPK) {
        tv[m][s * UR + r] = v;
        if (J.y) J.y[(size_t)m * J.ldy + UR * t + r] = v;
      } else {
        __builtin_nontemporal_store(v, &J.y[(size_t)m * J.ldy + UR * t + r]);   // written once
      }
    }
  }
  if constexpr (TOPK) {   // the same pick as k_gemv_q4x's
    __shared__ uint32_t s_flag;
    __syncthreads();
    const int nr = (NU - u0 < rpw ? NU - u0 : rpw) * UR;
    topk_epilogue<M, WAVES>(b.tk, tv, nr, (uint32_t)(UR * u0), &s_flag);
  }
}

// Q8 with the workgroup's activations staged once in LDS and an unconditional
// buffer-load chunk ring: the same structure as k_gemv_q4x, so a step waits
// only for its own chunk.
//
// Lane mapping: each 16-byte load instruction of a wave reads eight whole
// 128-byte lines of the code region (lanes 8a .. 8a+7 one line each), so no
// line is fetched into the CU more than once.
//   layout A (byte 32k + r), lane 8g + s, load i: byte 1024g + 128i + 16s =
//     column 32g + 4i + s/2, rows 16(s&1) .. +15.  The lane keeps group g and
//     row half s&1.
//   layout B, lane 8a + s, load i: byte 4096h + 512(g0 + i/4) + 128(i%4) + 16s
//     with h = a&1, g0 = 2(a>>1) = column 32(g0 + i/4) + 8(i%4) + s, rows
//     16h .. +15.  The lane keeps row half h and groups g0 (loads 0-3) and
//     g0 + 1 (loads 4-7).
// The activation rows sit in LDS permuted inside every 256-column span so that
// a lane's eight columns, in load order, are one 16-byte read.  The chunk's
// 512-byte scale region is fetched with one 8-byte load per lane and turned
// around in a per-wave LDS slot ([group][row]), from which a lane reads the 16
// scales of each of its groups (rows of its half) as two 16-byte reads.
template <int KIND>
struct Q8Lines {
  static constexpr bool kA = KIND == KIND_Q8_A;
  static constexpr int kGroups = kA ? 1 : 2;        // groups per lane
  static constexpr int kHalfBit = kA ? 0 : 3;       // lane bit that selects the row half
  __device__ static __forceinline__ uint32_t piece(int lane, int i) {
    const int a = lane >> 3, s = lane & 7;
    if constexpr (kA) return 1024 * a + 128 * i + 16 * s;
    else return 4096 * (a & 1) + 512 * (2 * (a >> 1) + (i >> 2)) + 128 * (i & 3) + 16 * s;
  }
  __device__ static __forceinline__ int half(int lane) { return (lane >> kHalfBit) & 1; }
  __device__ static __forceinline__ int group0(int lane) { return kA ? lane >> 3 : 2 * (lane >> 4); }
  // LDS position (bf16 units, inside the span) of the lane's eight columns
  __device__ static __forceinline__ int xread(int lane) {
    return kA ? 32 * (lane >> 3) + 8 * ((lane >> 1) & 3) : 64 * (lane >> 4) + 8 * (lane & 7);
  }
  // LDS position of column u (0..255) of a span
  __device__ static __forceinline__ int xperm(int u) {
    const int g = u >> 5, w = u & 31;
    if constexpr (kA) return 32 * g + 8 * (w & 3) + (w >> 2);
    else return 64 * (g >> 1) + 8 * (w & 7) + 4 * (g & 1) + (w >> 3);
  }
};

struct Q8ChunkX {
  u32x4 pc[8];
  u32x2 dp;   // scales d(r, g) with 8r + g = 4 lane .. 4 lane + 3
};

template <int KIND>
__device__ __forceinline__ void q8x_load_rs(__amdgpu_buffer_rsrc_t rs, uint32_t off, int lane, Q8ChunkX& c) {
  constexpr int kNt = 2;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    c.pc[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rs, off + Q8Lines<KIND>::piece(lane, i), 0, kNt));
  c.dp = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 8192 + 8 * lane, 0, kNt));
}

// acc[rho][m] += sum over the lane's groups q of d(16h + rho, g0 + q) *
// sum over the group's loads i of code(16h + rho, column of load i) * x[m][i].
// Every product of an int8 code and a bf16 is exact in fp32.
template <int NG, int M>
__device__ __forceinline__ void q8x_compute(const u32x4 (&pc)[8], const uint32_t (&dv)[NG][8],
                                            const Q8XRaw<M>& xr, float (&acc)[16][M]) {
  float xf[M][8];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xf[m][2 * t] = bf16lo(xr.v[m][t]);
      xf[m][2 * t + 1] = bf16hi(xr.v[m][t]);
    }
  constexpr int L = 8 / NG;   // loads per group
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    float part[16][M];
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) part[r][m] = 0.f;
#pragma unroll
    for (int i = q * L; i < (q + 1) * L; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float cf = (float)(int8_t)(pc[i][r >> 2] >> (8 * (r & 3)));
#pragma unroll
        for (int m = 0; m < M; ++m) part[r][m] = fmaf(cf, xf[m][i], part[r][m]);
      }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float d = (r & 1) ? bf16hi(dv[q][r >> 1]) : bf16lo(dv[q][r >> 1]);
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = fmaf(d, part[r][m], acc[r][m]);
    }
  }
}

template <int KIND, int M, int WAVES, int D, bool TOPK = false>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_q8x(const GemvBatch b) {
  using Map = Q8Lines<KIND>;
  constexpr int NG = Map::kGroups, HB = Map::kHalfBit;
  constexpr int NT = 64 * WAVES;
  constexpr int XRP8 = 4;
  constexpr int CB = 8704;
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];
  __shared__ __attribute__((aligned(16))) uint16_t dsl[WAVES][8 * 32];
  __shared__ float red[WAVES][32][M];
  const GemvJob J = gemv_job(b);
  const int ks = J.ks, rpw = WAVES / ks;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave / ks, part = wave % ks;
  const int tr0 = (blockIdx.x - J.wg_begin) * rpw;
  const int tr = tr0 + slot < J.TR ? tr0 + slot : J.TR - 1;
  const int TC = J.TC, K = TC * 256;
  const int c0 = part * TC / ks, c1 = (part + 1) * TC / ks;
  const int h = Map::half(lane), g0 = Map::group0(lane);
  const int NP = M * TC * 32;   // 16-byte pieces of the M activation rows

  // 1. activations: piece p of row m holds x[m][8 p' .. 8 p' + 7] (p' = p - 32 TC m)
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(J.x, (uint32_t)(((M - 1) * J.ldx + K) * 2));
  u32x4 xr[XRP8];
#pragma unroll
  for (int p = 0; p < XRP8; ++p) {
    const int pc = tid + NT * p, m = pc / (TC * 32), pp = pc - m * TC * 32;
    xr[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          xrs, (uint32_t)(m * J.ldx + 8 * pp) * 2, 0, 0));
  }
  // 2. the first D chunks of the wave's run
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(J.w + ((size_t)tr * TC + c0) * CB, (uint32_t)((c1 - c0) * CB));
  Q8ChunkX ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) q8x_load_rs<KIND>(wrs, j * CB, lane, ring[j]);
  // 3. rows to LDS, permuted inside each 256-column span: row m at bf16 m * K
  uint16_t* xh = reinterpret_cast<uint16_t*>(xl);
#pragma unroll
  for (int p = 0; p < XRP8; ++p) {
    const int pc = tid + NT * p;
    if (pc < NP) {
      const int m = pc / (TC * 32), pp = pc - m * TC * 32;
      const int span = m * K + 256 * (pp >> 5), u0 = 8 * (pp & 31);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = xr[p][e >> 1];
        xh[span + Map::xperm(u0 + e)] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
      }
    }
  }
  __syncthreads();

  float acc[16][M];
#pragma unroll
  for (int r = 0; r < 16; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
  uint16_t* ds = dsl[wave];
  const int dr = lane >> 1, dg0 = 4 * (lane & 1);
  const int xoff = Map::xread(lane);
  auto step = [&](int j, int c) {
    __builtin_amdgcn_sched_barrier(0);
    // scales: (row dr, groups dg0 .. dg0+3) -> slot [group][row]; the wave's
    // LDS operations run in order, so the reads below see every lane's writes
    const u32x2 dp = ring[j].dp;
    ds[(dg0 + 0) * 32 + dr] = (uint16_t)(dp.x & 0xFFFFu);
    ds[(dg0 + 1) * 32 + dr] = (uint16_t)(dp.x >> 16);
    ds[(dg0 + 2) * 32 + dr] = (uint16_t)(dp.y & 0xFFFFu);
    ds[(dg0 + 3) * 32 + dr] = (uint16_t)(dp.y >> 16);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    u32x4 pcs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pcs[i] = ring[j].pc[i];
    uint32_t dv[NG][8];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const u32x4 d0 = *reinterpret_cast<const u32x4*>(ds + (g0 + q) * 32 + 16 * h);
      const u32x4 d1 = *reinterpret_cast<const u32x4*>(ds + (g0 + q) * 32 + 16 * h + 8);
      dv[q][0] = d0.x; dv[q][1] = d0.y; dv[q][2] = d0.z; dv[q][3] = d0.w;
      dv[q][4] = d1.x; dv[q][5] = d1.y; dv[q][6] = d1.z; dv[q][7] = d1.w;
    }
    Q8XRaw<M> xv;
#pragma unroll
    for (int m = 0; m < M; ++m)
      xv.v[m] = *reinterpret_cast<const u32x4*>(xh + m * K + 256 * c + xoff);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // the slot's reads come before
    __builtin_amdgcn_wave_barrier();                          // the next step's writes
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    q8x_compute<NG, M>(pcs, dv, xv, acc);
    q8x_load_rs<KIND>(wrs, (uint32_t)(c + D - c0) * CB, lane, ring[j]);
  };
  int base = c0;
  for (; base + D <= c1; base += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) step(j, base + j);
  }
#pragma unroll
  for (int j = 0; j + 1 < D; ++j)
    if (base + j < c1) step(j, base + j);

  // sum over the 32 lanes of each row half (every lane bit but HB)
#pragma unroll
  for (int r = 0; r < 16; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int bit = 0; bit < 6; ++bit)
        if (bit != HB) v += __shfl_xor(v, 1 << bit);
      acc[r][m] = v;
    }
  if ((lane & ~(1 << HB)) == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave][16 * h + r][m] = acc[r][m];
  }
  __syncthreads();
  __shared__ float tv[TOPK ? M : 1][TOPK ? kTopkRows : 1];
  for (int idx = tid; idx < rpw * 32 * M; idx += NT) {
    const int s = idx / (32 * M), rem = idx - s * 32 * M;
    const int r = rem / M, m = rem - r * M;
    const int t = tr0 + s;
    if (t < J.TR) {
      float v = 0.f;
      for (int p = 0; p < ks; ++p) v += red[s * ks + p][r][m];
      if constexpr (TOPK) {
        tv[m][s * 32 + r] = v;
        if (J.y) J.y[(size_t)m * J.ldy + 32 * t + r] = v;
      } else {
        __builtin_nontemporal_store(v, &J.y[(size_t)m * J.ldy + 32 * t + r]);   // written once
      }
    }
  }
  if constexpr (TOPK) {
    __shared__ uint32_t s_flag;
    __syncthreads();
    const int nr = (J.TR - tr0 < rpw ? J.TR - tr0 : rpw) * 32;
    topk_epilogue<M, WAVES>(b.tk, tv, nr, (uint32_t)(32 * tr0), &s_flag);
  }
}

template <int KIND, int M, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_q8(const GemvBatch b) {
  constexpr int CB = 8704;
  __shared__ float red[WAVES][32][M];
  const GemvJob J = gemv_job(b);
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
      __builtin_nontemporal_store(v, &J.y[(size_t)m * J.ldy + 32 * t + r]);   // written once
    }
  }
}

// ===========================================================================
// launcher
// ===========================================================================
// Chunks in flight per wave in k_gemv_q4x: 2, or 1 for M > 1 in 16-wave
// workgroups, whose waves hold at most 128 registers.  (Deeper rings cost
// occupancy in the large launches and measured slower over a decode step.)
#ifndef Q4NX_GEMVX_DEPTH
#define Q4NX_GEMVX_DEPTH 2
#endif
template <int M, int WAVES>
struct GemvXDepth {
  static constexpr int value = (WAVES == 16 && M > 1) ? 1 : Q4NX_GEMVX_DEPTH;
};

// Launch of a prepared-activation kernel; more than 64 KB of dynamic LDS is
// declared to the runtime first.
template <typename F>
static void launch_xl(F* kern, int n_wg, int threads, int xl_bytes, hipStream_t s, const GemvBatch& b) {
  if (xl_bytes > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, xl_bytes);
  hipLaunchKernelGGL(kern, dim3(n_wg), dim3(threads), xl_bytes, s, b);
}

// The top-k GEMV: 4-wave workgroups, prepared activations, M <= 4.
template <int KIND, int M>
static hipError_t launch_topk(const GemvBatch& b, int n_wg, int xl_bytes, hipStream_t s) {
  constexpr int D = GemvXDepth<M, 4>::value;
  if constexpr ((KIND == KIND_Q4_1 || KIND == KIND_Q4_K) && M >= kGemvMfmaMinM && M >= 2) {
    // the products of q4nx_gemv at this M, so the picked values are its logits bit for bit
    if (b.sl == 2) launch_xl(k_gemv_q4m<KIND, M, 4, D, 2, true>, n_wg, 256, xl_bytes, s, b);
    else if (b.sl == 1) launch_xl(k_gemv_q4m<KIND, M, 4, D, 1, true>, n_wg, 256, xl_bytes, s, b);
    else launch_xl(k_gemv_q4m<KIND, M, 4, D, 4, true>, n_wg, 256, xl_bytes, s, b);
  } else if constexpr (KIND == KIND_Q4_1 || KIND == KIND_Q4_K) {
    if (b.sl == 2) launch_xl(k_gemv_q4x<KIND, M, 4, D, 2, true>, n_wg, 256, xl_bytes, s, b);
    else if (b.sl == 1) launch_xl(k_gemv_q4x<KIND, M, 4, D, 1, true>, n_wg, 256, xl_bytes, s, b);
    else launch_xl(k_gemv_q4x<KIND, M, 4, D, 4, true>, n_wg, 256, xl_bytes, s, b);
  } else {
    hipLaunchKernelGGL((k_gemv_q8x<KIND, M, 4, M == 1 ? 2 : 1, true>), dim3(n_wg), dim3(256), xl_bytes, s, b);
  }
  return hipGetLastError();
}

template <int KIND>
static hipError_t launch_topk_m(int M, const GemvBatch& b, int n_wg, int xl, hipStream_t s) {
  switch (M) {
    case 1: return launch_topk<KIND, 1>(b, n_wg, xl, s);
    case 2: return launch_topk<KIND, 2>(b, n_wg, xl, s);
    case 3: return launch_topk<KIND, 3>(b, n_wg, xl, s);
    case 4: return launch_topk<KIND, 4>(b, n_wg, xl, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_topk(int kind, int M, const GemvBatch& b, int n_wg, int xl_bytes, hipStream_t s) {
  if (xl_bytes <= 0) return hipErrorInvalidValue;
  switch (kind) {
    case KIND_Q4_1: return launch_topk_m<KIND_Q4_1>(M, b, n_wg, xl_bytes, s);
    case KIND_Q4_K: return launch_topk_m<KIND_Q4_K>(M, b, n_wg, xl_bytes, s);
    case KIND_Q8_A: return launch_topk_m<KIND_Q8_A>(M, b, n_wg, xl_bytes, s);
    case KIND_Q8_B: return launch_topk_m<KIND_Q8_B>(M, b, n_wg, xl_bytes, s);
  }
  return hipErrorInvalidValue;
}

template <int KIND, int M, int WAVES>
static hipError_t launch_one(const GemvBatch& b, int n_wg, int xl_bytes, hipStream_t s) {
  if constexpr (KIND == KIND_Q4_1 || KIND == KIND_Q4_K) {
    constexpr int D = GemvXDepth<M, WAVES>::value;
    if constexpr (M >= kGemvMfmaMinM && M >= 2) {   // the matrix-core products
      if (xl_bytes > 0) {
        if (b.sl == 2) launch_xl(k_gemv_q4m<KIND, M, WAVES, D, 2>, n_wg, 64 * WAVES, xl_bytes, s, b);
        else if (b.sl == 1) launch_xl(k_gemv_q4m<KIND, M, WAVES, D, 1>, n_wg, 64 * WAVES, xl_bytes, s, b);
        else launch_xl(k_gemv_q4m<KIND, M, WAVES, D, 4>, n_wg, 64 * WAVES, xl_bytes, s, b);
        return hipGetLastError();
      }
    }
    if (xl_bytes > 0 && b.sl == 2)
      launch_xl(k_gemv_q4x<KIND, M, WAVES, D, 2>, n_wg, 64 * WAVES, xl_bytes, s, b);
    else if (xl_bytes > 0 && b.sl == 1)
      launch_xl(k_gemv_q4x<KIND, M, WAVES, D, 1>, n_wg, 64 * WAVES, xl_bytes, s, b);
    else if (xl_bytes > 0)
      launch_xl(k_gemv_q4x<KIND, M, WAVES, D, 4>, n_wg, 64 * WAVES, xl_bytes, s, b);
    else
      hipLaunchKernelGGL((k_gemv_q4<KIND, M, WAVES>), dim3(n_wg), dim3(64 * WAVES), 0, s, b);
  } else {
    if (xl_bytes > 0)
      // two chunks in flight per wave at M = 1, except layout B's 16-wave
      // variant, whose two scale groups per lane leave no registers for it
      hipLaunchKernelGGL((k_gemv_q8x<KIND, M, WAVES, M == 1 && !(KIND == KIND_Q8_B && WAVES == 16) ? 2 : 1>), dim3(n_wg),
                         dim3(64 * WAVES), xl_bytes, s, b);
    else
      hipLaunchKernelGGL((k_gemv_q8<KIND, M, WAVES>), dim3(n_wg), dim3(64 * WAVES), 0, s, b);
  }
  return hipGetLastError();
}

template <int KIND, int WAVES>
static hipError_t launch_m(int M, const GemvBatch& b, int n_wg, int xl, hipStream_t s) {
  switch (M) {
    case 1: return launch_one<KIND, 1, WAVES>(b, n_wg, xl, s);
    case 2: return launch_one<KIND, 2, WAVES>(b, n_wg, xl, s);
    case 3: return launch_one<KIND, 3, WAVES>(b, n_wg, xl, s);
    case 4: return launch_one<KIND, 4, WAVES>(b, n_wg, xl, s);
    case 5: return launch_one<KIND, 5, WAVES>(b, n_wg, xl, s);
    case 6: return launch_one<KIND, 6, WAVES>(b, n_wg, xl, s);
    case 7: return launch_one<KIND, 7, WAVES>(b, n_wg, xl, s);
    case 8: return launch_one<KIND, 8, WAVES>(b, n_wg, xl, s);
  }
  return hipErrorInvalidValue;
}

template <int WAVES>
static hipError_t launch_w(int kind, int M, const GemvBatch& b, int n_wg, int xl, hipStream_t s) {
  switch (kind) {
    case KIND_Q4_1: return launch_m<KIND_Q4_1, WAVES>(M, b, n_wg, xl, s);
    case KIND_Q4_K: return launch_m<KIND_Q4_K, WAVES>(M, b, n_wg, xl, s);
    case KIND_Q8_A: return launch_m<KIND_Q8_A, WAVES>(M, b, n_wg, xl, s);
    case KIND_Q8_B: return launch_m<KIND_Q8_B, WAVES>(M, b, n_wg, xl, s);
  }
  return hipErrorInvalidValue;
}

template <int KIND>
static hipError_t launch_small(int M, const GemvBatch& b, int n_wg, int xl, hipStream_t s) {
  if (M == 1) return launch_one<KIND, 1, 16>(b, n_wg, xl, s);
  if (M == 2) return launch_one<KIND, 2, 16>(b, n_wg, xl, s);
  return hipErrorInvalidValue;
}

// Dynamic LDS a 4-wave workgroup may take: the device's limit (160 KB on
// gfx950) less the kernels' static arrays (at most 8 KB; see gemv_xl_bytes for
// 8 and 16 waves).
static int gemv_lds_budget() {
  static const int budget = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      v = 65536;
    return v - 8192 > 65536 ? v - 8192 : 65536;
  }();
  return budget;
}

int gemv_xl_bytes(int kind, int M, int waves, int max_tc) {
#if defined(Q4NX_GEMV_NO_XLDS)
  return 0;
#endif
  if (kind == KIND_Q8_A || kind == KIND_Q8_B) {   // raw rows, four 16-byte pieces per thread
    const int NP = M * max_tc * 32;
    if (NP > 4 * 64 * waves) return 0;
    return NP * 16 <= 65536 ? NP * 16 : 0;
  }
  if (kind != KIND_Q4_1 && kind != KIND_Q4_K) return 0;
  const int bytes = M * max_tc * 8 * 72;
  // 8-wave workgroups keep up to 9 KB of static arrays (the reduction buffer
  // and Q4_K's metadata slots at M = 4, whole tiles): 4 KB more held back
  const int lim = waves == 4 ? gemv_lds_budget() : waves == 8 ? gemv_lds_budget() - 4096 : 65536;
  return bytes <= lim ? bytes : 0;
}

// Eight-wave workgroups (two waves per SIMD, up to 256 registers): q4 kinds
// at M = 3 and 4.
template <int KIND>
static hipError_t launch_mid(int M, const GemvBatch& b, int n_wg, int xl, hipStream_t s) {
  if (M == 3) return launch_one<KIND, 3, 8>(b, n_wg, xl, s);
  if (M == 4) return launch_one<KIND, 4, 8>(b, n_wg, xl, s);
  return hipErrorInvalidValue;
}

// 16-wave workgroups hold at most 128 registers per lane, so they are used
// for M <= 2 only.
hipError_t launch_gemv(int kind, int M, int waves, const GemvBatch& b, int n_wg, int xl_bytes,
                       hipStream_t s) {
  if (waves == 4) return launch_w<4>(kind, M, b, n_wg, xl_bytes, s);
  if (waves == 8 && xl_bytes > 0) {
    if (kind == KIND_Q4_1) return launch_mid<KIND_Q4_1>(M, b, n_wg, xl_bytes, s);
    if (kind == KIND_Q4_K) return launch_mid<KIND_Q4_K>(M, b, n_wg, xl_bytes, s);
  }
  if (waves == 16 && M <= 2) {
    switch (kind) {
      case KIND_Q4_1: return launch_small<KIND_Q4_1>(M, b, n_wg, xl_bytes, s);
      case KIND_Q4_K: return launch_small<KIND_Q4_K>(M, b, n_wg, xl_bytes, s);
      case KIND_Q8_A: return launch_small<KIND_Q8_A>(M, b, n_wg, xl_bytes, s);
      case KIND_Q8_B: return launch_small<KIND_Q8_B>(M, b, n_wg, xl_bytes, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace q4nx
