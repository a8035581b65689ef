// Device-side arguments of the block GEMM and its workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4nx {

// One weight of a block-GEMM launch: its tile rows are workgroup rows
// nb0 .. nb0 + ceil(TR / 8) - 1 of the grid.
struct GemmJob {
  const uint8_t* w;
  float* Y;         // [M][32 * TR]
  int32_t TR, nb0;
};

constexpr int kGemmMaxJobs = 8;

struct GemmArgs {
  GemmJob job[kGemmMaxJobs];
  int32_t n_jobs;
  const uint16_t* X;
  float* partial;   // [NB][S][8 waves][8 groups][64 lanes][4] fp32 when S > 1
  uint32_t* cnt;    // [NB] parts arrived (of kGemmCntWords); zero between calls
  uint32_t* claim;  // [groups] XCD slots taken in each group of 8 workgroups; zero between calls
  uint32_t* rescued;   // [NB] 1 when a row was computed whole by a displaced workgroup; zero between calls
  uint32_t* diag;   // [0]: workgroups that found their XCD slot taken (never reset by the kernels)
  int32_t TC, M, S, NB;
  int32_t test_mode;   // 0; 1: every odd group's workgroups act as displaced (tests of that path)
};

// Tile rows per workgroup of the block GEMM: 8 for M <= 32 (a wave per row),
// 4 for M > 32 (a wave per row and K half).
constexpr int kGemmRowsPerWg = 8;
constexpr int kGemmRowsHalves = 4;
inline int gemm_rows(int M) { return M > 32 ? kGemmRowsHalves : kGemmRowsPerWg; }

// Workgroups a launch aims for (one per CU), and the fewest tile columns a K
// part may hold (so the fp32 partial tiles stay small next to the weights
// they summarise).
#ifndef Q4NX_GEMM_WG_TARGET
#define Q4NX_GEMM_WG_TARGET 256
#endif
#ifndef Q4NX_GEMM_MIN_COLS
#define Q4NX_GEMM_MIN_COLS 4
#endif

inline int gemm_blocks(int TR, int M) { return (TR + gemm_rows(M) - 1) / gemm_rows(M); }

// K parts for a launch of nb workgroup rows over TC tile columns: as many as
// keep all workgroups resident at once (nb * S <= the target), at most one
// per Q4NX_GEMM_MIN_COLS tile columns.
inline int gemm_parts(int nb, int TC) {
  int S = Q4NX_GEMM_WG_TARGET / nb;
  const int lim = TC / Q4NX_GEMM_MIN_COLS > 0 ? TC / Q4NX_GEMM_MIN_COLS : 1;
  if (S > lim) S = lim;
  if (S < 1) S = 1;
  return S;
}

// Workspace: a 4 KB header -- kGemmCntWords arrival counters (K is split only
// when nb * 2 <= the workgroup target, so nb stays below it), as many XCD
// claim words (one per group of 8 workgroups: ceil(NB / 8) * S <= 256 groups,
// since NB * S <= 256), as many rescue flags, then diagnostic words -- and
// then the partial tiles.  The header has the same size for every call, so one zeroed buffer of
// the largest size any call needs serves calls of any shape.
constexpr int kGemmCntWords = Q4NX_GEMM_WG_TARGET;
constexpr size_t kGemmClaimOff = (size_t)kGemmCntWords * 4;
constexpr size_t kGemmRescueOff = kGemmClaimOff + (size_t)kGemmCntWords * 4;
constexpr size_t kGemmDiagOff = kGemmRescueOff + (size_t)kGemmCntWords * 4;
constexpr size_t kGemmCntBytes = 4096;
static_assert(kGemmDiagOff + 256 <= kGemmCntBytes, "GEMM workspace header");
inline size_t gemm_ws_bytes(int nb, int TC, int M) {
  const int S = gemm_parts(nb, TC);
  if (S == 1) return 0;
  return kGemmCntBytes + (size_t)nb * S * 64 * gemm_rows(M) * 32 * 4;
}
// Workspace for a launch over weights of tile rows TR[0..n-1] at any M.
inline size_t gemm_ws_bytes_any_m(const int* TR, int n, int TC) {
  size_t best = 0;
  for (int M : {32, 64}) {
    int nb = 0;
    for (int i = 0; i < n; ++i) nb += gemm_blocks(TR[i], M);
    const size_t b = gemm_ws_bytes(nb, TC, M);
    if (b > best) best = b;
  }
  return best;
}

// local: lay the K parts of each workgroup row on one XCD (see gemm.hip).
hipError_t launch_gemm(int kind, const GemmArgs& a, bool local, hipStream_t s);
// 1 when this device deals a launch's workgroups to its 8 XCDs round-robin by
// linear id, from a starting XCD that may vary per launch.  Checked once per
// device with a 64-workgroup probe on a stream of the library's own, never on
// the caller's stream and never while the caller's stream is being captured
// (0 until the probe has run).
int xcd_round_robin(hipStream_t caller);
// The probe's answer if it has already run on this device, else 0; launches nothing.
int xcd_round_robin_known();

}  // namespace q4nx
