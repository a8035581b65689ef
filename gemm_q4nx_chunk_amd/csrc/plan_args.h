// Device-side tables of a GEMV plan (see plan.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4nx_dev.h"

namespace q4nx {

// Chunks per wave in one plan unit: 4 waves x CPW chunks per unit.
template <int KIND> struct PlanCpw { static constexpr int value = 4; };
template <> struct PlanCpw<KIND_Q8_A> { static constexpr int value = 2; };
template <> struct PlanCpw<KIND_Q8_B> { static constexpr int value = 2; };

inline int plan_cpw(int kind) { return (kind == KIND_Q8_A || kind == KIND_Q8_B) ? 2 : 4; }

struct PlanJob {
  const uint8_t* w;
  const uint16_t* x;
  float* y;
  int32_t TR, TC, ldx, ldy;
  int32_t S;       // units per tile row (> 1: parts added by the last to arrive)
  int32_t unit0;   // first unit of the job
  int32_t phase;   // phase within its launch
  int32_t slot0;   // first row slot of a split job (counters, partials)
};

struct PlanArgs {
  const PlanJob* jobs;
  const int32_t* unit_job;   // [n_units] job of each unit
  const uint32_t* need;      // [n_phases] tile rows each phase must finish
  uint32_t* done;            // [n_phases] tile rows finished so far
  uint32_t* row_cnt;         // [n_slots] parts arrived per split tile row
  float* partial;            // [n_slots][smax][32][M]
  uint32_t* ctl;             // [0] workgroups finished, [1] error flags
  int32_t n_units, n_phases, spin_limit, smax;
};

hipError_t plan_resident_blocks(int kind, int M, int* blocks);
hipError_t launch_plan(int kind, int M, const PlanArgs& a, int grid, hipStream_t s);

}  // namespace q4nx

namespace q4nx {

// ---------------------------------------------------------------------------
// Step kernel (step.hip): the same plans for q4 kinds, with a static schedule.
// ---------------------------------------------------------------------------
struct StepJob {
  const uint8_t* w;
  const uint16_t* x;
  float* y;
  int32_t TR, TC, ldx, ldy;
};

// One workgroup's piece of work: tile row tr of a job over chunk columns
// [c0, c1).  A tile row longer than one piece is cut into consecutive pieces
// of the same workgroup, which carry its sums in registers from the first
// (kStepFirst) to the last (kStepLast).
struct StepUnit {
  int32_t job;
  int32_t tr;
  int16_t c0, c1;
  int16_t phase;
  int16_t flags;
};
constexpr int kStepFirst = 1;
constexpr int kStepLast = 2;

// Chunk columns of one piece at most (longer tile rows are cut).
constexpr int kStepPieceCols = 64;
// Each compute wave's LDS ring: ns slots of one chunk each (q4_1 fills a
// slot; Q4_K uses 4736 bytes of it).
constexpr int kStepSlot = 5120;
constexpr int kStepMaxSlots = 8;

struct StepArgs {
  const StepJob* jobs;
  const StepUnit* units;      // workgroup b's pieces are [wg_first[b], wg_first[b + 1])
  const int32_t* wg_first;
  uint32_t* sync;             // word 16 x: workgroups on XCD x; word 128 + 16 (8 p + x):
                              // workgroups of XCD x done with phase p (zero between runs)
  uint32_t* ctl;              // [0] workgroups finished, [1] error flags
  int32_t n_phases, spin_limit;
  int32_t ring_off, ns;       // LDS byte offset of the rings (after the records), slots per ring
};

constexpr int kStepComputeWaves = 8;                    // two per SIMD: one hides the other's latencies
constexpr int kStepThreads = 64 * (kStepComputeWaves + 1);   // and one sync wave
// Dynamic LDS of the step kernel for jobs of at most max_tc tile columns:
// the prepared activations (rec bytes), then one ring of ns slots per compute
// wave; at least
// enough to keep one workgroup per CU.  ns = 0: the activations do not fit.
struct StepLds {
  size_t rec, total;
  int ns;
};
StepLds step_lds(int M, int max_tc);
inline size_t step_sync_words(int n_phases) { return 128 + (size_t)16 * 8 * n_phases; }
hipError_t launch_step(int kind, int M, const StepArgs& a, int grid, size_t lds, hipStream_t s);

}  // namespace q4nx
