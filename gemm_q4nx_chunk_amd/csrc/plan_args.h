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
