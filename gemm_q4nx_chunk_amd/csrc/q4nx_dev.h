// Internal device/host definitions shared by the HIP sources of libq4nx.so.
//
// Chunk facts used by the kernels (1bit engine docs, page "NPU engine",
// section "Q4NX chunks"): 32 x 256 tiles, one chunk per tile, row-major over
// the grid; q4_1 5120 B (w = code*scale + zero), Q4_K 4736 B
// (w = S*scale*code + M*min), Q8 8704 B (w = d*code) with the two printed code
// layouts.  In-chunk positions not printed there follow the library's layout
// (see include/q4nx.h): 4-bit codes at byte r*128 + k/2 (even k low nibble),
// q4_1 (scale, zero) at 4096 + 4*(8r+g), Q4_K (sc, mn) at 4096 + 2*(8r+g) and
// (S, M) at 4608 + 4r, Q8 d at 8192 + 2*(8r+g).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4nx {

enum Kind : int { KIND_Q4_1 = 0, KIND_Q4_K = 1, KIND_Q8_A = 2, KIND_Q8_B = 3 };

template <int KIND>
struct ChunkBytes;
template <> struct ChunkBytes<KIND_Q4_1> { static constexpr int value = 5120; };
template <> struct ChunkBytes<KIND_Q4_K> { static constexpr int value = 4736; };
template <> struct ChunkBytes<KIND_Q8_A> { static constexpr int value = 8704; };
template <> struct ChunkBytes<KIND_Q8_B> { static constexpr int value = 8704; };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One GEMV of a batched launch.  Workgroup wg of the launch belongs to the last
// job whose wg_begin <= wg.  ks = waves that split one tile row's chunks (a
// power of two up to the launch's waves per workgroup W); a workgroup covers
// W/ks tile rows.
struct GemvJob {
  const uint8_t* w;
  const uint16_t* x;
  float* y;
  int32_t TR, TC;
  int32_t ldx, ldy;   // row strides of x and y, in elements
  int32_t wg_begin;
  int32_t ks;
};

constexpr int kMaxBatch = 64;

// Top-k of the outputs in the same launch (topk.h); k = 0 for a plain GEMV.
struct TopkArgs {
  int32_t k;           // 0: no top-k (plain GEMV)
  int32_t n_wg, n_grp;
  uint64_t* cand;      // [n_wg + n_grp][M][k] keys: level 0, then level 1
  uint32_t* cnt;       // [n_grp + 1] arrival counters (zero between calls)
  int32_t* ids;        // [M][k] rows, best first; -1 past the last number
  float* vals;         // [M][k] or null
};

struct GemvBatch {
  GemvJob job[kMaxBatch];
  // Or, when tab is set, the jobs come from device memory (any number of
  // them): workgroup b runs job tab[tab_wg[b]], and job[] / n_jobs are unused.
  const GemvJob* tab;
  const int32_t* tab_wg;
  int32_t n_jobs;
  // chunk slices per unit of work: 4 (a unit is a tile row), or 2 (a unit is
  // 16 rows of a tile; q4 kinds with prepared activations only).  The jobs'
  // wg_begin and ks then count units.
  int32_t sl;
  TopkArgs tk;   // one job, 4-wave workgroups, M <= 4; job[0].y may be null
};

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ u32x4 load_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float dot2bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum over the 8 lanes that differ in bits 0..2 of the lane id; fixed order,
// so every lane of the group ends with the same bits.
__device__ __forceinline__ float sum_lanes_xor7(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  return v;
}

// Cache-policy operand of the buffer-load builtins: sc1 = device-scope coherent.
constexpr int kCpolSc1 = 16;

// Buffer resource over n bytes at p (raw, untyped; offsets past n read as 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

// Device-scope (sc1) 4-byte store and load: they reach past this XCD's L2,
// so another workgroup of the same launch reads what was written.
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every store this wave issued is complete (visible at device scope
// for sc1 stores), and keep the compiler from moving memory operations across.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Tables that never change during a launch, read through the constant address
// space so the loads are scalar and never wait behind vector memory traffic.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int i) {
  static_assert(sizeof(T) % 4 == 0, "whole words");
  typedef const __attribute__((address_space(4))) uint32_t* cword;
  const cword q = (cword)(p + i);
  uint32_t w[sizeof(T) / 4];
#pragma unroll
  for (unsigned j = 0; j < sizeof(T) / 4; ++j) w[j] = q[j];
  T v;
  __builtin_memcpy(&v, w, sizeof(T));
  return v;
}

// Pick the job of workgroup `wg`: the last one whose wg_begin <= wg.
__device__ __forceinline__ int find_job(const GemvBatch& b, int wg) {
  int j = 0;
  for (int t = 1; t < b.n_jobs; ++t)
    if (wg >= b.job[t].wg_begin) j = t;
  return j;
}

// The job of this workgroup, from the kernel arguments or the device table.
__device__ __forceinline__ GemvJob gemv_job(const GemvBatch& b) {
  if (b.tab) return ld_const(b.tab, ld_const(b.tab_wg, (int)blockIdx.x));
  return b.job[find_job(b, blockIdx.x)];
}

// Host-side launchers (gemv.hip, gemm.hip, decode.hip, moe.hip).
// Dynamic LDS bytes of the prepared-activation GEMV for a launch whose jobs
// have at most max_tc tile columns, or 0 when that kernel does not apply.
// Activation rows from which q4 launches with prepared records take the
// matrix-core products (k_gemv_q4m) instead of the dot chain (k_gemv_q4x).
#ifndef Q4NX_GEMV_MFMA_MIN_M
#define Q4NX_GEMV_MFMA_MIN_M 2
#endif
constexpr int kGemvMfmaMinM = Q4NX_GEMV_MFMA_MIN_M;
int gemv_xl_bytes(int kind, int M, int waves, int max_tc);
hipError_t launch_gemv(int kind, int M, int waves, const GemvBatch& b, int n_wg, int xl_bytes,
                       hipStream_t s);
// The GEMV of b.job[0] with the top-k of its outputs (b.tk), 4-wave workgroups, M <= 4.
hipError_t launch_gemv_topk(int kind, int M, const GemvBatch& b, int n_wg, int xl_bytes, hipStream_t s);
hipError_t launch_unpack(int kind, const uint8_t* w, int TR, int TC, uint8_t* codes,
                         uint16_t* meta0, uint16_t* meta1, uint16_t* row_meta, hipStream_t s);
hipError_t launch_decode(int kind, const uint8_t* w, int TR, int TC, float* out, hipStream_t s);
hipError_t launch_repack_q4k(const uint8_t* w, int tiles, uint8_t* out, hipStream_t s);
// A described in-chunk layout (the fields of q4nx_chunk_layout), checked on the host.
struct ChunkLayout {
  int32_t chunk_bytes;
  int32_t code_off, code_row, code_group, code_step, code_pairing, code_high_first;
  int32_t f0_off, f0_row, f0_group;
  int32_t f1_off, f1_row, f1_group;
  int32_t s_off, s_row, m_off, m_row;
};
hipError_t launch_relayout(const ChunkLayout& L, const uint8_t* src, int tiles, uint8_t* out, hipStream_t s);
hipError_t launch_gguf_q41(int gtype, const uint8_t* src, int TR, int TC, uint8_t* out, hipStream_t s);
hipError_t launch_q8_rows(int kind, const uint8_t* w, int rows, int TC, const int32_t* ids, int T,
                          float* out, hipStream_t s);
// Split argmax: slices of this many values per workgroup, one 8-byte key each
// in the workspace.
constexpr int kArgmaxSlice = 4096;
inline int argmax_parts(int n) { return (n + kArgmaxSlice - 1) / kArgmaxSlice; }
hipError_t launch_argmax(const float* y, int n, int ldy, int M, int32_t* idx, float* val, void* ws,
                         hipStream_t s);
hipError_t launch_moe_router(const uint16_t* R, const uint16_t* X, int T, int D, int E, int k,
                             int renorm, int32_t* ids, float* p, float* logits, hipStream_t s);

}  // namespace q4nx
