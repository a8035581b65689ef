// Top-k of a GEMV's outputs in the GEMV's own launch (the greedy / top-k pick
// after the lm_head: NPU engine page, "Q4NX chunks", the Q8 tied embedding and
// lm_head; onw technical notes, host work of one step, which samples from the
// head's logits).
//
// A candidate is one 64-bit key, order-preserving value bits << 32 | ~row, so
// the larger key is the larger value and, among equal values, the lower row;
// zeros of either sign are equal and a NaN ranks below every number.  Keys are
// unique (the row is in them), so "the largest key below the last one taken"
// walks the keys in decreasing order without marking anything.
//
// For k = 1 one 64-bit atomic maximum per activation row is enough (below).
// Otherwise three levels, each a single wave per activation row:
//   0. every workgroup: the top k of its own rows, written to the workspace;
//   1. the last workgroup of each group of 64 to finish: the top k of the
//      group's 64 lists (lane j holds member j's list, already in decreasing
//      order, and advances its head when it wins a round);
//   2. the last group to finish: the same over the groups' lists, then the
//      ids and values.
// Lists move through device-scope stores, each publisher waits for its stores
// before it counts itself in, and mergers read with device-scope loads, so
// the protocol works whatever XCD each workgroup runs on.  The last arriver of
// each counter puts it back to zero for the next call.
#pragma once

#include "q4nx_dev.h"

namespace q4nx {

constexpr int kTopkMax = 16;        // k of one call
constexpr int kTopkGroup = 64;      // workgroups merged by one group merger
constexpr int kTopkMaxWg = kTopkGroup * 64;   // workgroups of one launch
constexpr int kTopkRows = 128;      // rows per workgroup (at most) in a level-0 pick

__device__ __forceinline__ uint64_t topk_key(float v, uint32_t row) {
  uint32_t b = __float_as_uint(v);
  if (v == 0.f) b = 0;                                                     // -0 == +0
  const uint32_t ord = v != v ? 0u : ((b & 0x80000000u) ? ~b : (b | 0x80000000u));   // NaN lowest
  return ((uint64_t)ord << 32) | (uint32_t)~row;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

// Device-scope 8-byte store and load (they reach past this XCD's L2).
__device__ __forceinline__ void st_key(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_key(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Level 0 for activation row m, run by one whole wave: the top k of the
// workgroup's nr values vals[0..nr) (global rows row0 + i), written to out[0..k).
__device__ __forceinline__ void topk_local(const float* vals, int nr, uint32_t row0, int k, int lane,
                                           uint64_t* out) {
  uint64_t a = 0, b = 0;   // key 0: no candidate
  if (lane < nr) a = topk_key(vals[lane], row0 + lane);
  if (lane + 64 < nr) b = topk_key(vals[lane + 64], row0 + lane + 64);
  uint64_t last = ~0ull;
  for (int j = 0; j < k; ++j) {
    const uint64_t ca = a < last ? a : 0, cb = b < last ? b : 0;
    const uint64_t w = wave_max_u64(ca > cb ? ca : cb);
    if (lane == 0) st_key(out + j, w);
    last = w;
  }
}

// Levels 1 and 2 for activation row m, one whole wave: merge n lists of k keys
// (list j at in + j * stride, decreasing) into out[0..k).  Returns the merged
// keys in lane j < k of `mine` (for the caller that writes the ids).
__device__ __forceinline__ uint64_t topk_merge(const uint64_t* in, int stride, int n, int k, int lane,
                                               uint64_t* out) {
  uint64_t list[kTopkMax];
#pragma unroll
  for (int j = 0; j < kTopkMax; ++j) list[j] = (lane < n && j < k) ? ld_key(in + (size_t)lane * stride + j) : 0;
  int head = 0;
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t h = 0;
#pragma unroll
    for (int t = 0; t < kTopkMax; ++t) h = t == head ? list[t] : h;
    const uint64_t w = wave_max_u64(h);
    if (h == w && w != 0) ++head;   // keys are unique: only the owner advances
    if (out && lane == 0) st_key(out + j, w);
    if (lane == j) mine = w;
  }
  return mine;
}

__device__ __forceinline__ void topk_write(const TopkArgs& tk, int m, int lane, uint64_t key) {
  if (lane >= tk.k) return;
  const uint32_t ord = (uint32_t)(key >> 32);
  int32_t id = -1;
  float v = __builtin_nanf("");
  if (ord != 0) {
    id = (int32_t)~(uint32_t)key;
    v = __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
  }
  tk.ids[(size_t)m * tk.k + lane] = id;
  if (tk.vals) tk.vals[(size_t)m * tk.k + lane] = v;
}

// k = 1 (greedy): every workgroup folds its best key of activation row m into
// one device-scope 64-bit atomic maximum (returning, so it has landed before
// the workgroup counts itself in); the last workgroup reads the maxima, writes
// the picks and clears the words.  best[m] sits in the workspace where the
// level-0 lists would.
template <int M, int WAVES>
__device__ __forceinline__ void topk1_epilogue(const TopkArgs& tk, const float (*tv)[kTopkRows], int nr,
                                               uint32_t row0, uint32_t* s_flag) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t* best = tk.cand;
  if (wave < M) {
    uint64_t a = 0, b = 0;
    if (lane < nr) a = topk_key(tv[wave][lane], row0 + lane);
    if (lane + 64 < nr) b = topk_key(tv[wave][lane + 64], row0 + lane + 64);
    const uint64_t w = wave_max_u64(a > b ? a : b);
    if (lane == 0) {
      const uint64_t old = __hip_atomic_fetch_max(best + wave, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("" ::"v"(old));   // the returned value is waited for: the maximum has landed
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(tk.cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = old == (uint32_t)tk.n_wg - 1;
    if (*s_flag) __hip_atomic_store(tk.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!*s_flag) return;
  if (threadIdx.x < M) {
    const uint64_t w = __hip_atomic_exchange(best + threadIdx.x, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    TopkArgs t1 = tk;
    topk_write(t1, threadIdx.x, 0, w);
  }
}

// The whole protocol after a workgroup's values are in LDS: tv[m][i] for
// i < nr, global rows row0 + i.  Call with every thread of the workgroup,
// after a barrier that makes tv visible.  WAVES >= M.
template <int M, int WAVES>
__device__ __forceinline__ void topk_epilogue(const TopkArgs& tk, const float (*tv)[kTopkRows], int nr,
                                              uint32_t row0, uint32_t* s_flag) {
  static_assert(WAVES >= M, "one wave per activation row");
  if (tk.k == 1) {
    topk1_epilogue<M, WAVES>(tk, tv, nr, row0, s_flag);
    return;
  }
  const int wg = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = tk.k, grp = wg / kTopkGroup;
  uint64_t* lvl0 = tk.cand;
  uint64_t* lvl1 = tk.cand + (size_t)tk.n_wg * M * k;
  if (wave < M) topk_local(tv[wave], nr, row0, k, lane, lvl0 + ((size_t)wg * M + wave) * k);
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int members = min(kTopkGroup, tk.n_wg - grp * kTopkGroup);
    const uint32_t old = __hip_atomic_fetch_add(tk.cnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = old == (uint32_t)members - 1;
    if (*s_flag) __hip_atomic_store(tk.cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!*s_flag) return;
  // level 1: this group's members
  const int members = min(kTopkGroup, tk.n_wg - grp * kTopkGroup);
  if (wave < M)
    topk_merge(lvl0 + ((size_t)grp * kTopkGroup * M + wave) * k, M * k, members, k, lane,
               lvl1 + ((size_t)grp * M + wave) * k);
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(tk.cnt + tk.n_grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = old == (uint32_t)tk.n_grp - 1;
    if (*s_flag) __hip_atomic_store(tk.cnt + tk.n_grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!*s_flag) return;
  // level 2: every group
  if (wave < M) {
    const uint64_t mine = topk_merge(lvl1 + (size_t)wave * k, M * k, tk.n_grp, k, lane, nullptr);
    topk_write(tk, wave, lane, mine);
  }
}

}  // namespace q4nx
