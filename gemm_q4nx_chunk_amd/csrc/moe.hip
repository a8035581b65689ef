// Routed-expert MoE layer on Q4NX weights (gfx950).
//
// Shape and order of the layer (Strata article, section 2 "target model"):
// 512 routed experts per layer, the router's top 10 per token, a shared expert
// used by every token, then the sum.  The selected experts' chunks are read in
// place from one arena per projection, by expert id (onw technical notes,
// "MoE on the NPU": bind only the selected experts, never copy the table), and
// the (token, slot) pairs are grouped by expert so that each selected expert
// is read once for all the tokens that chose it (onw technical notes,
// "computing MoE prompts together").
//
// Four kernels on one stream:
//   route   one workgroup: stable sort of the pairs by (expert, token, slot);
//           per-expert segments; batch counts.  Ids outside [0, n_experts) go
//           to the end, are never dereferenced, and set bit 0 of the error word.
//   gateup  per (token batch, tile row): gate and up rows of the expert for up
//           to TB tokens, h = silu(g) * u in fp32.
//   down    per (token batch, group of tile rows): d = Down h, fp32; h is
//           read as fp16 records with a power-of-two scale per 32 values
//           (each h to 2^-12 of its size).
//   combine y[t] = sum_j p[t][j] d[t][j] in slot order, then + the shared d.
// No floating-point atomics anywhere; every sum has a fixed order.
#include <type_traits>

#include "gemv_core.h"
#include "mfma_q4.h"
#include "moe_args.h"

namespace q4nx {

// ---------------------------------------------------------------------------
// route
// ---------------------------------------------------------------------------
// Blocks of at most 64 tokens over at most 1024 experts whose ids are all in
// range and whose tokens name distinct experts need no sort: bit t of mask[e]
// says token t picked expert e.  A token's slots name distinct experts, so an
// expert's pairs in token order are its pairs in pair-index order, and a
// pair's place in its segment is the number of earlier tokens in the mask.
// Counts, batch counts and segment flags are one prefix sum over the experts
// (one per thread); each routed batch's record is then written by its own
// thread.  The tables are the ones the sort below produces.  Returns false,
// having written nothing, when the block does not qualify.
constexpr int kRouteMaskTokens = 64, kRouteMaskExperts = 1024;

// A segment of cnt pairs runs on the matrix cores (and has no batches).
__device__ __forceinline__ bool moe_hot(const MoeArgs& a, int cnt) {
  return a.hot_min > 0 && cnt >= a.hot_min;
}
__device__ __forceinline__ bool moe_shared_hot(const MoeArgs& a) {
  return a.Ds > 0 && a.hot_min > 0 && a.T >= a.hot_min;
}

__device__ __forceinline__ uint64_t block_incl_scan64(uint64_t v, uint64_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  if (w == 0) {
    uint64_t t = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint64_t o = __shfl_up(t, off);
      if (lane >= off) t += o;
    }
    if (lane < 16) wsum[lane] = t;
  }
  __syncthreads();
  return w > 0 ? v + wsum[w - 1] : v;
}

__device__ __forceinline__ bool moe_route_masks(const MoeArgs& a, uint32_t* lds16k, int32_t* sorted_lds,
                                                uint64_t* wsum, int32_t* flags) {
  const int T = a.T, k = a.k, P = T * k, E = a.n_experts, tid = threadIdx.x;
  if (T > kRouteMaskTokens || E > kRouteMaskExperts) return false;
  uint64_t* mask = reinterpret_cast<uint64_t*>(lds16k);           // [1024]
  int32_t* s_start = reinterpret_cast<int32_t*>(mask + 1024);     // [1024]
  int32_t* s_bstart = s_start + 1024;                             // [1024]
  mask[tid] = 0;
  if (tid == 0) { flags[0] = 0; flags[1] = 0; }
  __syncthreads();
  int e_mine = -1;
  if (tid < P) {   // P <= 64 * 16 = 1024
    const int e = a.ids[tid];
    if (e < 0 || e >= E) atomicOr(&flags[0], 1);
    else {
      atomicOr(reinterpret_cast<unsigned long long*>(&mask[e]), 1ull << (tid / k));
      e_mine = e;
    }
  }
  __syncthreads();
  const uint64_t m = tid < E ? mask[tid] : 0;
  const int cnt = __popcll(m);
  if (cnt) atomicAdd(&flags[1], cnt);
  __syncthreads();
  if (flags[0] || flags[1] != P) return false;   // an id out of range, or a token naming an expert twice
  const int nb = moe_hot(a, cnt) ? 0 : (cnt + a.tb - 1) / a.tb;
  const uint64_t own = (uint64_t)cnt | ((uint64_t)nb << 16) | ((uint64_t)(cnt > 0) << 32);
  const uint64_t inc = block_incl_scan64(own, wsum);
  const uint64_t ex = inc - own;
  const int start = (int)(ex & 0xFFFFu), bstart = (int)((ex >> 16) & 0xFFFFu), u = (int)(ex >> 32);
  s_start[tid] = start;
  s_bstart[tid] = bstart;
  if (cnt) {
    a.seg[3 * u + 0] = tid;
    a.seg[3 * u + 1] = start;
    a.seg[3 * u + 2] = cnt;
    a.batch0[u] = bstart;
  }
  if (tid == 1023) {
    const int nseg = (int)(inc >> 32), nbatch = (int)((inc >> 16) & 0xFFFFu);
    a.hdr[0] = 0u;
    a.hdr[1] = (uint32_t)nseg;
    a.hdr[2] = (uint32_t)nbatch;
    a.batch0[nseg] = nbatch;
    flags[2] = nbatch;
  }
  __syncthreads();
  if (e_mine >= 0) {
    const int t = tid / k;
    const int pos = s_start[e_mine] + __popcll(mask[e_mine] & ((1ull << t) - 1));
    sorted_lds[pos] = tid;
    a.sorted[pos] = tid;
  }
  __syncthreads();
  if (tid < flags[2]) {   // batch tid: the last expert whose first batch is at or before it
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_bstart[mid] <= tid) lo = mid; else hi = mid - 1;
    }
    const int e = lo, bi = tid - s_bstart[e], c = __popcll(mask[e]);
    const int pos0 = s_start[e] + bi * a.tb, ntok = min(a.tb, c - bi * a.tb);
    int32_t* r = a.btab + (size_t)tid * kMoeBatchInts;
    r[0] = e;
    r[1] = pos0;
    r[2] = ntok;
    r[3] = 0;
    for (int mm = 0; mm < 4; ++mm) {
      const int pair = sorted_lds[pos0 + (mm < ntok ? mm : 0)];
      r[4 + mm] = pair / k;
      r[8 + mm] = pair;
    }
  }
  return true;
}

// Matrix-core units: the segments of at least hot_min pairs in segment order,
// then the shared expert when T >= hot_min; each with the first of its work
// items in both item spaces (items of 64 token rows times groups of 2 gate/up
// or 8 down tile rows).  Wave 0 walks the segment table the route kernel has
// just written, 64 segments at a time.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ void moe_route_hot(const MoeArgs& a) {
  if (a.hot_min <= 0) return;
  __syncthreads();   // the segment table and header are written
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int nseg = (int)a.hdr[1];
  const int g_gu = a.De / 64, g_dn = a.D / 256;   // row groups per token block
  int nh = 0, igu = 0, idn = 0;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    const int sg = s0 + lane;
    int e = 0, start = 0, cnt = 0;
    if (sg < nseg) {
      e = a.seg[3 * sg];
      start = a.seg[3 * sg + 1];
      cnt = a.seg[3 * sg + 2];
    }
    const bool hot = sg < nseg && moe_hot(a, cnt);
    const int nblk = hot ? (cnt + kMoeHotTokens - 1) / kMoeHotTokens : 0;
    const int ih = wave_incl_scan(hot ? 1 : 0);
    const int ig = wave_incl_scan(nblk * g_gu);
    const int id = wave_incl_scan(nblk * g_dn);
    if (hot) {
      int32_t* r = a.hot + (size_t)(nh + ih - 1) * kMoeHotInts;
      r[0] = e;
      r[1] = start;
      r[2] = cnt;
      r[3] = igu + ig - nblk * g_gu;
      r[4] = idn + id - nblk * g_dn;
    }
    nh += __shfl(ih, 63);
    igu += __shfl(ig, 63);
    idn += __shfl(id, 63);
  }
  if (moe_shared_hot(a)) {
    const int nblk = (a.T + kMoeHotTokens - 1) / kMoeHotTokens;
    if (lane == 0) {
      int32_t* r = a.hot + (size_t)nh * kMoeHotInts;
      r[0] = -1;
      r[1] = 0;
      r[2] = a.T;
      r[3] = igu;
      r[4] = idn;
    }
    nh += 1;
    igu += nblk * (a.Ds / 64);
    idn += nblk * g_dn;
  }
  if (lane == 0) {
    a.hdr[3] = (uint32_t)nh;
    a.hdr[4] = (uint32_t)igu;
    a.hdr[5] = (uint32_t)idn;
  }
}

__global__ __launch_bounds__(1024) void k_moe_route(MoeArgs a) {
  __shared__ uint32_t key[kMoeMaxPairs];
  __shared__ int32_t scan[1024];
  __shared__ int32_t nbad;
  __shared__ uint64_t wsum[16];
  __shared__ int32_t flags[4];
  static_assert(kMoeMaxPairs * 4 >= 1024 * 16, "the masks and prefix tables fit the key array");
  if (moe_route_masks(a, key, scan, wsum, flags)) {
    moe_route_hot(a);
    return;
  }
  __syncthreads();   // the masks' LDS is the sort's
  const int P = a.T * a.k;
  int NP = 1;
  while (NP < P) NP <<= 1;
  const int tid = threadIdx.x;
  if (tid == 0) nbad = 0;
  __syncthreads();
  int bad_local = 0;
  for (int i = tid; i < NP; i += 1024) {
    uint32_t kv = 0xFFFFFFFFu;
    if (i < P) {
      const int e = a.ids[i];
      const bool ok = e >= 0 && e < a.n_experts;
      bad_local |= !ok;
      kv = ((uint32_t)(ok ? e : a.n_experts) << 12) | (uint32_t)i;
    }
    key[i] = kv;
  }
  if (bad_local) atomicOr(&nbad, 1);
  // bitonic sort, ascending
  for (int size = 2; size <= NP; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = tid; i < NP; i += 1024) {
        const int jx = i ^ stride;
        if (jx > i) {
          const uint32_t ki = key[i], kj = key[jx];
          const bool up = (i & size) == 0;
          if ((ki > kj) == up) { key[i] = kj; key[jx] = ki; }
        }
      }
    }
  }
  __syncthreads();
  // segment starts among valid pairs, scanned in chunks of 1024
  int base_seg = 0, base_batch = 0;
  for (int c0 = 0; c0 < P; c0 += 1024) {
    const int s = c0 + tid;
    int start = 0, cnt = 0, e = -1;
    if (s < P) {
      e = (int)(key[s] >> 12);
      if (e < a.n_experts && (s == 0 || (int)(key[s - 1] >> 12) != e)) {
        start = 1;
        int end = s + 1;
        while (end < P && (int)(key[end] >> 12) == e) ++end;
        cnt = end - s;
      }
      a.sorted[s] = (int32_t)(key[s] & 0xFFFu);
    }
    // inclusive scans of start flags and of batch counts, packed in one int
    const int nb = start && !moe_hot(a, cnt) ? (cnt + a.tb - 1) / a.tb : 0;
    scan[tid] = (start << 20) | nb;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (start) {
      const int u = base_seg + (scan[tid] >> 20) - 1;
      const int bstart = base_batch + (scan[tid] & 0xFFFFF) - nb;
      a.seg[3 * u + 0] = e;
      a.seg[3 * u + 1] = s;
      a.seg[3 * u + 2] = cnt;
      a.batch0[u] = bstart;
      // the segment's batch records, so a work item finds its batch in one load
      for (int bi = 0; bi < nb; ++bi) {
        int32_t* r = a.btab + (size_t)(bstart + bi) * kMoeBatchInts;
        const int pos0 = s + bi * a.tb, ntok = min(a.tb, cnt - bi * a.tb);
        r[0] = e;
        r[1] = pos0;
        r[2] = ntok;
        r[3] = 0;
        for (int m = 0; m < 4; ++m) {
          const int pair = (int)(key[pos0 + (m < ntok ? m : 0)] & 0xFFFu);
          r[4 + m] = pair / a.k;
          r[8 + m] = pair;
        }
      }
    }
    base_seg += scan[1023] >> 20;
    base_batch += scan[1023] & 0xFFFFF;
    __syncthreads();
  }
  if (tid == 0) {
    a.hdr[0] = nbad ? 1u : 0u;        // error word
    a.hdr[1] = (uint32_t)base_seg;    // segments
    a.hdr[2] = (uint32_t)base_batch;  // routed token batches
    a.batch0[base_seg] = base_batch;
  }
  moe_route_hot(a);
}

// Work item of a (batch, tile-row group) launch: which expert, which tokens.
struct MoeItem {
  const uint8_t* w0;    // gate (gateup) or down (down) chunks of the expert
  const uint8_t* w1;    // up chunks (gateup only)
  int tr;               // first tile row
  int ntok;             // tokens in this batch (1..TB)
  int pos0;             // first sorted position (routed) or P + first token (shared)
  bool shared;
  const int32_t* rec;   // routed: the batch's record (tokens at [4], pairs at [8])
};

// Token of row m < TB of an item (past ntok: the first again), and its pair
// index (routed) or P + token (shared).
__device__ __forceinline__ int moe_item_tok(const MoeArgs& a, const MoeItem& it, int m) {
  if (!it.shared) return it.rec[4 + m];
  return it.pos0 - a.T * a.k + (m < it.ntok ? m : 0);
}
__device__ __forceinline__ int moe_item_pair(const MoeArgs& a, const MoeItem& it, int m) {
  if (!it.shared) return it.rec[8 + m];
  return it.pos0 + (m < it.ntok ? m : 0);
}

// Items are numbered routed first (every routed batch times its tile-row
// groups), then shared.  rpw = tile rows per workgroup for each kind of item.
template <int TB>
__device__ __forceinline__ bool moe_item(const MoeArgs& a, int nbr, int item, int rows_r, int rows_s,
                                         int rpw_r, int rpw_s, bool down, MoeItem& it) {
  static_assert(TB <= 4, "batch records hold 4 tokens");
  const int P = a.T * a.k;
  const int gr = rows_r / rpw_r, gs = rows_s / rpw_s;
  if (item < nbr * gr) {
    const int b = item / gr;
    const int32_t* r = a.btab + (size_t)b * kMoeBatchInts;
    const int e = r[0];
    it.tr = (item - b * gr) * rpw_r;
    it.pos0 = r[1];
    it.ntok = r[2];
    it.shared = false;
    it.rec = r;
    if (down) {
      it.w0 = a.down + (size_t)e * a.down_stride;
      it.w1 = nullptr;
    } else {
      it.w0 = a.gate + (size_t)e * a.gate_stride;
      it.w1 = a.up + (size_t)e * a.up_stride;
    }
    return true;
  }
  item -= nbr * gr;
  const int nbs = a.Ds && !moe_shared_hot(a) ? (a.T + TB - 1) / TB : 0;
  if (item < nbs * gs) {
    const int b = item / gs;
    it.tr = (item - b * gs) * rpw_s;
    it.pos0 = P + b * TB;
    it.ntok = min(TB, a.T - b * TB);
    it.shared = true;
    it.rec = nullptr;
    it.w0 = down ? a.sdown : a.sgate;
    it.w1 = down ? nullptr : a.sup;
    return true;
  }
  return false;
}

// ---------------------------------------------------------------------------
// weight-stationary gate/up and down
// ---------------------------------------------------------------------------
// One work item is one tile row of one selected expert (or of the shared
// expert) for ALL the tokens routed to it: each wave loads its chunks of the
// row once, keeps them in registers, and runs every batch of TB tokens against
// them, so an expert's weights cross HBM once per call however popular it is.
// A batch's activations are prepared once per workgroup into LDS (the dot-chain
// pairs and group sums of k_gemv_q4x), so the loop waits on nothing but LDS.
// The arithmetic per token is the one of the GEMV (same chunk split, chunk
// order and reduction order), so a token's bits do not depend on its batch.
//
// With at most kMoeSmallPairs (token, slot) pairs every workgroup sorts them
// itself (one wave, rank by comparison) and no route kernel runs.

constexpr int kMoeSmallPairs = 64;
#ifndef Q4NX_MOE_SPLIT_SINGLE
#define Q4NX_MOE_SPLIT_SINGLE 1
#endif
// Chunks a wave keeps in registers: gate/up waves hold half a d_model row
// (4 chunks at d_model 2048), down waves one or two chunks.
constexpr int kMoeCpwGateUp = 4;
constexpr int kMoeCpwDown = 2;
// Chunks a wave of the prompt-block gate/up kernel holds at once (fewer
// registers, so more of its workgroups fit on a CU).
#ifndef Q4NX_MOE_CPW_BATCH
#define Q4NX_MOE_CPW_BATCH 2
#endif
constexpr int kMoeCpwBatch = Q4NX_MOE_CPW_BATCH;

struct MoeSmallRoute {
  int32_t sorted[kMoeSmallPairs];   // pair index at each sorted position
  int32_t seg[kMoeSmallPairs][3];   // (expert, first position, count)
  int32_t nseg, bad;
};

// Wave 0 sorts the pairs by (expert, pair); invalid ids go last, unsegmented.
__device__ __forceinline__ void moe_route_small(const MoeArgs& a, MoeSmallRoute& rt) {
  const int lane = threadIdx.x & 63, P = a.T * a.k;
  if (threadIdx.x < 64) {
    uint32_t key = 0xFFFFFFFFu;
    int e = a.n_experts;
    bool ok = false;
    if (lane < P) {
      e = a.ids[lane];
      ok = e >= 0 && e < a.n_experts;
      key = ((uint32_t)(ok ? e : a.n_experts) << 12) | (uint32_t)lane;
    }
    int rank = 0;
    for (int j = 0; j < P; ++j) rank += (uint32_t)__builtin_amdgcn_readlane(key, j) < key ? 1 : 0;
    const uint64_t bad = __ballot(lane < P && !ok);
    if (lane < P) rt.sorted[rank] = lane;
    // From here lane s describes sorted position s (LDS is in order within a wave);
    // its pair's id comes from the lane that loaded it.
    __builtin_amdgcn_wave_barrier();
    const int pi = lane < P ? rt.sorted[lane] : 0;
    const int e_of_pi = __shfl(e, pi);
    const int es = lane < P ? e_of_pi : -1;
    const bool vs = lane < P && es >= 0 && es < a.n_experts;
    const int eprev = __shfl_up(es, 1);
    const bool start = vs && (lane == 0 || eprev != es);
    const uint64_t starts = __ballot(start);
    const uint64_t valid = __ballot(vs);
    if (start) {
      const int u = __popcll(starts & ((1ull << lane) - 1));
      const uint64_t later = starts & ~((2ull << lane) - 1);
      const int end = later ? __ffsll((long long)later) - 1 : __popcll(valid);
      rt.seg[u][0] = es;
      rt.seg[u][1] = lane;
      rt.seg[u][2] = end - lane;
    }
    if (lane == 0) {
      rt.nseg = __popcll(starts);
      rt.bad = bad ? 1 : 0;
    }
  }
  __syncthreads();
}

// Prepared activation records of TB rows (row m at base + rows[m], rows in
// LDS) over TC tile columns: record r = (m * TC + c) * 8 + g at xl[16 r], its
// (f, X) at xl[16 R + 2 r] (gemv_core.h); all threads of the workgroup take
// part.  (A thread's row comes from LDS: picking it from a register array by a
// lane-varying index would put the array in private memory, whose loads wait
// for every weight load in flight.)
template <int TB>
__device__ __forceinline__ void moe_stage(const uint16_t* base, const int64_t* rows, int TC, uint32_t* xl) {
  const int R = TB * TC * 8;
  float* sums = reinterpret_cast<float*>(xl + 16 * R);
  // four consecutive lanes per record (blockDim is a multiple of 4, so a
  // record's lanes run each iteration together); part d = q & 3 takes 8 values.
  // A thread's parts are loaded NB at a time and then built, so the staging
  // waits for one round trip per NB parts rather than one per part (one row of
  // d_model 2048 is one part per thread of 256).
  constexpr int NB = TB < 4 ? TB : 4;
  for (int q0 = threadIdx.x; q0 < 4 * R; q0 += NB * blockDim.x) {
    u32x4 v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = q0 + i * blockDim.x;
      if (q < 4 * R) {
        const int r = q >> 2, m = r / (TC * 8), rem = r - m * TC * 8;
        v[i] = load16(base + rows[m] + 32 * rem + 8 * (q & 3));
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = q0 + i * blockDim.x;
      if (q < 4 * R) {   // whole quads alike: 4 R and blockDim are multiples of 4
        const int r = q >> 2;
        uint32_t pr[4];
        float f, X;
        x_record_part(v[i], pr, f, X);
        *reinterpret_cast<u32x4*>(xl + 16 * r + 4 * (q & 3)) = u32x4{pr[0], pr[1], pr[2], pr[3]};
        if ((q & 3) == 0) {
          sums[2 * r] = f;
          sums[2 * r + 1] = X;
        }
      }
    }
  }
}

// fp16 records of TB rows of fp32 h (h_record_part), in the layout of
// moe_stage: four consecutive lanes per record.
template <int TB>
__device__ __forceinline__ void moe_stage_h(const float* base, const int64_t* rows, int TC, uint32_t* xl) {
  const int R = TB * TC * 8;
  float* sums = reinterpret_cast<float*>(xl + 16 * R);
  for (int q = threadIdx.x; q < 4 * R; q += blockDim.x) {
    const int r = q >> 2, m = r / (TC * 8), rem = r - m * TC * 8;
    const float* p = base + rows[m] + 32 * rem + 8 * (q & 3);
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    uint32_t pr[4];
    float f, X;
    h_record_part(a, b, pr, f, X);
    *reinterpret_cast<u32x4*>(xl + 16 * r + 4 * (q & 3)) = u32x4{pr[0], pr[1], pr[2], pr[3]};
    if ((q & 3) == 0) {
      sums[2 * r] = f;
      sums[2 * r + 1] = X;
    }
  }
}

// acc += one held chunk (tile column c) against the staged rows.
template <int KIND, int TB>
__device__ __forceinline__ void moe_chunk(const Q4Chunk<KIND>& ch, int c, int TC, const uint32_t* xl,
                                          const Q4Consts& k, float (&acc)[4][TB]) {
  const int R = TB * TC * 8, g = threadIdx.x & 7;
  const float* sums = reinterpret_cast<const float*>(xl + 16 * R);
  XRec<TB> xp;
#pragma unroll
  for (int m = 0; m < TB; ++m) {
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
  q4_compute<KIND, TB>(ch, xp, k, acc);
}

// acc += the held chunks [0, nc) (tile columns c0 + j) against the staged rows.
template <int KIND, int TB, int CPW>
__device__ __forceinline__ void moe_chunks(const Q4Chunk<KIND> (&ch)[CPW], int nc, int c0, int TC,
                                           const uint32_t* xl, const Q4Consts& k, float (&acc)[4][TB]) {
#pragma unroll
  for (int j = 0; j < CPW; ++j)
    if (j < nc) moe_chunk<KIND, TB>(ch[j], c0 + j, TC, xl, k, acc);
}

// The same for units of 8 SL rows (slices i0 .. i0 + SL - 1 of every chunk):
// a row's arithmetic does not depend on how many rows a lane holds.
template <int KIND, int TB, int CPW, int SL>
__device__ __forceinline__ void moe_chunks_sl(const Q4Chunk<KIND, SL> (&ch)[CPW], int nc, int c0, int TC,
                                              const uint32_t* xl, const Q4Consts& k, float (&acc)[SL][TB]) {
  const int R = TB * TC * 8, g = threadIdx.x & 7;
  const float* sums = reinterpret_cast<const float*>(xl + 16 * R);
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    if (j < nc) {
      XRec<TB> xp;
#pragma unroll
      for (int m = 0; m < TB; ++m) {
        const int r = (m * TC + c0 + j) * 8 + g;
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
      q4_compute<KIND, TB, SL>(ch[j], xp, k, acc);
    }
  }
}

template <int KIND, int CPW>
__device__ __forceinline__ void moe_load(const uint8_t* row, int c0, int nc, int lane,
                                         Q4Chunk<KIND> (&ch)[CPW]) {
  constexpr int CB = ChunkBytes<KIND>::value;
#pragma unroll
  for (int j = 0; j < CPW; ++j)
    if (j < nc) q4_load<KIND>(row + (size_t)(c0 + j) * CB, lane, ch[j]);
}

// Segment u: (expert, first sorted position, count).
template <bool SMALL>
__device__ __forceinline__ void moe_seg(const MoeArgs& a, const MoeSmallRoute& rt, int u, int& e,
                                        int& start, int& cnt) {
  if constexpr (SMALL) {
    e = rt.seg[u][0]; start = rt.seg[u][1]; cnt = rt.seg[u][2];
  } else {
    e = a.seg[3 * u]; start = a.seg[3 * u + 1]; cnt = a.seg[3 * u + 2];
  }
}

template <bool SMALL>
__device__ __forceinline__ int moe_sorted(const MoeArgs& a, const MoeSmallRoute& rt, int pos) {
  if constexpr (SMALL) return rt.sorted[pos];
  else return a.sorted[pos];
}

// Items: nseg * (De / 32) routed tile rows, then Ds / 32 shared ones, each cut
// into 4 / SL units of 8 SL rows (more, smaller workgroups for a launch bound
// by each CU's share of the bytes).  Waves 0-1 take the gate rows, 2-3 the up
// rows, each half of the row's chunks.
template <int KIND, int TB, bool SMALL, int SL>
__global__ __launch_bounds__(256) void k_moe_gateup_s(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];
  __shared__ float red[4][8 * SL][TB];
  __shared__ int64_t s_rows[TB];   // the batch's activation rows (element offsets)
  __shared__ MoeSmallRoute rt;
  constexpr int PARTS = 4 / SL, CB = ChunkBytes<KIND>::value;
  if constexpr (SMALL) {
    moe_route_small(a, rt);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.hdr[0] = (uint32_t)rt.bad;
  }
  const int nseg = SMALL ? rt.nseg : (int)a.hdr[1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int TC = a.D / 256, P = a.T * a.k;
  const int rows_r = a.De / 32, rows_s = a.Ds / 32;
  const int n_items = (nseg * rows_r + rows_s) * PARTS;
  const Q4Consts kc = q4_consts();
  const int half = wave & 1;
  const int c0 = half * TC / 2, nc = (half + 1) * TC / 2 - c0;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int unit = item / PARTS, i0 = SL * (item - unit * PARTS);
    const bool shared = unit >= nseg * rows_r;
    int e = 0, start = 0, cnt = a.T, tr;
    if (!shared) {
      const int u = unit / rows_r;
      tr = unit - u * rows_r;
      moe_seg<SMALL>(a, rt, u, e, start, cnt);
    } else {
      tr = unit - nseg * rows_r;
    }
    const uint8_t* w = shared ? (wave < 2 ? a.sgate : a.sup)
                              : (wave < 2 ? a.gate + (size_t)e * a.gate_stride : a.up + (size_t)e * a.up_stride);
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(w + ((size_t)tr * TC + c0) * CB, (uint32_t)(nc * CB));
    constexpr int CPW = kMoeCpwGateUp;
    Q4Chunk<KIND, SL> ch[CPW];
    auto load = [&](int r0) {
#pragma unroll
      for (int j = 0; j < CPW; ++j)
        if (r0 + j < nc) q4_load_rs<KIND, SL>(wrs, (uint32_t)((r0 + j) * CB), lane, ch[j], i0);
    };
    for (int b0 = 0; b0 < cnt; b0 += TB) {
      const int ntok = min(TB, cnt - b0);
      if (threadIdx.x < TB) {
        const int mm = (int)threadIdx.x < ntok ? (int)threadIdx.x : 0;
        const int t = shared ? b0 + mm : moe_sorted<SMALL>(a, rt, start + b0 + mm) / a.k;
        s_rows[threadIdx.x] = (int64_t)t * a.D;
      }
      float acc[SL][TB];
#pragma unroll
      for (int i = 0; i < SL; ++i)
#pragma unroll
        for (int m = 0; m < TB; ++m) acc[i][m] = 0.f;
      // weights first (held across batches when the wave's run fits), then this batch's rows
      if (b0 == 0 && nc <= CPW) load(0);
      __syncthreads();
      moe_stage<TB>(a.X, s_rows, TC, xl);
      __syncthreads();
      for (int r0 = 0; r0 < nc; r0 += CPW) {
        if (nc > CPW) load(r0);
        moe_chunks_sl<KIND, TB, CPW, SL>(ch, min(CPW, nc - r0), c0 + r0, TC, xl, kc, acc);
      }
      q4_lane_reduce<TB, SL>(acc);
      if ((lane & 7) == 0) {
#pragma unroll
        for (int i = 0; i < SL; ++i)
#pragma unroll
          for (int m = 0; m < TB; ++m) red[wave][8 * i + (lane >> 3)][m] = acc[i][m];
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < 8 * SL * TB; idx += 256) {
        const int r = idx / TB, m = idx - r * TB;
        if (m < ntok) {
          const float g = red[0][r][m] + red[1][r][m];
          const float u = red[2][r][m] + red[3][r][m];
          const float hv = g / (1.0f + expf(-g)) * u;
          const int col = 32 * tr + 8 * i0 + r;
          const int pos = shared ? P + b0 + m : start + b0 + m;
          a.hbuf[(size_t)pos * a.hstride + col] = hv;
          if (shared) {
            if (a.dbg_h_shared) a.dbg_h_shared[(size_t)(b0 + m) * a.Ds + col] = hv;
          } else if (a.dbg_h) {
            a.dbg_h[(size_t)moe_sorted<SMALL>(a, rt, pos) * a.De + col] = hv;
          }
        }
      }
      __syncthreads();   // red and xl are reused by the next batch
    }
  }
}

// Items: nseg * (D / 32 / rpw_r) routed row groups, then the shared ones; ks
// waves split a tile row's chunks, rpw = WAVES / ks rows per workgroup.
template <int KIND, int TB, bool SMALL, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_moe_down_s(MoeArgs a, int ks_r, int ks_s) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];
  __shared__ float red[WAVES][32][TB];
  __shared__ int64_t s_rows[TB];   // the batch's activation rows (element offsets)
  __shared__ MoeSmallRoute rt;
  if constexpr (SMALL) moe_route_small(a, rt);
  const int nseg = SMALL ? rt.nseg : (int)a.hdr[1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = a.D / 32, P = a.T * a.k;
  const int gr = rows / (WAVES / ks_r), gs = a.Ds ? rows / (WAVES / ks_s) : 0;
  const int n_items = nseg * gr + gs;
  const Q4Consts kc = q4_consts();
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const bool shared = item >= nseg * gr;
    int e = 0, start = 0, cnt = a.T, grp;
    if (!shared) {
      const int u = item / gr;
      grp = item - u * gr;
      moe_seg<SMALL>(a, rt, u, e, start, cnt);
    } else {
      grp = item - nseg * gr;
    }
    const int ks = shared ? ks_s : ks_r, rpw = WAVES / ks;
    const int TC = (shared ? a.Ds : a.De) / 256;
    const int slot = wave / ks, part = wave % ks;
    const int tr0 = grp * rpw, tr = tr0 + slot;
    const int c0 = part * TC / ks, nc = (part + 1) * TC / ks - c0;
    const uint8_t* row = (shared ? a.sdown : a.down + (size_t)e * a.down_stride) +
                         (size_t)tr * TC * ChunkBytes<KIND>::value;
    constexpr int CPW = kMoeCpwDown;
    Q4Chunk<KIND> ch[CPW];
    for (int b0 = 0; b0 < cnt; b0 += TB) {
      const int ntok = min(TB, cnt - b0);
      if (threadIdx.x < TB) {
        const int mm = (int)threadIdx.x < ntok ? (int)threadIdx.x : 0;
        const int pos = shared ? P + b0 + mm : start + b0 + mm;
        s_rows[threadIdx.x] = (int64_t)pos * a.hstride;
      }
      float acc[4][TB];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < TB; ++m) acc[i][m] = 0.f;
      // weights first (held across batches when the wave's run fits), then this batch's rows
      if (b0 == 0 && nc <= CPW) moe_load<KIND, CPW>(row, c0, nc, lane, ch);
      __syncthreads();
      moe_stage_h<TB>(a.hbuf, s_rows, TC, xl);
      __syncthreads();
      for (int r0 = 0; r0 < nc; r0 += CPW) {
        if (nc > CPW) moe_load<KIND, CPW>(row, c0 + r0, min(CPW, nc - r0), lane, ch);
        moe_chunks<KIND, TB, CPW>(ch, min(CPW, nc - r0), c0 + r0, TC, xl, kc, acc);
      }
      q4_lane_reduce<TB>(acc);
      if ((lane & 7) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int m = 0; m < TB; ++m) red[wave][8 * i + (lane >> 3)][m] = acc[i][m];
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < rpw * 32 * TB; idx += 64 * WAVES) {
        const int s2 = idx / (32 * TB), rem = idx - s2 * 32 * TB;
        const int r = rem / TB, m = rem - r * TB;
        const int t_row = tr0 + s2;
        if (m < ntok) {
          float v = 0.f;
          for (int p2 = 0; p2 < ks; ++p2) v += red[s2 * ks + p2][r][m];
          const int dst = shared ? P + b0 + m : moe_sorted<SMALL>(a, rt, start + b0 + m);
          a.dbuf[(size_t)dst * a.D + 32 * t_row + r] = v;
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// prompt blocks: one work item per (token batch, tile row or row group)
// ---------------------------------------------------------------------------
// Many pairs (after the route kernel): an item is one batch of up to TB tokens
// of one segment against one tile row (gate/up) or row group (down), so a
// popular expert's batches spread over many CUs.  Each item issues its weight
// loads first, then prepares its batch's activation rows in LDS as the
// weight-stationary kernels do, and runs the same arithmetic (chunk split,
// chunk order, reduction order), so a token's bits do not depend on its batch.

// Waves 0-1 run the gate tile row, waves 2-3 the up tile row, each pair
// splitting the D/256 chunks in two halves.
// cls 0: every item; 1: only routed batches of one token (then TB = 1, whose
// registers let twice the workgroups share a CU); 2: every item but those.
// A token's arithmetic is the same in either kernel, so its bits are too.
template <int KIND, int TB>
__global__ __launch_bounds__(256) void k_moe_gateup(MoeArgs a, int cls) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];
  __shared__ float red[4][32][TB];
  __shared__ int64_t s_rows[TB];   // the batch's activation rows (element offsets)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int TC = a.D / 256;
  const int rows_r = a.De / 32, rows_s = a.Ds / 32;
  const int P = a.T * a.k;
  const int half = wave & 1;
  const int c0 = half * TC / 2, nc = (half + 1) * TC / 2 - c0;
  constexpr int CPW = kMoeCpwBatch;
  const Q4Consts kc = q4_consts();
  const int nbr = (int)a.hdr[2];
  for (int item = blockIdx.x;; item += gridDim.x) {
    MoeItem it;
    if (cls == 1 && item >= nbr * rows_r) break;   // the routed items come first
    if (!moe_item<TB>(a, nbr, item, rows_r, rows_s, 1, 1, false, it)) break;
    if ((cls == 1 && it.ntok != 1) || (cls == 2 && !it.shared && it.ntok == 1)) continue;
    const uint8_t* row = (wave < 2 ? it.w0 : it.w1) + (size_t)it.tr * TC * ChunkBytes<KIND>::value;
    Q4Chunk<KIND> ch[CPW];
    moe_load<KIND, CPW>(row, c0, min(CPW, nc), lane, ch);   // weights first: the first CPW chunks
    if (threadIdx.x < TB) s_rows[threadIdx.x] = (int64_t)moe_item_tok(a, it, threadIdx.x) * a.D;
    float acc[4][TB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < TB; ++m) acc[i][m] = 0.f;
    __syncthreads();
    moe_stage<TB>(a.X, s_rows, TC, xl);
    __syncthreads();
    // a ring of CPW slots: chunk j in slot j % CPW, and once its products are
    // done, chunk j + CPW is issued into the slot (same chunk order as ever)
    for (int j0 = 0; j0 < nc; j0 += CPW) {
#pragma unroll
      for (int jj = 0; jj < CPW; ++jj) {
        const int j = j0 + jj;
        if (j < nc) {
          moe_chunk<KIND, TB>(ch[jj], c0 + j, TC, xl, kc, acc);
          if (j + CPW < nc) q4_load<KIND>(row + (size_t)(c0 + j + CPW) * ChunkBytes<KIND>::value, lane, ch[jj]);
        }
      }
    }
    q4_lane_reduce<TB>(acc);
    if ((lane & 7) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < TB; ++m) red[wave][8 * i + (lane >> 3)][m] = acc[i][m];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * TB; idx += 256) {
      const int r = idx / TB, m = idx - r * TB;
      if (m < it.ntok) {
        const float g = red[0][r][m] + red[1][r][m];
        const float u = red[2][r][m] + red[3][r][m];
        const float hv = g / (1.0f + expf(-g)) * u;
        const int col = 32 * it.tr + r;
        a.hbuf[(size_t)(it.pos0 + m) * a.hstride + col] = hv;
        if (it.shared) {
          if (a.dbg_h_shared) a.dbg_h_shared[(size_t)(it.pos0 - P + m) * a.Ds + col] = hv;
        } else if (a.dbg_h) {
          a.dbg_h[(size_t)moe_item_pair(a, it, m) * a.De + col] = hv;
        }
      }
    }
    __syncthreads();   // red and xl are reused by the next item
  }
}

// ks waves split one tile row's chunks; WAVES/ks tile rows per workgroup.
// cls as in k_moe_gateup.
template <int KIND, int TB, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_moe_down(MoeArgs a, int ks_r, int ks_s, int cls) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];
  __shared__ float red[WAVES][32][TB];
  __shared__ int64_t s_rows[TB];   // the batch's activation rows (element offsets)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = a.D / 32;
  constexpr int CPW = kMoeCpwDown;
  const Q4Consts kc = q4_consts();
  const int nbr = (int)a.hdr[2];
  for (int item = blockIdx.x;; item += gridDim.x) {
    MoeItem it;
    if (cls == 1 && item >= nbr * (rows / (WAVES / ks_r))) break;   // the routed items come first
    if (!moe_item<TB>(a, nbr, item, rows, rows, WAVES / ks_r, WAVES / ks_s, true, it)) break;
    if ((cls == 1 && it.ntok != 1) || (cls == 2 && !it.shared && it.ntok == 1)) continue;
    const int ks = it.shared ? ks_s : ks_r, rpw = WAVES / ks;
    const int TC = (it.shared ? a.Ds : a.De) / 256;
    const int slot = wave / ks, part = wave % ks;
    const int tr = it.tr + slot < rows ? it.tr + slot : rows - 1;   // past the last row: redone, unstored
    const int c0 = part * TC / ks, nc = (part + 1) * TC / ks - c0;
    const uint8_t* row = it.w0 + (size_t)tr * TC * ChunkBytes<KIND>::value;
    Q4Chunk<KIND> ch[CPW];
    if (nc <= CPW) moe_load<KIND, CPW>(row, c0, nc, lane, ch);   // weights first
    if (threadIdx.x < TB) {
      const int mm = (int)threadIdx.x < it.ntok ? (int)threadIdx.x : 0;
      s_rows[threadIdx.x] = (int64_t)(it.pos0 + mm) * a.hstride;
    }
    float acc[4][TB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < TB; ++m) acc[i][m] = 0.f;
    __syncthreads();
    moe_stage_h<TB>(a.hbuf, s_rows, TC, xl);
    __syncthreads();
    for (int r0 = 0; r0 < nc; r0 += CPW) {
      if (nc > CPW) moe_load<KIND, CPW>(row, c0 + r0, min(CPW, nc - r0), lane, ch);
      moe_chunks<KIND, TB, CPW>(ch, min(CPW, nc - r0), c0 + r0, TC, xl, kc, acc);
    }
    q4_lane_reduce<TB>(acc);
    if ((lane & 7) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < TB; ++m) red[wave][8 * i + (lane >> 3)][m] = acc[i][m];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < rpw * 32 * TB; idx += 64 * WAVES) {
      const int s2 = idx / (32 * TB), rem = idx - s2 * 32 * TB;
      const int r = rem / TB, m = rem - r * TB;
      const int t_row = it.tr + s2;
      if (m < it.ntok && t_row < rows) {
        float v = 0.f;
        for (int p2 = 0; p2 < ks; ++p2) v += red[s2 * ks + p2][r][m];
        a.dbuf[(size_t)moe_item_pair(a, it, m) * a.D + 32 * t_row + r] = v;
      }
    }
    __syncthreads();   // red and xl are reused by the next item
  }
}

// ---------------------------------------------------------------------------
// experts with many tokens: bf16 matrix-core tiles
// ---------------------------------------------------------------------------
// A unit (a segment of at least hot_min pairs, or the shared expert when
// T >= hot_min) is cut into work items of 64 token rows times a group of tile
// rows.  Each chunk of the group is read once per item and dequantised once to
// two bf16 parts (hi = bf16(w), lo = bf16(w - hi): each weight to 2^-16 of
// its size, so the per-output bound holds however the terms of a sum are
// distributed), and v_mfma_f32_32x32x16 multiplies both against all 64 rows
// at once, where the batched kernels above would re-read the expert per batch
// of 4 tokens and spend a dot2 chain per token.  The token rows are gathered into an LDS tile per tile column,
// double buffered, shared by the workgroup's 8 waves.  Rows past the unit's
// count repeat its first token and are never stored.
//
// A token's bits depend on whether its expert reached hot_min pairs in the
// call (a different order of sums and of roundings), within the same
// per-output bound either way.

// The unit of work item `item` (first items at field f of the unit records),
// or -1 when none holds it.  *s_unit is -1 on entry; the caller sets it back
// before the barrier that ends the item.
__device__ __forceinline__ int moe_hot_unit(const MoeArgs& a, int item, int nh, int nitems, int f,
                                            int32_t* s_unit) {
  for (int u = threadIdx.x; u < nh; u += blockDim.x) {
    const int f0 = a.hot[(size_t)u * kMoeHotInts + f];
    const int f1 = u + 1 < nh ? a.hot[(size_t)(u + 1) * kMoeHotInts + f] : nitems;
    if (f0 <= item && item < f1) *s_unit = u;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_unit);
}

// Token slots of an item: X row (element offset, gate/up), h row (hbuf row,
// down), destination (pair index routed, P + t shared), valid flag.
struct MoeHotSlots {
  int64_t xrow[kMoeHotTokens];
  int32_t hrow[kMoeHotTokens];
  int32_t dst[kMoeHotTokens];
  int32_t valid[kMoeHotTokens];
};

__device__ __forceinline__ void moe_hot_slots(const MoeArgs& a, bool shared, int start, int m0, int nb,
                                              MoeHotSlots& sl) {
  const int P = a.T * a.k, t = threadIdx.x;
  if (t < kMoeHotTokens) {
    const int mm = m0 + (t < nb ? t : 0);
    int tok, hrow, dst;
    if (shared) {
      tok = mm;
      hrow = P + mm;
      dst = P + mm;
    } else {
      dst = a.sorted[start + mm];
      tok = dst / a.k;
      hrow = start + mm;
    }
    sl.xrow[t] = (int64_t)tok * a.D;
    sl.hrow[t] = hrow;
    sl.dst[t] = dst;
    sl.valid[t] = t < nb;
  }
}

// gate/up: an item is 64 token rows times 2 tile rows of gate and the same 2
// of up.  Wave w runs tile row 2g + (w & 1) of gate or up ((w >> 1) & 1) over
// one half of K (w >> 2); the halves meet in LDS (first + second), then the
// up waves hand their sums to the gate waves, which write h = silu(g) u in
// fp32.  Items of at most 32 token rows skip the second token tile.
template <int KIND>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_moe_hot_gu(MoeArgs a) {
  constexpr int CB = ChunkBytes<KIND>::value, NH = 256, XR = kMoeHotTokens;
  constexpr int XP = XR * 32 / NH;   // 16-byte X pieces per thread and tile of its half
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][2][XR * kXs];   // [buffer][half]
  __shared__ MoeHotSlots sl;
  __shared__ int32_t s_unit;
  static_assert(sizeof(xs) >= (4 + 2) * 8 * 64 * 16, "LDS for the exchanges of sums");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n = lane & 31;
  const int half = wave >> 2, proj = (wave >> 1) & 1, rsub = wave & 1;
  const int th = tid & (NH - 1);
  const int nh = (int)a.hdr[3], nitems = (int)a.hdr[4];
  const int TC = a.D / 256, P = a.T * a.k;
  const int mid = (TC + 1) / 2, hc0 = half ? mid : 0, hc1 = half ? TC : mid;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.X, (uint32_t)((size_t)a.T * a.D * 2));
  uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  asm volatile("" : "+s"(kMaskLo));
  asm volatile("" : "+s"(kMaskHi));
  asm volatile("" : "+v"(kMagic));
  if (tid == 0) s_unit = -1;
  __syncthreads();
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int u = moe_hot_unit(a, item, nh, nitems, 3, &s_unit);
    if (u < 0) {   // (a unit table that does not cover the item: nothing to do)
      __syncthreads();   // every wave has read the unit before any writes the next
      continue;
    }
    const int32_t* rec = a.hot + (size_t)u * kMoeHotInts;
    const int e = rec[0], start = rec[1], cnt = rec[2], first = rec[3];
    const bool shared = e < 0;
    const int G = (shared ? a.Ds : a.De) / 64;
    const int local = item - first, blk = local / G, g = local - blk * G;
    const int tr = 2 * g + rsub;
    const int m0 = blk * XR, nb = min(XR, cnt - m0);
    moe_hot_slots(a, shared, start, m0, nb, sl);
    const uint8_t* wbase = shared ? (proj ? a.sup : a.sgate)
                                  : (proj ? a.up + (size_t)e * a.up_stride : a.gate + (size_t)e * a.gate_stride);
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(wbase + ((size_t)tr * TC + hc0) * CB, (uint32_t)((hc1 - hc0) * CB));
    GemmChunk<KIND> c[2];
    gemm_load<KIND>(wrs, 0, n, h, c[0]);
    gemm_load<KIND>(wrs, CB, n, h, c[1]);
    __syncthreads();   // the slots are in LDS
    uint32_t xo[XP];
#pragma unroll
    for (int p = 0; p < XP; ++p) xo[p] = (uint32_t)(sl.xrow[(th >> 5) + 8 * p] + (th & 31) * 8) * 2;
    u32x4 xr[XP];
    auto xload = [&](int t) {   // tile column hc0 + t of this half
#pragma unroll
      for (int p = 0; p < XP; ++p)
        xr[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xo[p] + (hc0 + t) * 512, 0, 0));
    };
    auto xstore = [&](int buf) {
#pragma unroll
      for (int p = 0; p < XP; ++p)
        *reinterpret_cast<u32x4*>(&xs[buf][half][((th >> 5) + 8 * p) * kXs + (th & 31) * 8]) = xr[p];
    };
    f32x16 acc0, acc1;
#pragma unroll
    for (int v = 0; v < 16; ++v) { acc0[v] = 0.f; acc1[v] = 0.f; }
    if (hc0 < hc1) xload(0);
    xstore(0);
    // The second half may have one step fewer: its waves skip that step's
    // loads and products but keep to the barriers.
    auto run = [&](auto two_c) {
      constexpr bool TWO = decltype(two_c)::value;
      auto step = [&](int jc, int t) {
        const int j = t & 1;
        const bool mine = hc0 + t < hc1, next = hc0 + t + 1 < hc1;
        __syncthreads();   // X tile t is in xs[j]; xs[j ^ 1] is free
        if (next) xload(t + 1);
        __builtin_amdgcn_sched_barrier(0);
        if (mine)
          mfma_tile_w2<KIND, TWO>(c[jc], xs[j][half] + n * kXs + 128 * h, 32 * kXs, acc0, acc1, kMaskLo,
                                  kMaskHi, kMagic);
        gemm_load<KIND>(wrs, (uint32_t)(t + 2) * CB, n, h, c[jc]);   // past the half: zeros
        if (next) xstore(j ^ 1);
      };
      for (int t = 0; t < mid; t += 2) {
        step(0, t);
        if (t + 1 < mid) step(1, t + 1);
      }
    };
    if (nb > 32) run(std::true_type{});
    else run(std::false_type{});
    __syncthreads();   // every product is done: xs holds the exchanges now
    f32x4* red = reinterpret_cast<f32x4*>(&xs[0][0][0]);   // [4 waves of half 1][8 groups][64 lanes]
    f32x4* red2 = red + 4 * 8 * 64;                       // [2 up waves][8 groups][64 lanes]
    // group g8 of a wave's sums: registers 4 g8 .. 4 g8 + 3 of acc0 (g8 < 4) or acc1
    auto part = [&](int g8) -> f32x4 {
      const f32x16& A = g8 < 4 ? acc0 : acc1;
      const int b = 4 * (g8 & 3);
      return f32x4{A[b], A[b + 1], A[b + 2], A[b + 3]};
    };
    auto add = [&](int g8, f32x4 v) {
      f32x16& A = g8 < 4 ? acc0 : acc1;
      const int b = 4 * (g8 & 3);
#pragma unroll
      for (int i = 0; i < 4; ++i) A[b + i] += v[i];
    };
    if (half == 1) {
#pragma unroll
      for (int g8 = 0; g8 < 8; ++g8) red[((wave & 3) * 8 + g8) * 64 + lane] = part(g8);
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int g8 = 0; g8 < 8; ++g8) add(g8, red[((wave & 3) * 8 + g8) * 64 + lane]);
      if (proj == 1) {
#pragma unroll
        for (int g8 = 0; g8 < 8; ++g8) red2[(rsub * 8 + g8) * 64 + lane] = part(g8);
      }
    }
    __syncthreads();
    if (half == 0 && proj == 0) {
      const int col = 32 * tr + n;
#pragma unroll
      for (int g8 = 0; g8 < 8; ++g8) {
        const f32x4 uu = red2[(rsub * 8 + g8) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // register v of a 32x32 tile: token row 8 (v / 4) + 4 h + v % 4
          const int m = 32 * (g8 >> 2) + 8 * (g8 & 3) + 4 * h + i;
          const float gv = (g8 < 4 ? acc0 : acc1)[4 * (g8 & 3) + i];
          if (sl.valid[m]) {
            const float hv = gv / (1.0f + expf(-gv)) * uu[i];
            a.hbuf[(size_t)sl.hrow[m] * a.hstride + col] = hv;
            if (shared) {
              if (a.dbg_h_shared) a.dbg_h_shared[(size_t)(sl.dst[m] - P) * a.Ds + col] = hv;
            } else if (a.dbg_h) {
              a.dbg_h[(size_t)sl.dst[m] * a.De + col] = hv;
            }
          }
        }
      }
    }
    if (tid == 0) s_unit = -1;
    __syncthreads();   // xs, the slots and the unit are reused by the next item
  }
}

// down: an item is 64 token rows times 8 tile rows of down (one per wave) over
// all of the unit's inner width (items of at most 32 token rows skip the
// second token tile).  h (fp32) enters as two bf16 tiles,
// hi = bf16(h) and lo = bf16(h - hi), which carry h to 2^-16 of its size;
// d = whi hhi + wlo hhi + whi hlo in fp32, stored by pair for the combine.
template <int KIND>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_moe_hot_dn(MoeArgs a) {
  constexpr int CB = ChunkBytes<KIND>::value, NT = 512, XR = kMoeHotTokens;
  constexpr int HP = XR * 64 / NT;   // 16-byte pieces of fp32 h per thread and tile
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][2][XR * kXs];   // [buffer][hi, lo]
  __shared__ MoeHotSlots sl;
  __shared__ int32_t s_unit;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n = lane & 31;
  const int nh = (int)a.hdr[3], nitems = (int)a.hdr[5];
  const int G = a.D / 256;
  const __amdgpu_buffer_rsrc_t hrs =
      make_rsrc(a.hbuf, (uint32_t)((size_t)(a.T * a.k + a.T) * a.hstride * 4));
  uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  asm volatile("" : "+s"(kMaskLo));
  asm volatile("" : "+s"(kMaskHi));
  asm volatile("" : "+v"(kMagic));
  if (tid == 0) s_unit = -1;
  __syncthreads();
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int u = moe_hot_unit(a, item, nh, nitems, 4, &s_unit);
    if (u < 0) {   // (a unit table that does not cover the item: nothing to do)
      __syncthreads();   // every wave has read the unit before any writes the next
      continue;
    }
    const int32_t* rec = a.hot + (size_t)u * kMoeHotInts;
    const int e = rec[0], start = rec[1], cnt = rec[2], first = rec[4];
    const bool shared = e < 0;
    const int TC = (shared ? a.Ds : a.De) / 256;
    const int local = item - first, blk = local / G, g = local - blk * G;
    const int tr = 8 * g + wave;
    const int m0 = blk * XR, nb = min(XR, cnt - m0);
    moe_hot_slots(a, shared, start, m0, nb, sl);
    const uint8_t* wbase = shared ? a.sdown : a.down + (size_t)e * a.down_stride;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wbase + (size_t)tr * TC * CB, (uint32_t)(TC * CB));
    GemmChunk<KIND> c[2];
    gemm_load<KIND>(wrs, 0, n, h, c[0]);
    gemm_load<KIND>(wrs, CB, n, h, c[1]);
    __syncthreads();   // the slots are in LDS
    uint32_t ho[HP];
#pragma unroll
    for (int p = 0; p < HP; ++p) ho[p] = (uint32_t)(sl.hrow[(tid >> 6) + 8 * p] * a.hstride + (tid & 63) * 4) * 4;
    f32x4 hr[HP];
    auto hload = [&](int t) {
#pragma unroll
      for (int p = 0; p < HP; ++p)
        hr[p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(hrs, ho[p] + t * 1024, 0, 0));
    };
    auto hstore = [&](int buf) {
#pragma unroll
      for (int p = 0; p < HP; ++p) {
        const int off = ((tid >> 6) + 8 * p) * kXs + (tid & 63) * 4;
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 b = (__bf16)hr[p][i];
          hi[i] = __builtin_bit_cast(uint16_t, b);
          lo[i] = __builtin_bit_cast(uint16_t, (__bf16)(hr[p][i] - (float)b));
        }
        *reinterpret_cast<u32x2*>(&xs[buf][0][off]) = u32x2{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)};
        *reinterpret_cast<u32x2*>(&xs[buf][1][off]) = u32x2{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16)};
      }
    };
    f32x16 acc0, acc1;
#pragma unroll
    for (int v = 0; v < 16; ++v) { acc0[v] = 0.f; acc1[v] = 0.f; }
    hload(0);
    hstore(0);
    auto run = [&](auto two_c) {
      constexpr bool TWO = decltype(two_c)::value;
      auto step = [&](int jc, int t) {
        const int j = t & 1;
        __syncthreads();   // h tiles of step t are in xs[j]; xs[j ^ 1] is free
        if (t + 1 < TC) hload(t + 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_tile_hl<KIND, TWO>(c[jc], xs[j][0] + n * kXs + 128 * h, 32 * kXs, XR * kXs, acc0, acc1, kMaskLo,
                                kMaskHi, kMagic);
        gemm_load<KIND>(wrs, (uint32_t)(t + 2) * CB, n, h, c[jc]);   // past the row: zeros
        if (t + 1 < TC) hstore(j ^ 1);
      };
      for (int t = 0; t < TC; t += 2) {
        step(0, t);
        if (t + 1 < TC) step(1, t + 1);
      }
    };
    if (nb > 32) run(std::true_type{});
    else run(std::false_type{});
    const int col = 32 * tr + n;
#pragma unroll
    for (int v = 0; v < 32; ++v) {
      const int m = 32 * (v >> 4) + 8 * ((v & 15) >> 2) + 4 * h + (v & 3);
      const float dv = v < 16 ? acc0[v] : acc1[v - 16];
      if (sl.valid[m]) a.dbuf[(size_t)sl.dst[m] * a.D + col] = dv;
    }
    if (tid == 0) s_unit = -1;
    __syncthreads();   // xs, the slots and the unit are reused by the next item
  }
}

// ---------------------------------------------------------------------------
// decode-sized down projection and combine in one launch
// ---------------------------------------------------------------------------
// A workgroup owns 8 output rows (one slice of a tile row) for every token:
// it computes d of those rows for every valid pair and for the shared expert,
// then sums them per token in slot order, so d never goes through memory and
// no second launch runs.  The arithmetic is that of k_moe_down_s and
// k_moe_combine -- per row the same chunk split over ks waves, the same chunk
// order, lane reduction, part order and slot order -- so the results are
// those of the two-launch path bit for bit (a row's sum does not depend on how
// many rows a lane holds).  With D / 8 workgroups every CU streams a share of
// the selected experts' down rows.
constexpr int kMoeDcSlices = 4;   // chunk slices a down task may hold (tile columns per wave)

constexpr int kMoeDcWaves = 16;

template <int KIND>
__global__ __launch_bounds__(64 * kMoeDcWaves) void k_moe_down_c(MoeArgs a, int ks_r, int ks_s) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];
  __shared__ MoeSmallRoute rt;
  __shared__ int32_t s_pos[kMoeSmallPairs];   // each pair's sorted position, -1 when invalid
  __shared__ int32_t s_exp[kMoeSmallPairs];   // the expert of each valid sorted position
  constexpr int CB = ChunkBytes<KIND>::value, W = kMoeDcWaves, NT = 64 * W;
  moe_route_small(a, rt);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = a.T * a.k, T = a.T;
  const int nseg = rt.nseg;
  const int Pv = nseg ? rt.seg[nseg - 1][1] + rt.seg[nseg - 1][2] : 0;   // valid pairs sort first
  const int TCr = a.De / 256, TCs = a.Ds / 256;
  const int u = blockIdx.x, tr = u >> 2, i0 = u & 3;   // output rows 8u .. 8u + 7
  const int NRr = Pv * TCr * 8, NR = NRr + T * TCs * 8;
  float* sums = reinterpret_cast<float*>(xl + 16 * NR);
  float* dpart = sums + 2 * NR;   // [task][8 rows]
  const int n_r = Pv * ks_r, n_tasks = n_r + (a.Ds ? T * ks_s : 0);
  for (int q = tid; q < P; q += NT) {
    const int pr = rt.sorted[q];
    s_pos[pr] = q < Pv ? q : -1;
  }
  if (tid < nseg)
    for (int q = rt.seg[tid][1]; q < rt.seg[tid][1] + rt.seg[tid][2]; ++q) s_exp[q] = rt.seg[tid][0];
  __syncthreads();

  // A task: one wave's chunks [c0, c1) of one row (a valid pair's routed row,
  // or a token's shared row), against that row's h records.
  struct Task {
    __amdgpu_buffer_rsrc_t rs;
    int nc, c0, rbase, TC;
  };
  auto task = [&](int ti) {
    Task tk;
    const bool shared = ti >= n_r;
    const int ks = shared ? ks_s : ks_r, TC = shared ? TCs : TCr;
    const int idx = shared ? (ti - n_r) / ks_s : ti / ks_r, part = shared ? (ti - n_r) - idx * ks_s : ti - idx * ks_r;
    const int c0 = part * TC / ks, c1 = (part + 1) * TC / ks;
    const uint8_t* row = shared ? a.sdown : a.down + (size_t)s_exp[idx] * a.down_stride;
    row += ((size_t)tr * TC + c0) * CB;
    tk.rs = make_rsrc(row, (uint32_t)((c1 - c0) * CB));
    tk.nc = c1 - c0;
    tk.c0 = c0;
    tk.rbase = shared ? NRr + idx * TCs * 8 : idx * TCr * 8;
    tk.TC = TC;
    return tk;
  };
  Q4Chunk<KIND, 1> ring[2][kMoeDcSlices];
  auto load = [&](int b, const Task& tk) {
#pragma unroll
    for (int j = 0; j < kMoeDcSlices; ++j)
      if (j < tk.nc) q4_load_rs<KIND, 1>(tk.rs, (uint32_t)(j * CB), lane, ring[b][j], i0);
  };
  const Q4Consts kc = q4_consts();
  auto compute = [&](int b, const Task& tk, int ti) {
    float acc[1][1] = {{0.f}};
    const int g = lane & 7;
#pragma unroll
    for (int j = 0; j < kMoeDcSlices; ++j) {
      if (j < tk.nc) {
        const int r = tk.rbase + (tk.c0 + j) * 8 + g;
        XRec<1> xp;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(xl + 16 * r + 4 * d);
          xp.p[0][4 * d] = v.x;
          xp.p[0][4 * d + 1] = v.y;
          xp.p[0][4 * d + 2] = v.z;
          xp.p[0][4 * d + 3] = v.w;
        }
        xp.f[0] = sums[2 * r];
        xp.X[0] = sums[2 * r + 1];
        q4_compute<KIND, 1, 1>(ring[b][j], xp, kc, acc);
      }
    }
    q4_lane_reduce<1, 1>(acc);
    if (g == 0) dpart[ti * 8 + (lane >> 3)] = acc[0][0];
  };

  // weights of the wave's first task first, then the h records of every row
  int ti = wave;
  Task cur;
  if (ti < n_tasks) {
    cur = task(ti);
    load(0, cur);
  }
  // h records, four quarter records per thread per round: all four rounds'
  // loads are issued before any is built (quarter records past 4 NR read a
  // valid row again and are not stored)
  auto hsrc = [&](int q4) {
    const int r = min(q4 >> 2, NR - 1);
    if (r < NRr) {
      const int q = r / (TCr * 8), rem = r - q * TCr * 8;
      return a.hbuf + (size_t)q * a.hstride + 32 * rem + 8 * (q4 & 3);
    }
    const int r2 = r - NRr, t = r2 / (TCs * 8), rem = r2 - t * TCs * 8;
    return a.hbuf + (size_t)(P + t) * a.hstride + 32 * rem + 8 * (q4 & 3);
  };
  constexpr int HB = 4;
  for (int q0 = tid; q0 < 4 * NR; q0 += NT * HB) {
    f32x4 va[HB], vb[HB];
#pragma unroll
    for (int i = 0; i < HB; ++i) {
      const float* src = hsrc(q0 + NT * i);
      va[i] = *reinterpret_cast<const f32x4*>(src);
      vb[i] = *reinterpret_cast<const f32x4*>(src + 4);
    }
#pragma unroll
    for (int i = 0; i < HB; ++i) {
      const int q4 = q0 + NT * i, r = q4 >> 2;
      if (r < NR) {
        uint32_t pr[4];
        float f, X;
        h_record_part(va[i], vb[i], pr, f, X);
        *reinterpret_cast<u32x4*>(xl + 16 * r + 4 * (q4 & 3)) = u32x4{pr[0], pr[1], pr[2], pr[3]};
        if ((q4 & 3) == 0) {
          sums[2 * r] = f;
          sums[2 * r + 1] = X;
        }
      }
    }
  }
  __syncthreads();
  // the wave's tasks, the next one's chunks loaded while the current one runs
  while (ti < n_tasks) {
    Task nxt;
    const bool more = ti + W < n_tasks;
    if (more) {
      nxt = task(ti + W);
      load(1, nxt);
    }
    compute(0, cur, ti);
    ti += W;
    if (!more) break;
    cur = nxt;
    const bool more2 = ti + W < n_tasks;
    if (more2) {
      nxt = task(ti + W);
      load(0, nxt);
    }
    compute(1, cur, ti);
    ti += W;
    if (!more2) break;
    cur = nxt;
  }
  __syncthreads();
  // y[t][row] = sum_j p[t][j] d[t][j][row] in slot order, then + the shared d
  for (int idx = tid; idx < T * 8; idx += NT) {
    const int t = idx >> 3, r = idx & 7, col = 8 * u + r;
    float y = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const int pair = t * a.k + j;
      const int e = a.ids[pair];
      const int pos = s_pos[pair];
      const bool ok = e >= 0 && e < a.n_experts && pos >= 0;
      float dj = 0.f;
      if (ok) {
        float v = 0.f;
        for (int p2 = 0; p2 < ks_r; ++p2) v += dpart[(pos * ks_r + p2) * 8 + r];
        dj = v;
        y = fmaf(a.p[pair], dj, y);
      }
      if (a.dbg_d) a.dbg_d[(size_t)pair * a.D + col] = dj;
    }
    if (a.Ds) {
      float ds = 0.f;
      for (int p2 = 0; p2 < ks_s; ++p2) ds += dpart[(n_r + t * ks_s + p2) * 8 + r];
      y += ds;
      if (a.dbg_d_shared) a.dbg_d_shared[(size_t)t * a.D + col] = ds;
    }
    a.Y[(size_t)t * a.D + col] = y;
  }
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------
// Every load of a thread is issued before the first product: ids, weights and
// the k partial rows come through buffer resources, so slots past k read zero
// without a branch, and the sum runs in slot order once they have arrived.
__global__ __launch_bounds__(256) void k_moe_combine(MoeArgs a) {
  constexpr int KM = kMoeMaxK;
  const int t = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= a.D) return;
  const int P = a.T * a.k;
  const __amdgpu_buffer_rsrc_t ir = make_rsrc(a.ids + (size_t)t * a.k, (uint32_t)a.k * 4u);
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.p + (size_t)t * a.k, (uint32_t)a.k * 4u);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.dbuf + (size_t)t * a.k * a.D, (uint32_t)(a.k * a.D) * 4u);
  int e[KM];
  float pj[KM], d[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    e[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, 4u * j, 0, 0);
    pj[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, 4u * j, 0, 0));
    d[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dr, (uint32_t)(j * a.D + n) * 4u, 0, 0));
  }
  const float ds = a.Ds ? a.dbuf[(size_t)(P + t) * a.D + n] : 0.f;
  float y = 0.f;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < a.k) {
      const bool ok = e[j] >= 0 && e[j] < a.n_experts;
      const float dj = ok ? d[j] : 0.f;
      if (ok) y = fmaf(pj[j], dj, y);
      if (a.dbg_d) a.dbg_d[(size_t)(t * a.k + j) * a.D + n] = dj;
    }
  }
  if (a.Ds) {
    y += ds;
    if (a.dbg_d_shared) a.dbg_d_shared[(size_t)t * a.D + n] = ds;
  }
  a.Y[(size_t)t * a.D + n] = y;
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
template <int KIND, int TB>
static hipError_t moe_run(const MoeArgs& a, hipStream_t s) {
  const int P = a.T * a.k;
  const int nseg_max = P < a.n_experts ? P : a.n_experts;
  const int tcr = a.De / 256, tcs = a.Ds ? a.Ds / 256 : 1;
  // Waves per tile row in the down kernels: about two chunks per wave.  (One
  // chunk per wave, ks = TC up to 4, measured 10% slower at T = 64 and 4%
  // faster at T = 1.  Both paths must use the same split for a token's bits
  // not to depend on T.)
  const int ks_r = tcr >= 8 ? 4 : (tcr >= 4 ? 2 : 1);
  const int ks_s = tcs >= 8 ? 4 : (tcs >= 4 ? 2 : 1);
  const int rows = a.D / 32;
  // Few pairs (decode): weight-stationary kernels with routing in every
  // workgroup, when a batch's prepared rows fit in 64 KB of LDS.  Many pairs
  // (prompt blocks): the route kernel, then one work item per (token batch,
  // tile row), which spreads a popular expert's batches over many CUs (holding
  // its chunks in one workgroup serialises them, measured slower).
  const int xl_gu = kMoeRecGateUp * TB * (a.D / 256);
  const int xl_dn = kMoeRecDown * TB * ((a.De > a.Ds ? a.De : a.Ds) / 256);
  const bool small = P <= kMoeSmallPairs;
  if (small && xl_gu <= 65536 && xl_dn <= 65536) {
    constexpr int kGuSl = 1;   // 8-row units: four workgroups per gate/up tile row
    const int gu_items = (nseg_max * (a.De / 32) + a.Ds / 32) * (4 / kGuSl);
    // decode-sized down: two-wave workgroups when a tile row takes at most two waves
    // (more, smaller workgroups for a latency-bound launch), else four
    const int dn_waves = (ks_r <= 2 && ks_s <= 2) ? 2 : 4;
    const int dn_items = nseg_max * (rows / (dn_waves / ks_r)) + (a.Ds ? rows / (dn_waves / ks_s) : 0);
    const dim3 g_gu(gu_items < 4096 ? gu_items : 4096), g_dn(dn_items < 4096 ? dn_items : 4096);
    hipLaunchKernelGGL((k_moe_gateup_s<KIND, TB, true, kGuSl>), g_gu, dim3(256), xl_gu, s, a);
    // down and combine in one launch when every row's h records fit in LDS and
    // a wave's run of a row is at most kMoeDcSlices chunks
    const int dc_rec = (P * tcr + (a.Ds ? a.T * tcs : 0)) * 8;
    const int dc_bytes = dc_rec * 72 + (P * ks_r + (a.Ds ? a.T * ks_s : 0)) * 8 * 4;
    const bool dc = dc_bytes <= 131072 && (tcr + ks_r - 1) / ks_r <= kMoeDcSlices &&
                    (tcs + ks_s - 1) / ks_s <= kMoeDcSlices;
    if (dc) {
      if (dc_bytes > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_moe_down_c<KIND>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, dc_bytes);
      hipLaunchKernelGGL((k_moe_down_c<KIND>), dim3(a.D / 8), dim3(64 * kMoeDcWaves), dc_bytes, s, a, ks_r, ks_s);
      return hipGetLastError();
    }
    if (dn_waves == 2)
      hipLaunchKernelGGL((k_moe_down_s<KIND, TB, true, 2>), g_dn, dim3(128), xl_dn, s, a, ks_r, ks_s);
    else
      hipLaunchKernelGGL((k_moe_down_s<KIND, TB, true, 4>), g_dn, dim3(256), xl_dn, s, a, ks_r, ks_s);
    hipLaunchKernelGGL(k_moe_combine, dim3((a.D + 255) / 256, a.T), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int nb_r = (P + nseg_max * (TB - 1)) / TB;        // bound on routed batches
  const int nb_s = a.Ds ? (a.T + TB - 1) / TB : 0;
  hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(1024), 0, s, a);
  // experts with at least hot_min pairs (and the shared expert when T >= hot_min)
  // on the matrix cores; one persistent workgroup per CU walks their items
  const bool hot = a.hot_min > 0;
  if (hot) hipLaunchKernelGGL((k_moe_hot_gu<KIND>), dim3(256), dim3(512), 0, s, a);
  // Batches of several tokens and the shared expert at TB; with TB = 4, the
  // batches of one token (most of a prompt block's experts) in a TB = 1 launch
  // of their own first.
  const bool split = TB > 1 && Q4NX_MOE_SPLIT_SINGLE;
  const int gu_items = nb_r * (a.De / 32) + nb_s * (a.Ds / 32);
  if (split) {
    const int gu1 = nb_r * (a.De / 32);
    hipLaunchKernelGGL((k_moe_gateup<KIND, 1>), dim3(gu1 < 4096 ? gu1 : 4096), dim3(256),
                       kMoeRecGateUp * (a.D / 256), s, a, 1);
  }
  hipLaunchKernelGGL((k_moe_gateup<KIND, TB>), dim3(gu_items < 4096 ? gu_items : 4096), dim3(256),
                     xl_gu, s, a, split ? 2 : 0);
  // prompt-block down: four-wave workgroups (two fit a CU at this register
  // count; eight-wave ones, one per CU, measured 20% slower)
  if (hot) hipLaunchKernelGGL((k_moe_hot_dn<KIND>), dim3(256), dim3(512), 0, s, a);
  constexpr int kDnWaves = 4;
  const int dn_items = nb_r * (rows / (kDnWaves / ks_r)) + nb_s * (rows / (kDnWaves / ks_s));
  if (split) {
    const int dn1 = nb_r * (rows / (kDnWaves / ks_r));
    hipLaunchKernelGGL((k_moe_down<KIND, 1, kDnWaves>), dim3(dn1 < 4096 ? dn1 : 4096), dim3(64 * kDnWaves),
                       kMoeRecDown * ((a.De > a.Ds ? a.De : a.Ds) / 256), s, a, ks_r, ks_s, 1);
  }
  hipLaunchKernelGGL((k_moe_down<KIND, TB, kDnWaves>), dim3(dn_items < 4096 ? dn_items : 4096), dim3(64 * kDnWaves),
                     xl_dn, s, a, ks_r, ks_s, split ? 2 : 0);
  hipLaunchKernelGGL(k_moe_combine, dim3((a.D + 255) / 256, a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_moe(int kind, const MoeArgs& a, hipStream_t s) {
  if (kind == KIND_Q4_1) return a.tb == 1 ? moe_run<KIND_Q4_1, 1>(a, s) : moe_run<KIND_Q4_1, 4>(a, s);
  if (kind == KIND_Q4_K) return a.tb == 1 ? moe_run<KIND_Q4_K, 1>(a, s) : moe_run<KIND_Q4_K, 4>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace q4nx
