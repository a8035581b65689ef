// Device-side arguments of the MoE kernels (one struct, passed by value).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4nx {

constexpr int kMoeMaxPairs = 4096;   // T * k per call (the route kernel sorts them in LDS)
constexpr int kMoeMaxK = 16;         // picks per token
constexpr int kMoeBatchInts = 12;    // ints per routed-batch record (batches of at most 4 tokens)
constexpr int kMoeHotInts = 8;       // ints per matrix-core unit record
constexpr int kMoeHotTokens = 64;    // token rows of one matrix-core work item

struct MoeArgs {
  // routed experts: expert e's chunks at base + e * stride
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  int64_t gate_stride, up_stride, down_stride;
  // shared expert (Ds == 0: none)
  const uint8_t* sgate;
  const uint8_t* sup;
  const uint8_t* sdown;
  int32_t n_experts, D, De, Ds;
  // inputs / outputs
  const uint16_t* X;
  const int32_t* ids;
  const float* p;
  float* Y;
  int32_t T, k;
  int32_t tb;        // tokens per work item (1 or 4)
  int32_t hstride;   // row stride of hbuf, max(De, Ds)
  int32_t hot_min;   // segments of at least this many pairs (and the shared expert when
                     // T >= hot_min) run on the matrix cores; 0: never
  // optional stage outputs
  float* dbg_h;
  float* dbg_d;
  float* dbg_h_shared;
  float* dbg_d_shared;
  // workspace
  uint32_t* hdr;     // [0] error word, [1] segments, [2] routed batches, [3] matrix-core
                     // units, [4] and [5] their gate/up and down work items
  int32_t* sorted;   // [P] pair index at each sorted position
  int32_t* seg;      // [P][3] (expert, first sorted position, count)
  int32_t* batch0;   // [P + 1] first routed batch of each segment
  int32_t* btab;     // [P][kMoeBatchInts] per routed batch: expert, first sorted position,
                     // tokens, -, then its tokens' ids and pair indices (4 each)
  int32_t* hot;      // [units][kMoeHotInts] matrix-core units: expert (-1: shared), first
                     // sorted position, pairs, first gate/up item, first down item
  float* hbuf;       // [P + T][hstride] fp32 h (routed by sorted position, shared at P + t)
  float* dbuf;       // [P + T][D] fp32 d (routed by pair index, shared at P + t)
};

// Workspace layout for P pairs and T tokens; returns the total bytes and fills
// the offsets (each 256-byte aligned).
struct MoeWsLayout {
  size_t hdr, sorted, seg, batch0, btab, hot, hbuf, dbuf, total;
};

inline MoeWsLayout moe_ws_layout(int P, int T, int D, int hstride) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  MoeWsLayout l;
  size_t o = 0;
  l.hdr = o;    o = up(o + 256);
  l.sorted = o; o = up(o + (size_t)P * 4);
  l.seg = o;    o = up(o + (size_t)P * 12);
  l.batch0 = o; o = up(o + (size_t)(P + 1) * 4);
  l.btab = o;   o = up(o + (size_t)P * kMoeBatchInts * 4);
  l.hot = o;    o = up(o + (size_t)(P + 1) * kMoeHotInts * 4);
  l.hbuf = o;   o = up(o + (size_t)(P + T) * hstride * 4);
  l.dbuf = o;   o = up(o + (size_t)(P + T) * D * 4);
  l.total = o;
  return l;
}

// Prepared-record bytes per (token, tile column) in LDS: fp16 records of the
// bf16 activations (gate/up) or of the fp32 h (down), 8 groups x 72 B.
constexpr int kMoeRecGateUp = 8 * 72;
constexpr int kMoeRecDown = 8 * 72;

hipError_t launch_moe(int kind, const MoeArgs& a, hipStream_t s);

}  // namespace q4nx
