// C ABI of libq4nx.so (declared in include/q4nx.h): host-side checks, then
// launches.  Every check runs before anything is enqueued, and no check
// touches the device, so the error paths can be exercised without a GPU.
//
// Check rules for a weight follow the 1bit engine docs, page "NPU engine"
// (section "Q4NX chunks": the chunk size names the kind, the two Q8 layouts
// cannot be told apart; section "From a GGUF": a checker refuses an unknown
// chunk size or a tensor shorter than its layout needs).
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <queue>
#include <tuple>
#include <string>
#include <vector>

#include "../../include/q4nx.h"
#include "gemm_args.h"
#include "moe_args.h"
#include "plan_args.h"
#include "q4nx_dev.h"
#include "topk.h"

static_assert(Q4NX_GEMM_BATCH_MAX_JOBS == q4nx::kGemmMaxJobs, "GEMM job table size");

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(q4nx_status_str(status)) + ": " + buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return Q4NX_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(Q4NX_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int kind_of(const q4nx_weight* w) {
  switch (w->chunk_bytes) {
    case Q4NX_Q4_1_BYTES: return q4nx::KIND_Q4_1;
    case Q4NX_Q4_K_BYTES: return q4nx::KIND_Q4_K;
    default: return w->q8_layout == Q4NX_Q8_LAYOUT_A ? q4nx::KIND_Q8_A : q4nx::KIND_Q8_B;
  }
}

int check_weight(const q4nx_weight* w, const char* name) {
  if (!w) return fail(Q4NX_E_ARG, "%s: null descriptor", name);
  if (!w->chunks) return fail(Q4NX_E_ARG, "%s: null chunk pointer", name);
  const int cb = w->chunk_bytes;
  if (cb != Q4NX_Q4_1_BYTES && cb != Q4NX_Q4_K_BYTES && cb != Q4NX_Q8_BYTES)
    return fail(Q4NX_E_CHUNK_KIND, "%s: unknown chunk size %d (5120 q4_1, 4736 Q4_K, 8704 Q8)",
                name, cb);
  if (cb == Q4NX_Q8_BYTES && w->q8_layout != Q4NX_Q8_LAYOUT_A && w->q8_layout != Q4NX_Q8_LAYOUT_B)
    return fail(Q4NX_E_Q8_LAYOUT, "%s: Q8 weight needs its code layout (A or B); it cannot be "
                "detected from the data", name);
  if (w->rows <= 0 || w->rows % 32 || w->cols <= 0 || w->cols % 256)
    return fail(Q4NX_E_SHAPE, "%s: %d x %d is not a whole number of 32 x 256 tiles", name,
                w->rows, w->cols);
  const int64_t need = (int64_t)(w->rows / 32) * (w->cols / 256) * cb;
  if (w->nbytes < need)
    return fail(Q4NX_E_SHORT, "%s: %lld bytes given, the %d x %d grid needs %lld", name,
                (long long)w->nbytes, w->rows, w->cols, (long long)need);
  if (!aligned(w->chunks, 16)) return fail(Q4NX_E_ALIGN, "%s: chunks not 16-byte aligned", name);
  return Q4NX_OK;
}

// Launch shape of a batch.  Many tile rows: 4-wave workgroups, waves per tile
// row chosen so the launch has about 2048 waves; each wave streams a run of
// chunks.  Few tile rows of long K (more than 16 tile columns): the launch is
// latency-bound on each wave's run of chunks, so 16-wave workgroups spread a
// tile row over enough waves that every wave holds about two chunks.  (Measured
// on the decode shapes: this halves the time of a 2560 x 9728 GEMV and slows
// the K = 2560 and K = 4096 ones, which keep 4-wave workgroups.)
#ifndef Q4NX_SMALL_ROWS
#define Q4NX_SMALL_ROWS 1024
#endif
#ifndef Q4NX_MKS_SHIFT
#define Q4NX_MKS_SHIFT 2
#endif
#ifndef Q4NX_SMALL_CPW
#define Q4NX_SMALL_CPW 2
#endif

int pow2_at_least(int v, int cap) {
  int p = 1;
  while (p < v && p < cap) p <<= 1;
  return p;
}

#ifndef Q4NX_SMALL_MIN_TC
#define Q4NX_SMALL_MIN_TC 17
#endif

// Launches of at most Q4NX_ROWSPLIT_TR tile rows (q4 kinds, prepared
// activations) split each tile's rows into two units of 16, and of at most
// Q4NX_ROWSPLIT4_TR into four units of 8, so they reach more CUs.
#ifndef Q4NX_ROWSPLIT_TR
#define Q4NX_ROWSPLIT_TR 1024
#endif
#ifndef Q4NX_ROWSPLIT4_TR
#define Q4NX_ROWSPLIT4_TR 0
#endif

// Three or four activation rows (q4 kinds): 4-wave workgroups hold their
// 168-235 registers three or two to a CU, so a launch of long K (at least
// Q4NX_MID_MIN_TC tile columns) or of few tile rows (at most Q4NX_MID_MAX_TR)
// would leave a wave alone on its SIMD with a long run of chunks; 8-wave
// workgroups split K eight ways instead.
#ifndef Q4NX_MID_MIN_TC
#define Q4NX_MID_MIN_TC 17
#endif
#ifndef Q4NX_MID_MAX_TR
#define Q4NX_MID_MAX_TR 0
#endif

int pick_waves(int kind, int64_t total_tr, int M, int max_tc) {
  const bool q4 = kind == q4nx::KIND_Q4_1 || kind == q4nx::KIND_Q4_K;
  if (q4 && (M == 3 || M == 4) && (max_tc >= Q4NX_MID_MIN_TC || total_tr <= Q4NX_MID_MAX_TR)) return 8;
  return (total_tr >= Q4NX_SMALL_ROWS || M > 2 || max_tc < Q4NX_SMALL_MIN_TC) ? 4 : 16;
}

int pick_ks(int waves, int64_t total_tr, int TC, bool mfma = false) {
  if (waves == 16) return pow2_at_least((TC + Q4NX_SMALL_CPW - 1) / Q4NX_SMALL_CPW, 16);
  if (waves == 8) return pow2_at_least((TC + Q4NX_SMALL_CPW - 1) / Q4NX_SMALL_CPW, 8);
  // the matrix-core kernel stages M >= 3 rows of records per workgroup, so
  // it takes fewer, longer workgroups
  if (mfma) total_tr <<= Q4NX_MKS_SHIFT;
  int ks = total_tr >= 2048 ? 1 : (total_tr >= 1024 ? 2 : 4);
  const int lim = TC >= 4 ? 4 : (TC >= 2 ? 2 : 1);
  return ks < lim ? ks : lim;
}

// Launch shape of one kind's jobs (all valid, same M) in one launch.
struct BatchShape {
  int waves, xl, parts;   // parts: units per tile row
  bool mfma;              // k_gemv_q4m (q4 kinds, prepared records, M >= kGemvMfmaMinM)
};

BatchShape batch_shape(int kind, int64_t total_tr, int max_tc, int M) {
  BatchShape sh;
  sh.waves = pick_waves(kind, total_tr, M, max_tc);
  sh.xl = q4nx::gemv_xl_bytes(kind, M, sh.waves, max_tc);
  if (sh.waves == 8 && sh.xl <= 0) {   // the 8-wave kernel stages its activations in LDS
    sh.waves = 4;
    sh.xl = q4nx::gemv_xl_bytes(kind, M, 4, max_tc);
  }
  const bool q4 = kind == q4nx::KIND_Q4_1 || kind == q4nx::KIND_Q4_K;
  sh.parts = !(q4 && sh.xl > 0) ? 1 : total_tr <= Q4NX_ROWSPLIT4_TR ? 4 : total_tr <= Q4NX_ROWSPLIT_TR ? 2 : 1;
  sh.mfma = q4 && sh.xl > 0 && M >= q4nx::kGemvMfmaMinM;
  return sh;
}

// Fills the kernel's job record of j, its workgroups starting at wg_begin;
// returns its workgroup count.
int fill_job(q4nx::GemvJob& g, const q4nx_gemv_job* j, const BatchShape& sh, int64_t total_tr, int wg_begin) {
  g.w = static_cast<const uint8_t*>(j->w.chunks);
  g.x = j->x;
  g.y = j->y;
  g.TR = j->w.rows / 32;
  g.TC = j->w.cols / 256;
  g.ldx = j->w.cols;
  g.ldy = j->w.rows;
  g.ks = pick_ks(sh.waves, total_tr, g.TC, sh.mfma);
  g.wg_begin = wg_begin;
  const int rpw = sh.waves / g.ks;
  return (g.TR * sh.parts + rpw - 1) / rpw;
}

// Launch one kind's jobs (all valid, same M) in as few launches as the job
// table allows.
int run_batch(int kind, const q4nx_gemv_job* const* jobs, int n, int M, hipStream_t s) {
  int64_t total_tr = 0;
  int max_tc = 0;
  for (int i = 0; i < n; ++i) {
    total_tr += jobs[i]->w.rows / 32;
    max_tc = std::max(max_tc, jobs[i]->w.cols / 256);
  }
  const BatchShape sh = batch_shape(kind, total_tr, max_tc, M);
  // q4 kinds at M = 5..8 whose records do not fit in LDS (long K): two passes
  // of 4 rows through the matrix-core kernel, rows 0..3 and then M-4..M-1,
  // instead of the kernel that loads activations per chunk.  Each pass reads
  // the weights once; a row computed by both comes out with the same bits
  // both times (same kernel, shape and K split), so the second write changes
  // nothing and a row's bits do not depend on its slot.
  const bool q4 = kind == q4nx::KIND_Q4_1 || kind == q4nx::KIND_Q4_K;
  if (q4 && M > 4 && sh.xl <= 0 && q4nx::gemv_xl_bytes(kind, 4, 4, max_tc) > 0) {
    std::vector<q4nx_gemv_job> part(n);
    std::vector<const q4nx_gemv_job*> ptr(n);
    for (int m0 : {0, M - 4}) {
      for (int i = 0; i < n; ++i) {
        part[i] = *jobs[i];
        part[i].x = jobs[i]->x + (size_t)m0 * jobs[i]->w.cols;
        part[i].y = jobs[i]->y + (size_t)m0 * jobs[i]->w.rows;
        ptr[i] = &part[i];
      }
      const int st = run_batch(kind, ptr.data(), n, 4, s);
      if (st != Q4NX_OK) return st;
    }
    return Q4NX_OK;
  }
  for (int i0 = 0; i0 < n; i0 += q4nx::kMaxBatch) {
    const int cnt = n - i0 < q4nx::kMaxBatch ? n - i0 : q4nx::kMaxBatch;
    q4nx::GemvBatch b;
    memset(&b, 0, sizeof b);
    b.sl = 4 / sh.parts;
    int wg = 0;
    for (int t = 0; t < cnt; ++t) wg += fill_job(b.job[t], jobs[i0 + t], sh, total_tr, wg);
    b.n_jobs = cnt;
    const hipError_t e = q4nx::launch_gemv(kind, M, sh.waves, b, wg, sh.xl, s);
    if (e != hipSuccess) return hip_status(e, "gemv launch");
  }
  return Q4NX_OK;
}

// Launch shape of the top-k GEMV (one job, 4-wave workgroups, the rules of
// run_batch otherwise).  Returns false when the shape does not fit it.
struct TopkShape {
  q4nx::GemvBatch b;
  int n_wg, xl;
  size_t ws_bytes;
};

constexpr size_t kTopkCntBytes = 256;   // n_grp + 1 <= 65 counters

bool topk_shape(const q4nx_weight* w, int M, int k, TopkShape& t) {
  const int kind = kind_of(w);
  const int TR = w->rows / 32, TC = w->cols / 256;
  t.xl = q4nx::gemv_xl_bytes(kind, M, 4, TC);
  if (t.xl <= 0) return false;
  const bool q4 = kind == q4nx::KIND_Q4_1 || kind == q4nx::KIND_Q4_K;
  const int parts = !q4 ? 1 : TR <= Q4NX_ROWSPLIT4_TR ? 4 : TR <= Q4NX_ROWSPLIT_TR ? 2 : 1;
  memset(&t.b, 0, sizeof t.b);
  t.b.sl = 4 / parts;
  q4nx::GemvJob& g = t.b.job[0];
  g.w = static_cast<const uint8_t*>(w->chunks);
  g.TR = TR;
  g.TC = TC;
  g.ldx = w->cols;
  g.ldy = w->rows;
  // the K split q4nx_gemv takes for this weight and M (so the logits agree bit for bit)
  g.ks = pick_ks(4, TR, TC, q4 && M >= q4nx::kGemvMfmaMinM);
  g.wg_begin = 0;
  t.b.n_jobs = 1;
  const int rpw = 4 / g.ks;
  t.n_wg = (TR * parts + rpw - 1) / rpw;
  if (t.n_wg > q4nx::kTopkMaxWg) return false;
  t.b.tk.k = k;
  t.b.tk.n_wg = t.n_wg;
  t.b.tk.n_grp = (t.n_wg + q4nx::kTopkGroup - 1) / q4nx::kTopkGroup;
  t.ws_bytes = kTopkCntBytes + (size_t)(t.n_wg + t.b.tk.n_grp) * M * k * 8;
  return true;
}

int check_gemv_io(const q4nx_weight* w, const void* x, const float* y, int M, const char* name) {
  int st = check_weight(w, name);
  if (st) return st;
  if (!x || !y) return fail(Q4NX_E_ARG, "%s: null x or y", name);
  if (M < 1 || M > Q4NX_GEMV_MAX_M)
    return fail(Q4NX_E_ARG, "%s: M = %d outside 1..%d", name, M, (int)Q4NX_GEMV_MAX_M);
  if (!aligned(x, 16)) return fail(Q4NX_E_ALIGN, "%s: x not 16-byte aligned", name);
  if (!aligned(y, 4)) return fail(Q4NX_E_ALIGN, "%s: y not 4-byte aligned", name);
  return Q4NX_OK;
}

}  // namespace

extern "C" {

const char* q4nx_status_str(int status) {
  switch (status) {
    case Q4NX_OK: return "ok";
    case Q4NX_E_ARG: return "invalid argument";
    case Q4NX_E_CHUNK_KIND: return "unknown or unsupported chunk kind";
    case Q4NX_E_SHAPE: return "bad shape";
    case Q4NX_E_SHORT: return "tensor shorter than its layout needs";
    case Q4NX_E_ALIGN: return "misaligned pointer";
    case Q4NX_E_WORKSPACE: return "workspace missing or too small";
    case Q4NX_E_Q8_LAYOUT: return "Q8 code layout not given";
    case Q4NX_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* q4nx_last_error(void) { return g_last_error.c_str(); }

int q4nx_version(void) { return 100; }

int q4nx_weight_check(const q4nx_weight* w) {
  const int st = check_weight(w, "weight");
  return st ? st : ok();
}

int q4nx_gemv(const q4nx_weight* w, const uint16_t* x, float* y, int M, void* stream) {
  const int st = check_gemv_io(w, x, y, M, "gemv");
  if (st) return st;
  q4nx_gemv_job j{*w, x, y};
  const q4nx_gemv_job* pj = &j;
  const int r = run_batch(kind_of(w), &pj, 1, M, static_cast<hipStream_t>(stream));
  return r ? r : ok();
}

int q4nx_gemv_batched(const q4nx_gemv_job* jobs, int n_jobs, int M, void* stream) {
  if (!jobs) return fail(Q4NX_E_ARG, "gemv_batched: null job array");
  if (n_jobs < 1 || n_jobs > Q4NX_BATCH_MAX_JOBS)
    return fail(Q4NX_E_ARG, "gemv_batched: %d jobs outside 1..%d", n_jobs,
                (int)Q4NX_BATCH_MAX_JOBS);
  for (int i = 0; i < n_jobs; ++i) {
    char name[48];
    snprintf(name, sizeof name, "gemv_batched job %d", i);
    const int st = check_gemv_io(&jobs[i].w, jobs[i].x, jobs[i].y, M, name);
    if (st) return st;
  }
  const q4nx_gemv_job* by_kind[4][Q4NX_BATCH_MAX_JOBS];
  int cnt[4] = {0, 0, 0, 0};
  for (int i = 0; i < n_jobs; ++i) {
    const int k = kind_of(&jobs[i].w);
    by_kind[k][cnt[k]++] = &jobs[i];
  }
  for (int k = 0; k < 4; ++k) {
    if (!cnt[k]) continue;
    const int r = run_batch(k, by_kind[k], cnt[k], M, static_cast<hipStream_t>(stream));
    if (r) return r;
  }
  return ok();
}

size_t q4nx_gemv_topk_ws(const q4nx_weight* w, int M, int k) {
  TopkShape t;
  if (check_weight(w, "gemv_topk_ws") || M < 1 || M > 4 || k < 1 || k > q4nx::kTopkMax ||
      !topk_shape(w, M, k, t))
    return 0;
  return t.ws_bytes;
}

int q4nx_gemv_topk(const q4nx_weight* w, const uint16_t* x, int M, int k, float* y, int32_t* ids,
                   float* vals, void* ws, size_t ws_bytes, void* stream) {
  int st = check_weight(w, "gemv_topk");
  if (st) return st;
  if (!x || !ids) return fail(Q4NX_E_ARG, "gemv_topk: null x or ids");
  if (M < 1 || M > 4) return fail(Q4NX_E_ARG, "gemv_topk: M = %d outside 1..4", M);
  if (k < 1 || k > q4nx::kTopkMax || k > w->rows)
    return fail(Q4NX_E_ARG, "gemv_topk: k = %d outside 1..min(%d, rows)", k, q4nx::kTopkMax);
  if (!aligned(x, 16)) return fail(Q4NX_E_ALIGN, "gemv_topk: x not 16-byte aligned");
  if ((y && !aligned(y, 4)) || !aligned(ids, 4) || (vals && !aligned(vals, 4)))
    return fail(Q4NX_E_ALIGN, "gemv_topk: y, ids and vals must be 4-byte aligned");
  TopkShape t;
  if (!topk_shape(w, M, k, t))
    return fail(Q4NX_E_SHAPE, "gemv_topk: %d x %d at M = %d does not fit the prepared-activation GEMV "
                "with at most %d workgroups", w->rows, w->cols, M, q4nx::kTopkMaxWg);
  if (!ws || ws_bytes < t.ws_bytes)
    return fail(Q4NX_E_WORKSPACE, "gemv_topk: workspace of %zu bytes, %zu needed", ws_bytes, t.ws_bytes);
  if (!aligned(ws, 256)) return fail(Q4NX_E_ALIGN, "gemv_topk: workspace not 256-byte aligned");
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  t.b.job[0].x = x;
  t.b.job[0].y = y;
  t.b.tk.cnt = reinterpret_cast<uint32_t*>(wsb);
  t.b.tk.cand = reinterpret_cast<uint64_t*>(wsb + kTopkCntBytes);
  t.b.tk.ids = ids;
  t.b.tk.vals = vals;
  const hipError_t e = q4nx::launch_gemv_topk(kind_of(w), M, t.b, t.n_wg, t.xl, static_cast<hipStream_t>(stream));
  return hip_status(e, "gemv_topk launch");
}

}  // extern "C"

namespace {

// q4nx_gemm_exchange_mode: 0 default, 1 odd groups act displaced, 2 device-coherent exchange.
std::atomic<int> g_gemm_exchange_mode{0};

// Checks a block-GEMM launch over weights w[0..n-1] sharing X and fills the
// kernel arguments (all but the workspace).  Returns a status.
int gemm_setup(const q4nx_weight* const* w, float* const* Y, int n, const uint16_t* X, int M,
               const char* name, q4nx::GemmArgs& a) {
  if (n < 1 || n > q4nx::kGemmMaxJobs)
    return fail(Q4NX_E_ARG, "%s: %d weights outside 1..%d", name, n, q4nx::kGemmMaxJobs);
  for (int i = 0; i < n; ++i) {
    const int st = check_weight(w[i], name);
    if (st) return st;
    if (w[i]->chunk_bytes == Q4NX_Q8_BYTES)
      return fail(Q4NX_E_CHUNK_KIND, "%s: Q8 weights are not supported by the block GEMM", name);
    if (kind_of(w[i]) != kind_of(w[0]) || w[i]->cols != w[0]->cols)
      return fail(Q4NX_E_SHAPE, "%s: weight %d differs from weight 0 in chunk kind or columns", name, i);
    if (!Y[i]) return fail(Q4NX_E_ARG, "%s: null Y of weight %d", name, i);
    if (!aligned(Y[i], 4)) return fail(Q4NX_E_ALIGN, "%s: Y of weight %d not 4-byte aligned", name, i);
  }
  if (!X) return fail(Q4NX_E_ARG, "%s: null X", name);
  if (M < 1 || M > Q4NX_GEMM_MAX_M)
    return fail(Q4NX_E_ARG, "%s: M = %d outside 1..%d", name, M, (int)Q4NX_GEMM_MAX_M);
  if (!aligned(X, 16)) return fail(Q4NX_E_ALIGN, "%s: X not 16-byte aligned", name);
  a = q4nx::GemmArgs{};
  int nb = 0;
  for (int i = 0; i < n; ++i) {
    a.job[i].w = static_cast<const uint8_t*>(w[i]->chunks);
    a.job[i].Y = Y[i];
    a.job[i].TR = (int32_t)(w[i]->rows / 32);
    a.job[i].nb0 = nb;
    nb += q4nx::gemm_blocks(a.job[i].TR, M);
  }
  a.n_jobs = n;
  a.X = X;
  a.TC = (int32_t)(w[0]->cols / 256);
  a.M = M;
  a.NB = nb;
  a.S = q4nx::gemm_parts(nb, a.TC);
  return Q4NX_OK;
}

int gemm_launch(q4nx::GemmArgs& a, int kind, void* ws, size_t ws_bytes, void* stream,
                const char* name, bool may_probe = true) {
  const size_t need = q4nx::gemm_ws_bytes(a.NB, a.TC, a.M);
  if (need && (!ws || ws_bytes < need))
    return fail(Q4NX_E_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", name, ws_bytes, need);
  if (need && !aligned(ws, 256)) return fail(Q4NX_E_ALIGN, "%s: workspace not 256-byte aligned", name);
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.cnt = need ? reinterpret_cast<uint32_t*>(w) : nullptr;
  a.claim = need ? reinterpret_cast<uint32_t*>(w + q4nx::kGemmClaimOff) : nullptr;
  a.rescued = need ? reinterpret_cast<uint32_t*>(w + q4nx::kGemmRescueOff) : nullptr;
  a.diag = need ? reinterpret_cast<uint32_t*>(w + q4nx::kGemmDiagOff) : nullptr;
  a.partial = need ? reinterpret_cast<float*>(w + q4nx::kGemmCntBytes) : nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int mode = g_gemm_exchange_mode.load(std::memory_order_relaxed);
  a.test_mode = mode == 1 ? 1 : 0;
  const bool local = a.S > 1 && mode != 2 &&
                     (may_probe ? q4nx::xcd_round_robin(st) : q4nx::xcd_round_robin_known()) == 1;
  const hipError_t e = q4nx::launch_gemm(kind, a, local, st);
  return hip_status(e, name);
}

}  // namespace

extern "C" {

int q4nx_gemm_block(const q4nx_weight* w, const uint16_t* X, float* Y, int M, void* ws,
                    size_t ws_bytes, void* stream) {
  q4nx::GemmArgs a;
  const int st = gemm_setup(&w, &Y, 1, X, M, "gemm_block", a);
  if (st) return st;
  const int r = gemm_launch(a, kind_of(w), ws, ws_bytes, stream, "gemm_block");
  return r ? r : ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// the allocation-free block GEMM
// ---------------------------------------------------------------------------
// Its workspace is `scratch`, in the code object: every GPU the library runs
// on holds one until the process ends.  Each call clears the header words
// that must start at zero (arrival counters, claim words, rescue flags) with a
// small kernel on the caller's stream before the GEMM; the partial tiles are
// written before they are read.  Calls that overlap on one GPU share the array
// and race.  Host code never passes the array's name to a kernel: its device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
constexpr size_t kNoAllocGemmBytes = q4nx::kGemmCntBytes + ((size_t)16 << 20);
static_assert(kNoAllocGemmBytes >= q4nx::kGemmCntBytes + (size_t)Q4NX_GEMM_WG_TARGET * 64 *
                                       q4nx::kGemmRowsPerWg * 32 * 4,
              "scratch holds the largest split any call makes (workgroup rows x parts <= the target)");

static __device__ __align__(256) uint8_t scratch[kNoAllocGemmBytes];

namespace {

constexpr int kHeaderZeroWords = (int)(q4nx::kGemmDiagOff / 4);

__global__ void __launch_bounds__(256) k_clear_words(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}

std::once_flag g_scratch_once[64];
void* g_scratch_ptr[64];
hipError_t g_scratch_err[64];

int scratch_address(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "gemm_block_noalloc: current device");
  if (dev < 0 || dev >= 64) return fail(Q4NX_E_HIP, "gemm_block_noalloc: device %d beyond 63", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_status(g_scratch_err[dev], "gemm_block_noalloc: scratch address");
  if (!g_scratch_ptr[dev]) return fail(Q4NX_E_HIP, "gemm_block_noalloc: scratch address is null");
  *out = g_scratch_ptr[dev];
  return Q4NX_OK;
}

}  // namespace

extern "C" {

size_t q4nx_gemm_block_noalloc_max(void) { return kNoAllocGemmBytes; }

int q4nx_gemm_block_noalloc(const q4nx_weight* w, const uint16_t* X, float* Y, int M, void* stream) {
  q4nx::GemmArgs a;
  const int st = gemm_setup(&w, &Y, 1, X, M, "gemm_block_noalloc", a);
  if (st) return st;
  const size_t need = q4nx::gemm_ws_bytes(a.NB, a.TC, a.M);
  if (need > kNoAllocGemmBytes)
    return fail(Q4NX_E_WORKSPACE, "gemm_block_noalloc: this call needs %zu bytes of scratch, the static "
                "array holds %zu", need, kNoAllocGemmBytes);
  void* ws = nullptr;
  if (need) {
    const int s2 = scratch_address(&ws);
    if (s2) return s2;
    k_clear_words<<<1, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<uint32_t*>(ws), kHeaderZeroWords);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "gemm_block_noalloc: clearing the scratch header");
  }
  const int r = gemm_launch(a, kind_of(w), ws, need, stream, "gemm_block_noalloc", false);
  return r ? r : ok();
}

size_t q4nx_gemm_block_ws(const q4nx_weight* w) {
  if (check_weight(w, "gemm_block_ws")) return 0;
  const int TR = (int)(w->rows / 32);
  return q4nx::gemm_ws_bytes_any_m(&TR, 1, (int)(w->cols / 256));
}

int q4nx_gemm_batched(const q4nx_gemm_job* jobs, int n_jobs, const uint16_t* X, int M, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!jobs) return fail(Q4NX_E_ARG, "gemm_batched: null job array");
  if (n_jobs < 1 || n_jobs > Q4NX_GEMM_BATCH_MAX_JOBS)
    return fail(Q4NX_E_ARG, "gemm_batched: %d jobs outside 1..%d", n_jobs, (int)Q4NX_GEMM_BATCH_MAX_JOBS);
  const q4nx_weight* w[Q4NX_GEMM_BATCH_MAX_JOBS];
  float* Y[Q4NX_GEMM_BATCH_MAX_JOBS];
  for (int i = 0; i < n_jobs; ++i) {
    w[i] = &jobs[i].w;
    Y[i] = jobs[i].Y;
  }
  q4nx::GemmArgs a;
  const int st = gemm_setup(w, Y, n_jobs, X, M, "gemm_batched", a);
  if (st) return st;
  const int r = gemm_launch(a, kind_of(w[0]), ws, ws_bytes, stream, "gemm_batched");
  return r ? r : ok();
}

int q4nx_gemm_exchange_mode(int mode) {
  if (mode < 0 || mode > 2) return fail(Q4NX_E_ARG, "gemm_exchange_mode: %d is not 0, 1 or 2", mode);
  g_gemm_exchange_mode.store(mode, std::memory_order_relaxed);
  return ok();
}

size_t q4nx_gemm_batched_ws(const q4nx_gemm_job* jobs, int n_jobs) {
  if (!jobs || n_jobs < 1 || n_jobs > Q4NX_GEMM_BATCH_MAX_JOBS) {
    fail(Q4NX_E_ARG, "gemm_batched_ws: bad job array");
    return 0;
  }
  int TR[Q4NX_GEMM_BATCH_MAX_JOBS];
  for (int i = 0; i < n_jobs; ++i) {
    if (check_weight(&jobs[i].w, "gemm_batched_ws")) return 0;
    TR[i] = (int)(jobs[i].w.rows / 32);
  }
  return q4nx::gemm_ws_bytes_any_m(TR, n_jobs, (int)(jobs[0].w.cols / 256));
}

// ---------------------------------------------------------------------------
// plans
// ---------------------------------------------------------------------------
}  // extern "C"

struct q4nx_plan_s {
  struct Seg {
    int kind, grid;
    bool step = false;   // the step kernel (static schedule) instead of the unit-dealing one
    size_t lds = 0;
    q4nx::PlanArgs args;
    q4nx::StepArgs sargs;
  };
  int M = 1;
  int mode = 0;          // 0: one GEMV launch per phase; 1: one persistent launch per segment
  std::vector<Seg> segs;
  struct Phase {         // mode 0: one batched GEMV launch over a device job table
    int kind, waves, xl, n_wg;
    q4nx::GemvBatch b;
  };
  std::vector<Phase> phases;
  void* dev = nullptr;
  size_t bytes = 0;
  std::vector<uint32_t*> ctl;   // per segment control words (device)
};

namespace {

constexpr int kPlanSpinLimit = 1 << 22;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

int q4nx_plan_create(const q4nx_gemv_job* jobs, const int32_t* phase, int n_jobs, int M,
                     q4nx_plan* out) {
  if (!jobs || !phase || !out) return fail(Q4NX_E_ARG, "plan: null jobs, phase or out");
  *out = nullptr;
  if (n_jobs < 1 || n_jobs > 65536)
    return fail(Q4NX_E_ARG, "plan: %d jobs outside 1..65536", n_jobs);
  if (M < 1 || M > 4) return fail(Q4NX_E_ARG, "plan: M = %d outside 1..4", M);
  for (int i = 0; i < n_jobs; ++i) {
    char name[40];
    snprintf(name, sizeof name, "plan job %d", i);
    const int st = check_gemv_io(&jobs[i].w, jobs[i].x, jobs[i].y, M, name);
    if (st) return st;
    if (phase[i] < 0) return fail(Q4NX_E_ARG, "plan job %d: negative phase", i);
  }
  std::vector<int> order(n_jobs);
  for (int i = 0; i < n_jobs; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return phase[a] < phase[b]; });
  // segments: maximal runs of phases whose jobs share one kind
  struct SegH {
    int kind;
    std::vector<int> jobs;
    std::vector<int> phase_of;   // local phase of each job
    int n_phases;
  };
  std::vector<SegH> segs;
  for (size_t t = 0; t < order.size();) {
    const int ph = phase[order[t]];
    const int kind = kind_of(&jobs[order[t]].w);
    size_t e = t;
    while (e < order.size() && phase[order[e]] == ph) {
      if (kind_of(&jobs[order[e]].w) != kind)
        return fail(Q4NX_E_CHUNK_KIND, "plan: phase %d mixes chunk kinds", ph);
      ++e;
    }
    if (segs.empty() || segs.back().kind != kind) segs.push_back({kind, {}, {}, 0});
    SegH& sg = segs.back();
    for (size_t i = t; i < e; ++i) {
      sg.jobs.push_back(order[i]);
      sg.phase_of.push_back(sg.n_phases);
    }
    ++sg.n_phases;
    t = e;
  }
  int n_cu = 0;
  {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_status(e, "plan device query");
  }
  // q4 segments whose activations fit the step kernel's LDS run on it
  struct StepT {
    bool use = false;
    size_t lds = 0, rec = 0;
    int ns = 0;
    std::vector<q4nx::StepJob> sj;
    std::vector<q4nx::StepUnit> units;
    std::vector<int32_t> first;
    size_t o_jobs = 0, o_units = 0, o_first = 0, o_sync = 0, o_ctl = 0;
  };
  std::vector<StepT> steps(segs.size());
  for (size_t si = 0; si < segs.size(); ++si) {
    SegH& sg = segs[si];
    if (sg.kind != q4nx::KIND_Q4_1 && sg.kind != q4nx::KIND_Q4_K) continue;
    int max_tc = 0;
    for (int ji : sg.jobs) max_tc = std::max(max_tc, (int)(jobs[ji].w.cols / 256));
    const q4nx::StepLds lds = q4nx::step_lds(M, max_tc);
    if (lds.ns < 2) continue;
    StepT& S = steps[si];
    S.use = true;
    S.lds = lds.total;
    S.rec = lds.rec;
    S.ns = lds.ns;
    for (int ji : sg.jobs) {
      const q4nx_gemv_job& j = jobs[ji];
      S.sj.push_back({static_cast<const uint8_t*>(j.w.chunks), j.x, j.y, (int32_t)(j.w.rows / 32),
                      (int32_t)(j.w.cols / 256), (int32_t)j.w.cols, (int32_t)j.w.rows});
    }
    // whole tile rows to workgroups, largest first, each to the least loaded in
    // its phase (then overall); a workgroup's rows in (job, row) order, cut into
    // pieces of at most kStepPieceCols chunk columns
    const int cap = q4nx::kStepPieceCols;
    std::vector<std::vector<q4nx::StepUnit>> per(n_cu);
    std::vector<long long> total(n_cu, 0);
    for (int ph = 0; ph < sg.n_phases; ++ph) {
      struct Row { int cost, job, tr; };
      std::vector<Row> rows;
      for (size_t i = 0; i < sg.jobs.size(); ++i)
        if (sg.phase_of[i] == ph)
          for (int tr = 0; tr < S.sj[i].TR; ++tr) rows.push_back({S.sj[i].TC, (int)i, tr});
      std::stable_sort(rows.begin(), rows.end(), [](const Row& a, const Row& b) { return a.cost > b.cost; });
      typedef std::tuple<long long, long long, int> Key;
      std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
      for (int b = 0; b < n_cu; ++b) heap.push(Key(0, total[b], b));
      std::vector<std::vector<Row>> mine(n_cu);
      for (const Row& r : rows) {
        Key k = heap.top();
        heap.pop();
        const int b = std::get<2>(k);
        mine[b].push_back(r);
        total[b] += r.cost;
        heap.push(Key(std::get<0>(k) + r.cost, total[b], b));
      }
      for (int b = 0; b < n_cu; ++b) {
        std::sort(mine[b].begin(), mine[b].end(),
                  [](const Row& a, const Row& c) { return a.job != c.job ? a.job < c.job : a.tr < c.tr; });
        for (const Row& r : mine[b]) {
          const int TC = S.sj[r.job].TC, n_sub = (TC + cap - 1) / cap;
          for (int t = 0; t < n_sub; ++t) {
            q4nx::StepUnit u;
            u.job = r.job;
            u.tr = r.tr;
            u.c0 = (int16_t)(t * TC / n_sub);
            u.c1 = (int16_t)((t + 1) * TC / n_sub);
            u.phase = (int16_t)ph;
            u.flags = (int16_t)((t == 0 ? q4nx::kStepFirst : 0) | (t == n_sub - 1 ? q4nx::kStepLast : 0));
            per[b].push_back(u);
          }
        }
      }
    }
    S.first.push_back(0);
    for (int b = 0; b < n_cu; ++b) {
      S.units.insert(S.units.end(), per[b].begin(), per[b].end());
      S.first.push_back((int32_t)S.units.size());
    }
  }
  // mode 0: every phase as one batched GEMV launch whose jobs come from a
  // device table (no limit on their number), shaped as q4nx_gemv_batched
  // shapes one kind's jobs
  struct PhaseT {
    int kind;
    BatchShape sh;
    int n_wg;
    std::vector<q4nx::GemvJob> jobs;
    std::vector<int32_t> wg_job;
    size_t o_jobs = 0, o_wg = 0;
  };
  std::vector<PhaseT> pts;
  for (size_t t = 0; t < order.size();) {
    const int ph = phase[order[t]];
    size_t e = t;
    int64_t total_tr = 0;
    int max_tc = 0;
    while (e < order.size() && phase[order[e]] == ph) {
      total_tr += jobs[order[e]].w.rows / 32;
      max_tc = std::max(max_tc, jobs[order[e]].w.cols / 256);
      ++e;
    }
    PhaseT P;
    P.kind = kind_of(&jobs[order[t]].w);
    P.sh = batch_shape(P.kind, total_tr, max_tc, M);
    int wg = 0;
    for (size_t i = t; i < e; ++i) {
      q4nx::GemvJob g;
      const int n = fill_job(g, &jobs[order[i]], P.sh, total_tr, wg);
      for (int b = 0; b < n; ++b) P.wg_job.push_back((int32_t)P.jobs.size());
      P.jobs.push_back(g);
      wg += n;
    }
    P.n_wg = wg;
    pts.push_back(std::move(P));
    t = e;
  }
  // host tables and device layout
  struct SegT {
    std::vector<q4nx::PlanJob> pj;
    std::vector<int32_t> unit_job;
    std::vector<uint32_t> need;
    int n_slots = 0, smax = 1;
    size_t o_jobs, o_unit, o_need, o_done, o_cnt, o_part, o_ctl;
  };
  std::vector<SegT> tabs(segs.size());
  size_t total = 0;
  for (size_t si = 0; si < segs.size(); ++si) {
    SegH& sg = segs[si];
    SegT& T = tabs[si];
    T.need.assign(sg.n_phases, 0);
    const int cpw = q4nx::plan_cpw(sg.kind);
    int units = 0;
    for (size_t i = 0; i < sg.jobs.size(); ++i) {
      const q4nx_gemv_job& j = jobs[sg.jobs[i]];
      q4nx::PlanJob p;
      p.w = static_cast<const uint8_t*>(j.w.chunks);
      p.x = j.x;
      p.y = j.y;
      p.TR = j.w.rows / 32;
      p.TC = j.w.cols / 256;
      p.ldx = j.w.cols;
      p.ldy = j.w.rows;
      p.S = (p.TC + 4 * cpw - 1) / (4 * cpw);
      p.unit0 = units;
      p.phase = sg.phase_of[i];
      p.slot0 = 0;
      if (p.S > 1) {
        p.slot0 = T.n_slots;
        T.n_slots += p.TR;
        T.smax = std::max(T.smax, p.S);
      }
      T.need[p.phase] += (uint32_t)p.TR;
      for (int u = 0; u < p.TR * p.S; ++u) T.unit_job.push_back((int32_t)i);
      units += p.TR * p.S;
      T.pj.push_back(p);
    }
    T.o_jobs = total;  total = align256(total + T.pj.size() * sizeof(q4nx::PlanJob));
    T.o_unit = total;  total = align256(total + T.unit_job.size() * 4);
    T.o_need = total;  total = align256(total + T.need.size() * 4);
    T.o_done = total;  total = align256(total + T.need.size() * 4);
    T.o_cnt = total;   total = align256(total + (size_t)std::max(T.n_slots, 1) * 4);
    T.o_part = total;  total = align256(total + (size_t)T.n_slots * T.smax * 32 * M * 4);
    T.o_ctl = total;   total = align256(total + 16);
    StepT& S = steps[si];
    if (S.use) {
      S.o_jobs = total;  total = align256(total + S.sj.size() * sizeof(q4nx::StepJob));
      S.o_units = total; total = align256(total + S.units.size() * sizeof(q4nx::StepUnit));
      S.o_first = total; total = align256(total + S.first.size() * 4);
      S.o_sync = total;  total = align256(total + q4nx::step_sync_words(segs[si].n_phases) * 4);
      S.o_ctl = total;   total = align256(total + 16);
    }
  }
  for (PhaseT& P : pts) {
    P.o_jobs = total; total = align256(total + P.jobs.size() * sizeof(q4nx::GemvJob));
    P.o_wg = total;   total = align256(total + P.wg_job.size() * 4);
  }
  // check every kernel can be resident before allocating anything
  std::vector<int> grids(segs.size());
  for (size_t si = 0; si < segs.size(); ++si) {
    int blocks = 0;
    const hipError_t e = q4nx::plan_resident_blocks(segs[si].kind, M, &blocks);
    if (e != hipSuccess) return hip_status(e, "plan occupancy");
    if (blocks < 1) return fail(Q4NX_E_HIP, "plan: kernel cannot be resident");
    grids[si] = std::min(blocks, (int)tabs[si].unit_job.size());
  }
  void* dev = nullptr;
  hipError_t e = hipMalloc(&dev, total);
  if (e != hipSuccess) return hip_status(e, "plan allocation");
  std::vector<uint8_t> host(total, 0);
  for (size_t si = 0; si < segs.size(); ++si) {
    SegT& T = tabs[si];
    memcpy(host.data() + T.o_jobs, T.pj.data(), T.pj.size() * sizeof(q4nx::PlanJob));
    memcpy(host.data() + T.o_unit, T.unit_job.data(), T.unit_job.size() * 4);
    memcpy(host.data() + T.o_need, T.need.data(), T.need.size() * 4);
    const StepT& S = steps[si];
    if (S.use) {
      memcpy(host.data() + S.o_jobs, S.sj.data(), S.sj.size() * sizeof(q4nx::StepJob));
      memcpy(host.data() + S.o_units, S.units.data(), S.units.size() * sizeof(q4nx::StepUnit));
      memcpy(host.data() + S.o_first, S.first.data(), S.first.size() * 4);
    }
  }
  for (const PhaseT& P : pts) {
    memcpy(host.data() + P.o_jobs, P.jobs.data(), P.jobs.size() * sizeof(q4nx::GemvJob));
    memcpy(host.data() + P.o_wg, P.wg_job.data(), P.wg_job.size() * 4);
  }
  e = hipMemcpy(dev, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(dev);
    return hip_status(e, "plan upload");
  }
  q4nx_plan_s* plan = new q4nx_plan_s;
  plan->M = M;
  plan->dev = dev;
  plan->bytes = total;
  uint8_t* d = static_cast<uint8_t*>(dev);
  for (size_t si = 0; si < segs.size(); ++si) {
    SegT& T = tabs[si];
    q4nx_plan_s::Seg s;
    s.kind = segs[si].kind;
    s.grid = grids[si];
    s.args.jobs = reinterpret_cast<const q4nx::PlanJob*>(d + T.o_jobs);
    s.args.unit_job = reinterpret_cast<const int32_t*>(d + T.o_unit);
    s.args.need = reinterpret_cast<const uint32_t*>(d + T.o_need);
    s.args.done = reinterpret_cast<uint32_t*>(d + T.o_done);
    s.args.row_cnt = reinterpret_cast<uint32_t*>(d + T.o_cnt);
    s.args.partial = reinterpret_cast<float*>(d + T.o_part);
    s.args.ctl = reinterpret_cast<uint32_t*>(d + T.o_ctl);
    s.args.n_units = (int32_t)T.unit_job.size();
    s.args.n_phases = segs[si].n_phases;
    s.args.spin_limit = kPlanSpinLimit;
    s.args.smax = T.smax;
    const StepT& S = steps[si];
    if (S.use) {
      s.step = true;
      s.grid = n_cu;
      s.lds = S.lds;
      s.sargs.jobs = reinterpret_cast<const q4nx::StepJob*>(d + S.o_jobs);
      s.sargs.units = reinterpret_cast<const q4nx::StepUnit*>(d + S.o_units);
      s.sargs.wg_first = reinterpret_cast<const int32_t*>(d + S.o_first);
      s.sargs.sync = reinterpret_cast<uint32_t*>(d + S.o_sync);
      s.sargs.ctl = reinterpret_cast<uint32_t*>(d + S.o_ctl);
      s.sargs.n_phases = segs[si].n_phases;
      s.sargs.spin_limit = kPlanSpinLimit;
      s.sargs.ring_off = (int32_t)S.rec;
      s.sargs.ns = S.ns;
      s.args.ctl = s.sargs.ctl;
    }
    plan->segs.push_back(s);
    plan->ctl.push_back(s.args.ctl);
  }
  for (const PhaseT& P : pts) {
    q4nx_plan_s::Phase ph;
    ph.kind = P.kind;
    ph.waves = P.sh.waves;
    ph.xl = P.sh.xl;
    ph.n_wg = P.n_wg;
    memset(&ph.b, 0, sizeof ph.b);
    ph.b.sl = 4 / P.sh.parts;
    ph.b.tab = reinterpret_cast<const q4nx::GemvJob*>(d + P.o_jobs);
    ph.b.tab_wg = reinterpret_cast<const int32_t*>(d + P.o_wg);
    plan->phases.push_back(ph);
  }
  *out = plan;
  return ok();
}

int q4nx_plan_set_mode(q4nx_plan plan, int mode) {
  if (!plan) return fail(Q4NX_E_ARG, "plan_set_mode: null plan");
  if (mode != 0 && mode != 1) return fail(Q4NX_E_ARG, "plan_set_mode: mode %d is neither 0 nor 1", mode);
  plan->mode = mode;
  return ok();
}

int q4nx_plan_run(q4nx_plan plan, void* stream) {
  if (!plan) return fail(Q4NX_E_ARG, "plan_run: null plan");
  if (plan->mode == 0) {
    for (const auto& ph : plan->phases) {
      const hipError_t e = q4nx::launch_gemv(ph.kind, plan->M, ph.waves, ph.b, ph.n_wg, ph.xl,
                                             static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_status(e, "plan phase launch");
    }
    return ok();
  }
  for (const auto& s : plan->segs) {
    const hipError_t e = s.step ? q4nx::launch_step(s.kind, plan->M, s.sargs, s.grid, s.lds,
                                                    static_cast<hipStream_t>(stream))
                                : q4nx::launch_plan(s.kind, plan->M, s.args, s.grid,
                                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_status(e, "plan launch");
  }
  return ok();
}

int q4nx_plan_errors(q4nx_plan plan, uint32_t* flags) {
  if (!plan || !flags) return fail(Q4NX_E_ARG, "plan_errors: null argument");
  uint32_t acc = 0;
  for (uint32_t* c : plan->ctl) {
    uint32_t v = 0;
    hipError_t e = hipMemcpy(&v, c + 1, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e, "plan_errors read");
    acc |= v;
    if (v) {
      const uint32_t zero = 0;
      e = hipMemcpy(c + 1, &zero, 4, hipMemcpyHostToDevice);
      if (e != hipSuccess) return hip_status(e, "plan_errors clear");
    }
  }
  *flags = acc;
  return ok();
}

size_t q4nx_plan_bytes(q4nx_plan plan) { return plan ? plan->bytes : 0; }

void q4nx_plan_destroy(q4nx_plan plan) {
  if (!plan) return;
  if (plan->dev) (void)hipFree(plan->dev);
  delete plan;
}

// ---------------------------------------------------------------------------
// MoE
// ---------------------------------------------------------------------------
static int check_arena(const void* base, int64_t stride, int64_t bytes, int n, int64_t need,
                       const char* name) {
  if (!base) return fail(Q4NX_E_ARG, "moe: null %s arena", name);
  if (!aligned(base, 16) || stride % 16)
    return fail(Q4NX_E_ALIGN, "moe: %s arena or stride not 16-byte aligned", name);
  if (stride < need) return fail(Q4NX_E_SHAPE, "moe: %s stride %lld below one expert's %lld bytes",
                                 name, (long long)stride, (long long)need);
  const int64_t total = (int64_t)(n - 1) * stride + need;
  if (bytes < total)
    return fail(Q4NX_E_SHORT, "moe: %s arena holds %lld bytes, %d experts need %lld", name,
                (long long)bytes, n, (long long)total);
  return Q4NX_OK;
}

static int check_moe_layer(const q4nx_moe_layer* L) {
  if (!L) return fail(Q4NX_E_ARG, "moe: null layer");
  if (L->n_experts < 1 || L->n_experts >= (1 << 19))
    return fail(Q4NX_E_ARG, "moe: n_experts = %d outside 1..524287", L->n_experts);
  if (L->chunk_bytes != Q4NX_Q4_1_BYTES && L->chunk_bytes != Q4NX_Q4_K_BYTES)
    return fail(Q4NX_E_CHUNK_KIND, "moe: experts must be q4_1 (5120) or Q4_K (4736), got %d",
                L->chunk_bytes);
  if (L->d_model <= 0 || L->d_model % 256 || L->d_expert <= 0 || L->d_expert % 256 ||
      L->d_shared < 0 || L->d_shared % 256)
    return fail(Q4NX_E_SHAPE, "moe: d_model, d_expert, d_shared must be multiples of 256 "
                "(d_shared may be 0), got %d, %d, %d", L->d_model, L->d_expert, L->d_shared);
  if (L->d_model > (1 << 20) || L->d_expert > (1 << 20) || L->d_shared > (1 << 20))
    return fail(Q4NX_E_SHAPE, "moe: d_model, d_expert, d_shared must be at most 1048576, got %d, %d, %d",
                L->d_model, L->d_expert, L->d_shared);
  const int64_t cb = L->chunk_bytes;
  const int64_t gu = (int64_t)(L->d_expert / 32) * (L->d_model / 256) * cb;
  const int64_t dn = (int64_t)(L->d_model / 32) * (L->d_expert / 256) * cb;
  int st = check_arena(L->gate, L->gate_stride, L->gate_bytes, L->n_experts, gu, "gate");
  if (!st) st = check_arena(L->up, L->up_stride, L->up_bytes, L->n_experts, gu, "up");
  if (!st) st = check_arena(L->down, L->down_stride, L->down_bytes, L->n_experts, dn, "down");
  if (st) return st;
  if (L->d_shared) {
    const q4nx_weight* sw[3] = {&L->sh_gate, &L->sh_up, &L->sh_down};
    const char* nm[3] = {"moe shared gate", "moe shared up", "moe shared down"};
    for (int i = 0; i < 3; ++i) {
      st = check_weight(sw[i], nm[i]);
      if (st) return st;
      if (sw[i]->chunk_bytes != L->chunk_bytes)
        return fail(Q4NX_E_CHUNK_KIND, "%s: kind differs from the routed experts'", nm[i]);
      const int rows = i < 2 ? L->d_shared : L->d_model;
      const int cols = i < 2 ? L->d_model : L->d_shared;
      if (sw[i]->rows != rows || sw[i]->cols != cols)
        return fail(Q4NX_E_SHAPE, "%s: %d x %d, expected %d x %d", nm[i], sw[i]->rows,
                    sw[i]->cols, rows, cols);
    }
  }
  return Q4NX_OK;
}

static int moe_hstride(const q4nx_moe_layer* L) {
  return L->d_expert > L->d_shared ? L->d_expert : L->d_shared;
}

size_t q4nx_moe_ws(const q4nx_moe_layer* L, int T, int k) {
  if (check_moe_layer(L) || T < 1 || k < 1 || T > 4096 || k > q4nx::kMoeMaxK || T * k > q4nx::kMoeMaxPairs)
    return 0;
  return q4nx::moe_ws_layout(T * k, T, L->d_model, moe_hstride(L)).total;
}

int q4nx_moe_experts(const q4nx_moe_layer* L, const uint16_t* X, const int32_t* ids,
                     const float* p, int T, int k, float* Y, const q4nx_moe_debug* dbg, void* ws,
                     size_t ws_bytes, void* stream) {
  int st = check_moe_layer(L);
  if (st) return st;
  if (!X || !ids || !p || !Y) return fail(Q4NX_E_ARG, "moe: null X, ids, p or Y");
  if (T < 1 || T > 4096 || k < 1 || k > q4nx::kMoeMaxK || T * k > q4nx::kMoeMaxPairs)
    return fail(Q4NX_E_ARG, "moe: T = %d, k = %d outside T 1..4096, k 1..16, T*k <= %d", T, k,
                q4nx::kMoeMaxPairs);
  if (!aligned(X, 16) || !aligned(ids, 4) || !aligned(p, 4) || !aligned(Y, 4))
    return fail(Q4NX_E_ALIGN, "moe: X must be 16-byte, ids/p/Y 4-byte aligned");
  {
    // a batch's prepared activation records (576 bytes per token and tile
    // column, of x for gate/up and of h for down) are staged in at most 64 KB
    // of LDS
    const int tb = T == 1 ? 1 : 4;
    const int inner = std::max(L->d_expert, L->d_shared);
    const int max_d = 65536 / (tb * q4nx::kMoeRecGateUp) * 256;
    const int max_inner = 65536 / (tb * q4nx::kMoeRecDown) * 256;
    if (L->d_model > max_d || inner > max_inner)
      return fail(Q4NX_E_SHAPE, "moe: for T = %d, d_model must be at most %d and d_expert, d_shared at most %d",
                  T, max_d, max_inner);
  }
  const q4nx::MoeWsLayout lay = q4nx::moe_ws_layout(T * k, T, L->d_model, moe_hstride(L));
  if (!ws || ws_bytes < lay.total)
    return fail(Q4NX_E_WORKSPACE, "moe: workspace of %zu bytes, %zu needed", ws_bytes, lay.total);
  if (!aligned(ws, 256)) return fail(Q4NX_E_ALIGN, "moe: workspace not 256-byte aligned");

  q4nx::MoeArgs a;
  memset(&a, 0, sizeof a);
  a.gate = static_cast<const uint8_t*>(L->gate);
  a.up = static_cast<const uint8_t*>(L->up);
  a.down = static_cast<const uint8_t*>(L->down);
  a.gate_stride = L->gate_stride;
  a.up_stride = L->up_stride;
  a.down_stride = L->down_stride;
  if (L->d_shared) {
    a.sgate = static_cast<const uint8_t*>(L->sh_gate.chunks);
    a.sup = static_cast<const uint8_t*>(L->sh_up.chunks);
    a.sdown = static_cast<const uint8_t*>(L->sh_down.chunks);
  }
  a.n_experts = L->n_experts;
  a.D = L->d_model;
  a.De = L->d_expert;
  a.Ds = L->d_shared;
  a.X = X;
  a.ids = ids;
  a.p = p;
  a.Y = Y;
  a.T = T;
  a.k = k;
  a.tb = T == 1 ? 1 : 4;
  a.hstride = moe_hstride(L);
  a.hot_min = L->hot_tokens > 0 ? L->hot_tokens : 0;
  if (dbg) {
    a.dbg_h = dbg->h;
    a.dbg_d = dbg->d;
    a.dbg_h_shared = dbg->h_shared;
    a.dbg_d_shared = dbg->d_shared;
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.hdr = reinterpret_cast<uint32_t*>(w + lay.hdr);
  a.sorted = reinterpret_cast<int32_t*>(w + lay.sorted);
  a.seg = reinterpret_cast<int32_t*>(w + lay.seg);
  a.batch0 = reinterpret_cast<int32_t*>(w + lay.batch0);
  a.btab = reinterpret_cast<int32_t*>(w + lay.btab);
  a.hot = reinterpret_cast<int32_t*>(w + lay.hot);
  a.hbuf = reinterpret_cast<float*>(w + lay.hbuf);
  a.dbuf = reinterpret_cast<float*>(w + lay.dbuf);
  const hipError_t e = q4nx::launch_moe(L->chunk_bytes == Q4NX_Q4_1_BYTES ? q4nx::KIND_Q4_1
                                                                          : q4nx::KIND_Q4_K,
                                        a, static_cast<hipStream_t>(stream));
  return hip_status(e, "moe launch");
}

// ---------------------------------------------------------------------------
// decoders
// ---------------------------------------------------------------------------
int q4nx_unpack(const q4nx_weight* w, uint8_t* codes, uint16_t* meta0, uint16_t* meta1,
                uint16_t* row_meta, void* stream) {
  int st = check_weight(w, "unpack");
  if (st) return st;
  if (!codes || !meta0) return fail(Q4NX_E_ARG, "unpack: null codes or meta0");
  if (!aligned(meta0, 2) || (meta1 && !aligned(meta1, 2)) || (row_meta && !aligned(row_meta, 2)))
    return fail(Q4NX_E_ALIGN, "unpack: metadata outputs must be 2-byte aligned");
  const hipError_t e = q4nx::launch_unpack(kind_of(w), static_cast<const uint8_t*>(w->chunks),
                                           w->rows / 32, w->cols / 256, codes, meta0, meta1,
                                           row_meta, static_cast<hipStream_t>(stream));
  return hip_status(e, "unpack launch");
}

int q4nx_repack_q4k_to_q41(const q4nx_weight* w, void* out, size_t out_bytes, void* stream) {
  int st = check_weight(w, "repack");
  if (st) return st;
  if (w->chunk_bytes != Q4NX_Q4_K_BYTES)
    return fail(Q4NX_E_CHUNK_KIND, "repack: input must be Q4_K (4736-byte chunks), got %d", w->chunk_bytes);
  if (!out) return fail(Q4NX_E_ARG, "repack: null output");
  if (!aligned(out, 16)) return fail(Q4NX_E_ALIGN, "repack: output not 16-byte aligned");
  const int64_t tiles = (int64_t)(w->rows / 32) * (w->cols / 256);
  if (out_bytes < (size_t)tiles * Q4NX_Q4_1_BYTES)
    return fail(Q4NX_E_SHORT, "repack: output holds %zu bytes, %lld needed", out_bytes,
                (long long)(tiles * Q4NX_Q4_1_BYTES));
  if (tiles > 0x7FFFFFFF) return fail(Q4NX_E_SHAPE, "repack: too many tiles");
  const hipError_t e = q4nx::launch_repack_q4k(static_cast<const uint8_t*>(w->chunks), (int)tiles,
                                               static_cast<uint8_t*>(out), static_cast<hipStream_t>(stream));
  return hip_status(e, "repack launch");
}

static_assert(sizeof(q4nx_chunk_layout) == sizeof(q4nx::ChunkLayout), "layout descriptor");

int q4nx_chunk_layout_default(int chunk_bytes, q4nx_chunk_layout* out) {
  if (!out) return fail(Q4NX_E_ARG, "chunk_layout_default: null output");
  if (chunk_bytes != Q4NX_Q4_1_BYTES && chunk_bytes != Q4NX_Q4_K_BYTES)
    return fail(Q4NX_E_CHUNK_KIND, "chunk_layout_default: %d is not 5120 (q4_1) or 4736 (Q4_K)", chunk_bytes);
  q4nx_chunk_layout L;
  memset(&L, 0, sizeof L);
  L.chunk_bytes = chunk_bytes;
  L.code_off = 0; L.code_row = 128; L.code_group = 16; L.code_step = 1;
  L.code_pairing = 0; L.code_high_first = 0;
  if (chunk_bytes == Q4NX_Q4_1_BYTES) {
    L.f0_off = 4096; L.f0_row = 32; L.f0_group = 4;
    L.f1_off = 4098; L.f1_row = 32; L.f1_group = 4;
  } else {
    L.f0_off = 4096; L.f0_row = 16; L.f0_group = 2;
    L.f1_off = 4097; L.f1_row = 16; L.f1_group = 2;
    L.s_off = 4608; L.s_row = 4;
    L.m_off = 4610; L.m_row = 4;
  }
  *out = L;
  return ok();
}

int q4nx_chunk_layout_check(const q4nx_chunk_layout* L) {
  if (!L) return fail(Q4NX_E_ARG, "chunk_layout_check: null layout");
  const int CB = L->chunk_bytes;
  if (CB != Q4NX_Q4_1_BYTES && CB != Q4NX_Q4_K_BYTES)
    return fail(Q4NX_E_CHUNK_KIND, "chunk_layout: chunk size %d is not 5120 (q4_1) or 4736 (Q4_K)", CB);
  if (L->code_pairing != 0 && L->code_pairing != 1)
    return fail(Q4NX_E_ARG, "chunk_layout: code_pairing %d is not 0 or 1", L->code_pairing);
  std::vector<uint8_t> used(CB, 0);
  // a field of `len` bytes at `off`: inside the chunk and on bytes nothing else uses
  auto mark = [&](int64_t off, int len, const char* what, int r, int g) -> int {
    if (off < 0 || off + len > CB)
      return fail(Q4NX_E_ARG, "chunk_layout: %s of row %d, group %d at byte %lld leaves the %d-byte chunk",
                  what, r, g, (long long)off, CB);
    for (int i = 0; i < len; ++i)
      if (used[off + i]++)
        return fail(Q4NX_E_ARG, "chunk_layout: %s of row %d, group %d shares byte %lld with another field",
                    what, r, g, (long long)(off + i));
    return Q4NX_OK;
  };
  for (int r = 0; r < 32; ++r)
    for (int g = 0; g < 8; ++g) {
      for (int b = 0; b < 16; ++b) {   // each code byte holds two codes: mark it once
        const int st = mark((int64_t)L->code_off + (int64_t)r * L->code_row + (int64_t)g * L->code_group +
                                (int64_t)b * L->code_step, 1, "a code byte", r, g);
        if (st) return st;
      }
      const int fl = CB == Q4NX_Q4_1_BYTES ? 2 : 1;
      int st = mark((int64_t)L->f0_off + (int64_t)r * L->f0_row + (int64_t)g * L->f0_group, fl, "field 0", r, g);
      if (!st) st = mark((int64_t)L->f1_off + (int64_t)r * L->f1_row + (int64_t)g * L->f1_group, fl, "field 1", r, g);
      if (st) return st;
    }
  if (CB == Q4NX_Q4_K_BYTES)
    for (int r = 0; r < 32; ++r) {
      int st = mark((int64_t)L->s_off + (int64_t)r * L->s_row, 2, "S", r, 0);
      if (!st) st = mark((int64_t)L->m_off + (int64_t)r * L->m_row, 2, "M", r, 0);
      if (st) return st;
    }
  for (int i = 0; i < CB; ++i)
    if (!used[i]) return fail(Q4NX_E_ARG, "chunk_layout: byte %d of the chunk belongs to no field", i);
  return ok();
}

int q4nx_relayout(const q4nx_chunk_layout* L, const q4nx_weight* src, void* out, size_t out_bytes, void* stream) {
  int st = q4nx_chunk_layout_check(L);
  if (st) return st;
  st = check_weight(src, "relayout");
  if (st) return st;
  if (src->chunk_bytes != L->chunk_bytes)
    return fail(Q4NX_E_CHUNK_KIND, "relayout: weight chunks of %d bytes, layout for %d", src->chunk_bytes,
                L->chunk_bytes);
  if (!out) return fail(Q4NX_E_ARG, "relayout: null output");
  if (!aligned(out, 16)) return fail(Q4NX_E_ALIGN, "relayout: output not 16-byte aligned");
  const int64_t tiles = (int64_t)(src->rows / 32) * (src->cols / 256);
  if (out_bytes < (size_t)(tiles * L->chunk_bytes))
    return fail(Q4NX_E_SHORT, "relayout: output holds %zu bytes, %lld needed", out_bytes,
                (long long)(tiles * L->chunk_bytes));
  if (tiles > 0x7FFFFFFF) return fail(Q4NX_E_SHAPE, "relayout: too many tiles");
  q4nx::ChunkLayout d;
  memcpy(&d, L, sizeof d);
  const hipError_t e = q4nx::launch_relayout(d, static_cast<const uint8_t*>(src->chunks), (int)tiles,
                                             static_cast<uint8_t*>(out), static_cast<hipStream_t>(stream));
  return hip_status(e, "relayout launch");
}

static int gguf_geometry(int gtype, int* block_bytes, int* block_cols, int* align) {
  switch (gtype) {
    case Q4NX_GGUF_Q4_0: *block_bytes = 18; *block_cols = 32; *align = 2; return 1;
    case Q4NX_GGUF_Q4_1: *block_bytes = 20; *block_cols = 32; *align = 4; return 1;
    case Q4NX_GGUF_Q4_K: *block_bytes = 144; *block_cols = 256; *align = 16; return 1;
    default: return 0;
  }
}

size_t q4nx_gguf_bytes(int gguf_type, int rows, int cols) {
  int bb, bc, al;
  if (!gguf_geometry(gguf_type, &bb, &bc, &al) || rows <= 0 || cols <= 0 || cols % bc) return 0;
  return (size_t)rows * (size_t)(cols / bc) * (size_t)bb;
}

int q4nx_gguf_to_q41(int gguf_type, const void* src, size_t src_bytes, int rows, int cols, void* out,
                     size_t out_bytes, void* stream) {
  int bb, bc, al;
  if (!gguf_geometry(gguf_type, &bb, &bc, &al))
    return fail(Q4NX_E_ARG, "gguf: type %d is not Q4_0 (2), Q4_1 (3) or Q4_K (12)", gguf_type);
  if (!src || !out) return fail(Q4NX_E_ARG, "gguf: null source or output");
  if (rows <= 0 || cols <= 0 || rows % 32 || cols % 256)
    return fail(Q4NX_E_SHAPE, "gguf: %d x %d is not a whole number of 32 x 256 tiles", rows, cols);
  const int64_t tiles = (int64_t)(rows / 32) * (cols / 256);
  if (tiles > 0x7FFFFFFF) return fail(Q4NX_E_SHAPE, "gguf: too many tiles");
  if (!aligned(src, al)) return fail(Q4NX_E_ALIGN, "gguf: source not %d-byte aligned", al);
  if (!aligned(out, 16)) return fail(Q4NX_E_ALIGN, "gguf: output not 16-byte aligned");
  const size_t need = q4nx_gguf_bytes(gguf_type, rows, cols);
  if (src_bytes < need)
    return fail(Q4NX_E_SHORT, "gguf: source holds %zu bytes, %zu needed", src_bytes, need);
  if (out_bytes < (size_t)tiles * Q4NX_Q4_1_BYTES)
    return fail(Q4NX_E_SHORT, "gguf: output holds %zu bytes, %lld needed", out_bytes,
                (long long)(tiles * Q4NX_Q4_1_BYTES));
  const hipError_t e = q4nx::launch_gguf_q41(gguf_type, static_cast<const uint8_t*>(src), rows / 32, cols / 256,
                                             static_cast<uint8_t*>(out), static_cast<hipStream_t>(stream));
  return hip_status(e, "gguf launch");
}

int q4nx_q8_rows(const q4nx_weight* w, const int32_t* ids, int T, float* out, void* stream) {
  int st = check_weight(w, "q8_rows");
  if (st) return st;
  if (w->chunk_bytes != Q4NX_Q8_BYTES)
    return fail(Q4NX_E_CHUNK_KIND, "q8_rows: weight must be Q8 (8704-byte chunks), got %d", w->chunk_bytes);
  if (!ids || !out) return fail(Q4NX_E_ARG, "q8_rows: null ids or output");
  if (T < 1 || T > 65535) return fail(Q4NX_E_ARG, "q8_rows: T = %d outside 1..65535", T);
  if (!aligned(ids, 4) || !aligned(out, 4)) return fail(Q4NX_E_ALIGN, "q8_rows: ids and out must be 4-byte aligned");
  const hipError_t e = q4nx::launch_q8_rows(kind_of(w), static_cast<const uint8_t*>(w->chunks), w->rows,
                                            w->cols / 256, ids, T, out, static_cast<hipStream_t>(stream));
  return hip_status(e, "q8_rows launch");
}

size_t q4nx_argmax_ws(int n, int M) {
  if (n < 1 || M < 1 || M > 65535) return 0;
  return (size_t)M * q4nx::argmax_parts(n) * 8;
}

int q4nx_argmax(const float* y, int n, int ldy, int M, int32_t* idx, float* val, void* ws,
                size_t ws_bytes, void* stream) {
  if (!y || !idx) return fail(Q4NX_E_ARG, "argmax: null y or idx");
  if (n < 1 || ldy < n || M < 1 || M > 65535)
    return fail(Q4NX_E_ARG, "argmax: n = %d, ldy = %d, M = %d (need 1 <= n <= ldy, 1 <= M <= 65535)", n, ldy, M);
  if (!aligned(y, 4) || !aligned(idx, 4) || (val && !aligned(val, 4)))
    return fail(Q4NX_E_ALIGN, "argmax: y, idx and val must be 4-byte aligned");
  if (ws) {
    const size_t need = q4nx_argmax_ws(n, M);
    if (ws_bytes < need)
      return fail(Q4NX_E_WORKSPACE, "argmax: workspace of %zu bytes, %zu needed", ws_bytes, need);
    if (!aligned(ws, 8)) return fail(Q4NX_E_ALIGN, "argmax: workspace not 8-byte aligned");
  }
  const hipError_t e = q4nx::launch_argmax(y, n, ldy, M, idx, val, ws, static_cast<hipStream_t>(stream));
  return hip_status(e, "argmax launch");
}

int q4nx_moe_router(const uint16_t* R, const uint16_t* X, int T, int D, int E, int k, int renorm,
                    int32_t* ids, float* p, float* logits, void* stream) {
  if (!R || !X || !ids || !p || !logits) return fail(Q4NX_E_ARG, "router: null R, X, ids, p or logits");
  if (T < 1 || T > 65535) return fail(Q4NX_E_ARG, "router: T = %d outside 1..65535", T);
  if (!(D == 512 || D == 1024 || D == 2048 || D == 4096))
    return fail(Q4NX_E_SHAPE, "router: D = %d is not 512, 1024, 2048 or 4096", D);
  if (E < 1 || E > 1024) return fail(Q4NX_E_ARG, "router: E = %d outside 1..1024", E);
  if (k < 1 || k > 16 || k > E) return fail(Q4NX_E_ARG, "router: k = %d outside 1..min(16, E)", k);
  if (!aligned(R, 16) || !aligned(X, 16) || !aligned(ids, 4) || !aligned(p, 4) || !aligned(logits, 4))
    return fail(Q4NX_E_ALIGN, "router: R and X must be 16-byte, ids/p/logits 4-byte aligned");
  const hipError_t e = q4nx::launch_moe_router(R, X, T, D, E, k, renorm ? 1 : 0, ids, p, logits,
                                               static_cast<hipStream_t>(stream));
  return hip_status(e, "router launch");
}

int q4nx_decode(const q4nx_weight* w, float* out, void* stream) {
  int st = check_weight(w, "decode");
  if (st) return st;
  if (!out) return fail(Q4NX_E_ARG, "decode: null output");
  if (!aligned(out, 4)) return fail(Q4NX_E_ALIGN, "decode: output not 4-byte aligned");
  const hipError_t e = q4nx::launch_decode(kind_of(w), static_cast<const uint8_t*>(w->chunks),
                                           w->rows / 32, w->cols / 256, out,
                                           static_cast<hipStream_t>(stream));
  return hip_status(e, "decode launch");
}

}  // extern "C"
