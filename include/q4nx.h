/*
 * q4nx.h -- C ABI of libq4nx.so: fused dequantize-and-multiply of Q4NX-tiled
 * low-bit weights against bf16 activations on AMD MI355X (gfx950).
 *
 * The weight format is the Q4NX chunk grid of the 1bit engine docs, page
 * "NPU engine", section "Q4NX chunks": a weight of `rows` outputs by `cols`
 * inputs is a grid of 32-row x 256-column tiles, one chunk per tile, row-major
 * over the grid (tile (tr, tc) is chunk tr*(cols/256) + tc), and the chunk size
 * names the kind:
 *
 *   5120 B  q4_1  weight = code * scale + zero    bf16 scale, zero per 32 columns of a row
 *   4736 B  Q4_K  weight = S * scale * code + M * min
 *                                                 u8 scale, min per 32 columns; bf16 S, M per row
 *   8704 B  Q8    weight = d * code               int8 codes; bf16 d per 32 columns
 *
 * Q8 has two code layouts under the one size, and nothing in a tensor tells
 * them apart (same section), so a Q8 weight must name its layout:
 *   Q4NX_Q8_LAYOUT_A: code (r, k) of a tile at byte k*32 + r
 *   Q4NX_Q8_LAYOUT_B: at (r/16)*4096 + (k/32)*512 + (k%32)*16 + r%16
 *
 * The byte order inside q4_1 and Q4_K chunks, and the place of the Q8 scales,
 * are deferred by that section to a header that is not published.  This
 * library reads them as follows (r = row in the tile 0..31, k = column in the
 * tile 0..255, g = k/32; all fields little-endian):
 *   q4_1: code (r, k) in byte r*128 + k/2, even k in the low nibble;
 *         (scale, zero) bf16 pair of (r, g) at byte 4096 + 4*(8r + g).
 *   Q4_K: codes as q4_1; (scale, min) u8 pair of (r, g) at 4096 + 2*(8r + g);
 *         (S, M) bf16 pair of row r at 4608 + 4r.
 *   Q8:   d bf16 of (r, g) at 8192 + 2*(8r + g).
 *
 * Conventions of every call:
 *  - Pointers marked DEVICE are device memory owned by the caller.  Only a
 *    plan (q4nx_plan_create) keeps pointers past the call that takes them, and
 *    only q4nx_plan_create allocates device memory; every other call keeps
 *    nothing and allocates nothing.
 *  - Calls that take a stream enqueue work on it and return without waiting;
 *    the caller synchronises before reading results.  `stream` is a
 *    hipStream_t passed as void* (NULL = the default stream).
 *  - Every argument, shape and size is checked on the host before anything is
 *    enqueued; a failing check returns its status and enqueues nothing.  The
 *    status of the last failing call on the calling thread is described by
 *    q4nx_last_error().  No C++ exception crosses this interface.
 *  - Activations are bf16 bit patterns (uint16_t); products accumulate in
 *    fp32 and outputs are fp32.  Denormals are kept, never flushed.
 *  - Results are deterministic: the same inputs give the same bytes on every
 *    run (no floating-point atomics; every sum has a fixed order).
 */
#ifndef Q4NX_H
#define Q4NX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call (0 = success). */
typedef enum q4nx_status {
  Q4NX_OK = 0,
  Q4NX_E_ARG = 1,        /* null pointer where one is required, or a count out of range */
  Q4NX_E_CHUNK_KIND = 2, /* chunk_bytes is not 5120, 4736 or 8704, or the kind is not
                            supported by the call */
  Q4NX_E_SHAPE = 3,      /* rows not a positive multiple of 32 or cols of 256, or shapes
                            that do not fit together */
  Q4NX_E_SHORT = 4,      /* nbytes smaller than (rows/32)*(cols/256)*chunk_bytes */
  Q4NX_E_ALIGN = 5,      /* a pointer is not aligned as the call requires */
  Q4NX_E_WORKSPACE = 6,  /* workspace missing or smaller than the *_ws() size */
  Q4NX_E_Q8_LAYOUT = 7,  /* a Q8 weight without Q4NX_Q8_LAYOUT_A or _B */
  Q4NX_E_HIP = 8         /* the HIP runtime refused a launch; see q4nx_last_error() */
} q4nx_status;

enum { Q4NX_Q4_1_BYTES = 5120, Q4NX_Q4_K_BYTES = 4736, Q4NX_Q8_BYTES = 8704 };
enum { Q4NX_Q8_LAYOUT_UNSET = -1, Q4NX_Q8_LAYOUT_A = 0, Q4NX_Q8_LAYOUT_B = 1 };

/* Largest M (activation rows) of one q4nx_gemv / q4nx_gemv_batched call. */
enum { Q4NX_GEMV_MAX_M = 8 };
/* Largest M of one q4nx_gemm_block call (a prompt block of 64 tokens). */
enum { Q4NX_GEMM_MAX_M = 64 };
/* Most jobs one q4nx_gemv_batched call takes. */
enum { Q4NX_BATCH_MAX_JOBS = 64 };
/* Most weights of one q4nx_gemm_batched call. */
enum { Q4NX_GEMM_BATCH_MAX_JOBS = 8 };

/* One Q4NX weight, described on the host. */
typedef struct q4nx_weight {
  const void* chunks;   /* DEVICE, [rows/32][cols/256][chunk_bytes], 16-byte aligned */
  int64_t nbytes;       /* bytes available at `chunks`; must cover every chunk */
  int32_t rows;         /* outputs N, a positive multiple of 32 */
  int32_t cols;         /* inputs K, a positive multiple of 256 */
  int32_t chunk_bytes;  /* 5120 (q4_1), 4736 (Q4_K) or 8704 (Q8): the kind */
  int32_t q8_layout;    /* Q4NX_Q8_LAYOUT_A or _B when chunk_bytes == 8704, else ignored */
} q4nx_weight;

/*
 * Host-only check of a weight descriptor: the chunk-kind and length rules of
 * the NPU engine page ("Q4NX chunks": an unknown chunk size or a tensor
 * shorter than its layout needs is refused; the Q8 layout cannot be detected,
 * so it must be given).  Touches no device memory.
 * Returns Q4NX_OK, E_ARG (w or w->chunks NULL), E_CHUNK_KIND, E_SHAPE, E_SHORT,
 * E_ALIGN (chunks not 16-byte aligned) or E_Q8_LAYOUT.
 */
int q4nx_weight_check(const q4nx_weight* w);

/*
 * y[m][n] = sum_k W[n][k] * x[m][k] for m < M: the dequantize-and-multiply of
 * decode (Strata article, section 1: decode speed is set by the weight bytes
 * read per token; section 4.1: a verify window reads the weights once for
 * several tokens' mat-vecs).  Each chunk is read from HBM once per call
 * whatever M is.
 *   w  host descriptor (checked as q4nx_weight_check)
 *   x  DEVICE bf16 [M][w->cols], row-major, 16-byte aligned
 *   y  DEVICE fp32 [M][w->rows], row-major, 4-byte aligned; fully overwritten
 *   M  1..Q4NX_GEMV_MAX_M
 * All chunk kinds.  Error |y - y_exact| stays far inside 2e-3 * sum_k |w x| for
 * the kernels' fp32 arithmetic (bf16 codes/activations exact, fp32 sums).
 */
int q4nx_gemv(const q4nx_weight* w, const uint16_t* x, float* y, int M, void* stream);

/* One independent GEMV of a batch. */
typedef struct q4nx_gemv_job {
  q4nx_weight w;
  const uint16_t* x;  /* DEVICE bf16 [M][w.cols] */
  float* y;           /* DEVICE fp32 [M][w.rows] */
} q4nx_gemv_job;

/*
 * Runs n_jobs independent GEMVs (all with the same M) as few launches as the
 * chunk kinds allow: one per kind present.  Meant for the projections of a
 * layer that read one input (q|k|v, gate|up) and, generally, for many small
 * GEMVs whose single launches would be dominated by launch cost.  Jobs must
 * not write overlapping y.
 *   jobs    HOST array of n_jobs descriptors (read during the call only)
 *   n_jobs  1..Q4NX_BATCH_MAX_JOBS
 * Errors as q4nx_gemv, checked for every job before anything is enqueued.
 */
int q4nx_gemv_batched(const q4nx_gemv_job* jobs, int n_jobs, int M, void* stream);

/*
 * A GEMV plan: a whole decode step's GEMVs, prepared once, run many times.
 *
 * A decode step is a chain of GEMV groups that depend on each other (per
 * layer q|k|v, o, gate|up, down, then the lm_head); the Strata article
 * (section 3.2) runs its whole pass as one captured graph so that no step
 * waits on the host.  A plan holds the step's job tables on the device and
 * runs every job of phase p only after every job of phase p-1 has written its
 * y.  Two ways to run it (q4nx_plan_set_mode):
 *   0 (default)  one batched GEMV launch per phase, its jobs read from the
 *                plan's device table (so a phase may hold any number of jobs:
 *                thousands of independent GEMVs go in one launch), each launch
 *                shaped as q4nx_gemv_batched shapes it.  Stream order makes
 *                the phases wait for each other.
 *   1            one persistent launch per run of same-kind phases: the
 *                workgroups wait for each other on the device, and the weight
 *                loads of phase p + 1 are issued before that wait.  (q4_1 and
 *                Q4_K runs whose activations fit in LDS use one workgroup per
 *                CU with a static schedule; other runs and Q8 deal tile rows
 *                to a resident grid.)  On MI355X a device-wide hand-off costs
 *                more than a kernel boundary, so mode 0 is the faster one for
 *                a decode step.
 *
 *   jobs    HOST array of n_jobs GEMVs (copied into the plan; the weights, x
 *           and y they point at must stay allocated while the plan is used)
 *   phase   HOST array of n_jobs phase numbers >= 0; a job's x may be written
 *           by jobs of lower phases; jobs of one phase must share a chunk kind
 *   n_jobs  1..65536;  M 1..4
 *   out     receives the plan handle
 * q4nx_plan_create allocates the plan's device tables (hipMalloc) and copies
 * them (synchronously); it is the only allocating call of the library.
 * q4nx_plan_run enqueues the plan's launches on `stream`; it allocates
 * nothing and may be captured in a HIP graph.  Runs of one plan must not
 * overlap each other.  In mode 1 a launch assumes the whole GPU (it sizes its
 * grid to stay resident); if a wait ever exceeds its spin limit (a grid that
 * could not become resident), the kernel sets an error flag instead of
 * hanging; q4nx_plan_errors reads and clears it (synchronous).
 */
typedef struct q4nx_plan_s* q4nx_plan;

int q4nx_plan_create(const q4nx_gemv_job* jobs, const int32_t* phase, int n_jobs, int M,
                     q4nx_plan* out);
int q4nx_plan_run(q4nx_plan plan, void* stream);
/* mode 0: one launch per phase (default); 1: persistent launches.  E_ARG otherwise. */
int q4nx_plan_set_mode(q4nx_plan plan, int mode);
/* flags: bit 0 = a phase wait timed out.  Returns Q4NX_OK or Q4NX_E_HIP. */
int q4nx_plan_errors(q4nx_plan plan, uint32_t* flags);
/* Device bytes the plan holds (tables, counters, partial rows). */
size_t q4nx_plan_bytes(q4nx_plan plan);
void q4nx_plan_destroy(q4nx_plan plan);

/*
 * Y[m][n] = sum_k W[n][k] * X[m][k] for a prompt block of M <= 64 rows (onw
 * technical notes, "dense model prompts in 64-token blocks": group-quantised
 * matmul throughput levels off at 64 rows).  Each chunk is read once and
 * dequantised once to bf16 (round to nearest even) for the bf16 matrix cores,
 * with fp32 accumulation.
 *   w  host descriptor; q4_1 or Q4_K (E_CHUNK_KIND for Q8)
 *   X  DEVICE bf16 [M][w->cols], 16-byte aligned
 *   Y  DEVICE fp32 [M][w->rows]; fully overwritten
 *   M  1..Q4NX_GEMM_MAX_M
 *   ws DEVICE workspace of q4nx_gemm_block_ws(w) bytes, 256-byte aligned (may
 *      be NULL when that size is 0).  It must hold zeros before its first use;
 *      every call leaves it ready for the next one.  Its layout does not
 *      depend on the call (a 4 KB header of counters, claim words and flags,
 *      then the partial tiles), so one buffer of the largest size any call
 *      needs serves calls of any shape, one call at a time.  (K is split over
 *      several workgroups when the tile rows alone would leave CUs idle; the
 *      workspace holds their partial tiles.  The parts of a row are placed on
 *      one XCD so they meet in its L2; a workgroup that lands elsewhere, as
 *      concurrent work on other streams can cause, detects it and computes its
 *      rows whole, so the result is the same wherever workgroups land.  The
 *      uint32 at byte 3072 of the workspace counts such workgroups; the
 *      library never resets it.)
 * The bf16 rounding of each weight moves it by at most 2^-8 of its size; with
 * random signs the error of a sum over K stays well inside 2e-3 * sum |w x|.
 */
int q4nx_gemm_block(const q4nx_weight* w, const uint16_t* X, float* Y, int M, void* ws,
                    size_t ws_bytes, void* stream);
/* Workspace bytes q4nx_gemm_block needs for this weight (0 = none). */
size_t q4nx_gemm_block_ws(const q4nx_weight* w);

/*
 * q4nx_gemm_block without a workspace argument and without allocating, for
 * callers that cannot allocate device memory: code under stream capture,
 * tight serving loops, hosts that forbid hipMalloc.  Same arguments, result
 * and errors as q4nx_gemm_block; its workspace is a static array of
 * q4nx_gemm_block_noalloc_max() bytes (a 4 KB header + 16 MiB, enough for
 * every split the GEMM makes) that each GPU the library runs on holds until
 * the process ends.  Each call first clears the array's header with a small
 * kernel on `stream` (no memset node), then runs the GEMM.  The array keeps
 * the last call's contents and is shared by every call on one GPU: calls that
 * may overlap on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.  A call whose split would need more than the array
 * returns Q4NX_E_WORKSPACE.  The XCD placement of the K parts is used only
 * when an earlier allocating call has already probed the device; otherwise
 * the parts exchange through device-coherent stores (the same result).
 */
int q4nx_gemm_block_noalloc(const q4nx_weight* w, const uint16_t* X, float* Y, int M, void* stream);
/* Bytes of the static workspace of q4nx_gemm_block_noalloc. */
size_t q4nx_gemm_block_noalloc_max(void);

/*
 * Test and tuning switch of the block GEMM's split-K exchange, for every later
 * call in the process: 0 (default) puts the K parts of a row on one XCD when a
 * one-time probe of the device shows workgroups dealt to XCDs round-robin;
 * 1 does the same but makes the workgroups of every odd group act displaced
 * (the path a workgroup takes when another of its group landed on its XCD);
 * 2 always uses the device-coherent exchange (partials through device-scope
 * stores and loads).  The results are the same in every mode.  Returns
 * Q4NX_OK or E_ARG.
 */
int q4nx_gemm_exchange_mode(int mode);

/*
 * The block GEMM of several weights that read the same X (the q, k and v
 * projections of a layer, or its gate and up projections) in one launch:
 * Y_j = W_j X for every job, exactly as q4nx_gemm_block computes each.
 *   jobs    n_jobs (1..Q4NX_GEMM_BATCH_MAX_JOBS) weights with their outputs;
 *           every weight has the chunk kind (q4_1 or Q4_K) and the column
 *           count of jobs[0] (E_SHAPE otherwise)
 *   X       DEVICE bf16 [M][cols], 16-byte aligned, shared by all jobs
 *   Y_j     DEVICE fp32 [M][w.rows]; fully overwritten
 *   ws      DEVICE workspace of q4nx_gemm_batched_ws(jobs, n_jobs) bytes, with
 *           the rules of q4nx_gemm_block's workspace
 */
typedef struct q4nx_gemm_job {
  q4nx_weight w;
  float* Y;
} q4nx_gemm_job;

int q4nx_gemm_batched(const q4nx_gemm_job* jobs, int n_jobs, const uint16_t* X, int M, void* ws,
                      size_t ws_bytes, void* stream);
/* Workspace bytes of q4nx_gemm_batched for these jobs (0 = none or bad jobs). */
size_t q4nx_gemm_batched_ws(const q4nx_gemm_job* jobs, int n_jobs);

/*
 * One routed-expert MoE layer (Strata article, section 2 "target model": per
 * layer 512 routed experts, the router picks 10, plus a shared expert every
 * token, then the sum; onw technical notes, "MoE on the NPU": only the
 * selected experts' weights are bound, by id, without copying the table).
 *
 * Routed experts all have the same kind and shape; expert e's gate, up and
 * down chunks start at gate + e*gate_stride (etc.) of one device arena.
 */
typedef struct q4nx_moe_layer {
  int32_t n_experts;     /* routed experts in the arena, >= 1 */
  int32_t d_model;       /* model width D: gate/up cols, down rows (mult. of 256, <= 1048576) */
  int32_t d_expert;      /* routed intermediate width: gate/up rows, down cols (mult. of 256, <= 1048576) */
  int32_t d_shared;      /* shared intermediate width (mult. of 256, <= 1048576), or 0 for none */
  int32_t chunk_bytes;   /* kind of every expert weight: 5120 (q4_1) or 4736 (Q4_K) */
  int32_t hot_tokens;    /* prompt-block calls (T * k > 64): an expert chosen by at least this
                            many pairs, and the shared expert when T reaches it, runs on the
                            bf16 matrix cores (see q4nx_moe_experts); 0 or negative: never
                            (the default: measured faster at the 512-expert block) */
  const void* gate;      /* DEVICE, expert e at gate + e*gate_stride, [d_expert/32][D/256] chunks */
  const void* up;        /* DEVICE, same shape as gate */
  const void* down;      /* DEVICE, expert e at down + e*down_stride, [D/32][d_expert/256] chunks */
  int64_t gate_stride, up_stride, down_stride;   /* bytes between experts, 16-byte multiples */
  int64_t gate_bytes, up_bytes, down_bytes;      /* bytes available in each arena */
  q4nx_weight sh_gate;   /* shared expert [d_shared][D]; ignored when d_shared == 0 */
  q4nx_weight sh_up;     /* [d_shared][D] */
  q4nx_weight sh_down;   /* [D][d_shared] */
} q4nx_moe_layer;

/* Optional stage outputs of q4nx_moe_experts, for stage-wise checking. */
typedef struct q4nx_moe_debug {
  float* h;             /* DEVICE fp32 [T][k][d_expert]: silu(G x) * (U x) */
  float* d;             /* DEVICE fp32 [T][k][D]: down projection of h, before weighting */
  float* h_shared;      /* DEVICE fp32 [T][d_shared] */
  float* d_shared;      /* DEVICE fp32 [T][D] */
} q4nx_moe_debug;

/* Workspace bytes q4nx_moe_experts needs for T tokens and k slots. */
size_t q4nx_moe_ws(const q4nx_moe_layer* L, int T, int k);

/*
 * Y[t] = sum_{j<k} p[t][j] * Down_e (silu(Gate_e X[t]) * (Up_e X[t])) + (shared expert, weight 1)
 * with e = ids[t][j].  The (token, slot) pairs are sorted by expert on the
 * device so that each selected expert's weights are read once per call
 * however many tokens chose it (onw technical notes, "computing MoE prompts
 * together": tokens grouped by expert, each expert read once per prompt).
 * The intermediate h stays fp32; the down projection reads it as fp16 with
 * a power-of-two scale per 32 values (round to nearest: each h moves by at
 * most 2^-12 of its size while it lies within 2^29 of the largest of its 32,
 * so d is within 2^-12 * sum |w h| plus the fp32 sums); the weighted sum over
 * slots runs in slot order, then the shared expert, in fp32, with no atomics.
 * In prompt-block calls (T * k > 64) an expert chosen by at least
 * L->hot_tokens pairs, and the shared expert when T reaches it, runs on the
 * bf16 matrix cores instead: each weight and each h carried as two bf16
 * parts, hi = bf16(v) and lo = bf16(v - hi) (to 2^-16 of its size), fp32
 * accumulation.  A token's bits then depend on
 * whether its experts reached that count in the call; with hot_tokens <= 0
 * (the default) they never do, and a token's bits do not depend on the other
 * tokens.
 *   X    DEVICE bf16 [T][D]; ids DEVICE int32 [T][k]; p DEVICE fp32 [T][k]
 *   Y    DEVICE fp32 [T][D], fully overwritten
 *   T    1..4096, k 1..16, T*k <= 4096.  A batch's prepared activations are
 *        staged in 64 KB of LDS, so d_model, d_expert and d_shared are at most
 *        28928 (T = 1) or 7168 (T > 1), else E_SHAPE
 *   dbg  NULL, or stage outputs to fill (any member may be NULL)
 *   ws   DEVICE workspace of at least q4nx_moe_ws(L, T, k) bytes, 256-byte aligned
 * An id outside [0, n_experts) is never dereferenced: its slot contributes 0
 * and bit 0 of the uint32 at ws[0] is set (cleared at the start of each call;
 * read it after synchronising).
 */
int q4nx_moe_experts(const q4nx_moe_layer* L, const uint16_t* X, const int32_t* ids,
                     const float* p, int T, int k, float* Y, const q4nx_moe_debug* dbg,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Q4_K -> q4_1 repack (NPU engine page, "Q4NX chunks": Q4_K repacks into
 * q4_1 exactly apart from rounding S * scale and M * min to bf16, so one
 * q4_1 kernel serves both kinds).  Writes tiles = (rows/32) * (cols/256)
 * q4_1 chunks of 5120 bytes in the same tile order: codes unchanged,
 * scale'(r, g) = bf16(S(r) * sc(r, g)) and zero'(r, g) = bf16(M(r) * mn(r, g)),
 * each product exact in fp32 and rounded once to nearest even.  Products
 * that overflow fp32 are outside the repack's domain (they give +-Inf).
 *   w          host descriptor of a Q4_K weight (E_CHUNK_KIND otherwise)
 *   out        DEVICE, 16-byte aligned, out_bytes >= tiles * 5120 (E_SHORT)
 * The result is a q4_1 weight of the same rows and cols; describe it with
 * chunk_bytes = 5120 to use it.  Asynchronous on stream.
 */
int q4nx_repack_q4k_to_q41(const q4nx_weight* w, void* out, size_t out_bytes, void* stream);

/*
 * In-chunk layout of a q4_1 or Q4_K chunk (NPU engine page, "Q4NX chunks":
 * the chunk sizes and what each kind holds are printed there, the byte order
 * inside a chunk is left to a header that is not published).  The library's
 * own order is the one at the top of this file; a layout descriptor says where
 * another producer's chunks keep each field, so its tensors can be converted
 * (q4nx_relayout) and then used by every call.  For row r (0..31), group
 * g = k/32 (0..7) and j = k%32 of a tile:
 *   code (r, k): byte code_off + r*code_row + g*code_group + b*code_step, with
 *     code_pairing 0: b = j/2, the codes j and j+1 share a byte, nibble n = j%2;
 *     code_pairing 1: b = j%16, the codes j and j+16 share a byte, n = j/16;
 *     nibble n = 0 is the low one, or the high one when code_high_first != 0.
 *   per (r, g): field 0 at f0_off + r*f0_row + g*f0_group, field 1 likewise:
 *     q4_1: bf16 scale, bf16 zero;  Q4_K: u8 scale, u8 min.
 *   per row r (Q4_K only): bf16 S at s_off + r*s_row, bf16 M at m_off + r*m_row.
 * Multi-byte fields are little-endian.  A valid layout puts every field inside
 * the chunk and uses each of its bytes exactly once (4096 code bytes plus the
 * metadata fill the chunk size exactly).
 */
typedef struct q4nx_chunk_layout {
  int32_t chunk_bytes;   /* 5120 (q4_1) or 4736 (Q4_K) */
  int32_t code_off, code_row, code_group, code_step, code_pairing, code_high_first;
  int32_t f0_off, f0_row, f0_group;
  int32_t f1_off, f1_row, f1_group;
  int32_t s_off, s_row;  /* Q4_K only */
  int32_t m_off, m_row;  /* Q4_K only */
} q4nx_chunk_layout;

/* The library's own layout for 5120 or 4736 (E_CHUNK_KIND otherwise). */
int q4nx_chunk_layout_default(int chunk_bytes, q4nx_chunk_layout* out);

/*
 * Host-only check of a layout: E_CHUNK_KIND for another chunk size, E_ARG when
 * a field leaves the chunk, two fields share a byte or a byte is unused (the
 * detail names the first such field and tile position).
 */
int q4nx_chunk_layout_check(const q4nx_chunk_layout* L);

/*
 * Chunks in layout L -> the same weight in the library's layout, bit for bit
 * (codes and metadata are moved, never changed).  src describes the input
 * tensor (its chunk_bytes must equal L->chunk_bytes); out receives
 * (rows/32)*(cols/256) chunks of the same size, 16-byte aligned (E_SHORT when
 * out_bytes is smaller).  One workgroup per chunk, staged through LDS.
 * Asynchronous on stream; src and out must not overlap.
 */
int q4nx_relayout(const q4nx_chunk_layout* L, const q4nx_weight* src, void* out, size_t out_bytes,
                  void* stream);

/*
 * GGUF 4-bit tensors -> q4_1 chunks (NPU engine page, section "From a GGUF":
 * the exact GGUF types map to q4_1 with codes unchanged, Q4_0 as scale d and
 * zero -8d, Q4_1 as scale d and zero m, Q4_K per 32-column sub-block as scale
 * d*sc and zero -dmin*mn, a Q4_K super-block covering one tile row's 256
 * columns; the only error is rounding scale and zero to bf16).  The type
 * numbers are GGUF's own.  The blocks are the GGUF format's, little-endian:
 *   Q4_0  18 B per 32 weights: fp16 d, 16 code bytes (weight j < 16 in the low
 *         nibble of byte j, weight j + 16 in its high nibble); w = d (q - 8)
 *   Q4_1  20 B per 32 weights: fp16 d, fp16 m, 16 code bytes as Q4_0; w = d q + m
 *   Q4_K  144 B per 256 weights: fp16 d, fp16 dmin, 12 bytes of 6-bit (sc, mn)
 *         for 8 sub-blocks, 128 code bytes (sub-block j in the low (j even) or
 *         high (j odd) nibbles of bytes 32 (j/2) .. 32 (j/2) + 31);
 *         w = d sc q - dmin mn
 * and the tensor is rows x cols weights, each row its cols/32 (Q4_K cols/256)
 * blocks in column order.  Each scale and zero is formed exactly in fp32 and
 * rounded once to nearest even bf16; non-finite fp16 fields are outside the
 * conversion's domain.
 *   gguf_type  Q4NX_GGUF_Q4_0, _Q4_1 or _Q4_K (E_ARG otherwise)
 *   src        DEVICE, src_bytes >= q4nx_gguf_bytes(type, rows, cols) (E_SHORT);
 *              2-byte (Q4_0), 4-byte (Q4_1) or 16-byte (Q4_K) aligned (E_ALIGN)
 *   rows, cols positive multiples of 32 and 256 (E_SHAPE)
 *   out        DEVICE, 16-byte aligned, out_bytes >= (rows/32)*(cols/256)*5120
 * The result is a q4_1 weight of the same shape (chunk_bytes = 5120), tiles in
 * the usual row-major order.  Asynchronous on stream.
 * q4nx_gguf_bytes returns the tensor's byte size, or 0 for an unknown type or
 * a cols that is not a whole number of blocks.
 */
enum { Q4NX_GGUF_Q4_0 = 2, Q4NX_GGUF_Q4_1 = 3, Q4NX_GGUF_Q4_K = 12 };
size_t q4nx_gguf_bytes(int gguf_type, int rows, int cols);
int q4nx_gguf_to_q41(int gguf_type, const void* src, size_t src_bytes, int rows, int cols, void* out,
                     size_t out_bytes, void* stream);

/*
 * Rows of a Q8 weight decoded to fp32: the token-embedding lookup of a tied
 * Q8 embedding / lm_head (NPU engine page, "Q4NX chunks": Q8 chunks hold that
 * tensor, in either code layout).  out[t][k] = d(r, k/32) * code(r, k) with
 * r = ids[t]; every value is exact in fp32.
 *   w    host descriptor of a Q8 weight (E_CHUNK_KIND otherwise)
 *   ids  DEVICE int32 [T]; an id outside [0, w->rows) yields a row of zeros
 *   out  DEVICE fp32 [T][w->cols]
 *   T    1..65535
 */
int q4nx_q8_rows(const q4nx_weight* w, const int32_t* ids, int T, float* out, void* stream);

/*
 * The lm_head GEMV with its greedy / top-k pick in the same launch (NPU
 * engine page, "Q4NX chunks": the Q8 tied embedding / lm_head; onw technical
 * notes, "host work of one step": a decode step ends by picking tokens from
 * the head's logits).  For every activation row m: the k largest of
 * y[m] = W x[m] in decreasing order, the lower row first among equal values
 * (zeros of either sign are equal); NaNs are skipped, and past the last
 * number ids are -1 and vals NaN.  The products are q4nx_gemv's (same bits).
 *   w     any chunk kind; the prepared-activation GEMV must fit it (cols at
 *         most 7168 at M = 4 ... 28672 at M = 1) and the launch must take at
 *         most 4096 workgroups, else E_SHAPE
 *   x     DEVICE bf16 [M][cols], 16-byte aligned;  M 1..4;  k 1..min(16, rows)
 *   y     DEVICE fp32 [M][rows] to receive the logits, or NULL (not written)
 *   ids   DEVICE int32 [M][k];  vals DEVICE fp32 [M][k] or NULL
 *   ws    DEVICE workspace of q4nx_gemv_topk_ws(w, M, k) bytes, 256-byte
 *         aligned, holding zeros before its first use; every call leaves it
 *         ready for the next one; calls that share it must not overlap.
 * Every workgroup picks the top k of its own rows; the last workgroup of each
 * group of 64 merges its group's lists, and the last group merges the groups'
 * (device-scope stores and counters in the workspace).
 */
size_t q4nx_gemv_topk_ws(const q4nx_weight* w, int M, int k);
int q4nx_gemv_topk(const q4nx_weight* w, const uint16_t* x, int M, int k, float* y, int32_t* ids,
                   float* vals, void* ws, size_t ws_bytes, void* stream);

/*
 * Greedy pick over logits already in memory (the same ordering as
 * q4nx_gemv_topk with k = 1; NPU engine page, "Q4NX chunks", the tied Q8
 * lm_head whose logits it reads): for each row m of y (fp32, row stride
 * ldy), the index of the largest of its first n values, the lowest index
 * among equal maxima (zeros of either sign are equal); NaNs are skipped, and
 * a row of only NaNs gives -1.
 *   y    DEVICE fp32, 4-byte aligned; 1 <= n <= ldy, 1 <= M <= 65535
 *   idx  DEVICE int32 [M];  val DEVICE fp32 [M] or NULL (y at the pick)
 *   ws   DEVICE workspace of at least q4nx_argmax_ws(n, M) bytes, 8-byte
 *        aligned, or NULL.  With it each row is cut into slices of 4096
 *        values, one workgroup each, and a second launch combines the slices;
 *        without it one workgroup reads the whole row.  Same result either way.
 *        Nothing in it needs initialising; calls that share it must not overlap.
 */
size_t q4nx_argmax_ws(int n, int M);
int q4nx_argmax(const float* y, int n, int ldy, int M, int32_t* idx, float* val, void* ws,
                size_t ws_bytes, void* stream);

/*
 * MoE router on the device (Strata article, section 2: per token the router
 * picks k = 10 of 512 experts by the softmax of its logits and weights them by
 * those probabilities rescaled to sum to one; section 4.3 "tail skip" keeps
 * them unrescaled).  Produces the ids / p that q4nx_moe_experts takes.
 *   R       DEVICE bf16 [E][D] router weights (row e contiguous), 16-byte aligned
 *   X       DEVICE bf16 [T][D] activations, 16-byte aligned
 *   D       512, 1024, 2048 or 4096 (E_SHAPE otherwise); E 1..1024; k 1..min(16, E)
 *   renorm  nonzero: p rescaled to sum to one over the k picks
 *   ids     DEVICE int32 [T][k]: picks in decreasing logit order, the lower id
 *           first among equal fp32 logits
 *   p       DEVICE fp32 [T][k]: expf(z - max z) / sum, rescaled when renorm
 *   logits  DEVICE fp32 [T][E]: receives the fp32 logits the picks are made on
 * Logits accumulate in fp32 in a fixed order; they must be finite.
 */
int q4nx_moe_router(const uint16_t* R, const uint16_t* X, int T, int D, int E, int k, int renorm,
                    int32_t* ids, float* p, float* logits, void* stream);

/*
 * Test surface of the decoders (NPU engine page, "Q4NX chunks": the decoders
 * of all three kinds are checked bit for bit).  Writes the fields of every
 * chunk in logical [rows][cols] order:
 *   codes    DEVICE u8 [rows][cols]: 4-bit code 0..15, or the int8 code's bits
 *   meta0    DEVICE u16 [rows][cols/32]: q4_1 scale bits | Q4_K scale | Q8 d bits
 *   meta1    DEVICE u16 [rows][cols/32] or NULL: q4_1 zero bits | Q4_K min | 0 for Q8
 *   row_meta DEVICE u16 [rows][cols/256][2] or NULL: Q4_K (S, M) bits | 0 otherwise
 */
int q4nx_unpack(const q4nx_weight* w, uint8_t* codes, uint16_t* meta0, uint16_t* meta1,
                uint16_t* row_meta, void* stream);

/*
 * Decoded weights as fp32 [rows][cols] (DEVICE `out`).  Each value is the
 * exact product-and-sum of the formula rounded once to fp32 (every product in
 * the three formulas is exact in fp32), so the result is bit-exact.
 */
int q4nx_decode(const q4nx_weight* w, float* out, void* stream);

/* Static text for a status code. */
const char* q4nx_status_str(int status);

/* Detail of the last failing call on this thread ("" if none). */
const char* q4nx_last_error(void);

/* Interface version: 100 * major + minor. */
int q4nx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4NX_H */
