"""Python binding of libq4nx.so (include/q4nx.h): argument marshalling only.

Every computation runs in the library's HIP kernels.  PyTorch supplies device
memory and streams: tensors are passed by ``data_ptr()`` and work is enqueued
on ``torch.cuda.current_stream()`` unless a stream is given.  When the
library has not been built, importing this package raises ImportError: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# Q4NX_LIB names another build of the same library (the host-sanitised one of
# build.py --sanitize); by default the in-tree libq4nx.so.
LIB_PATH = os.environ.get("Q4NX_LIB") or os.path.join(HERE, "libq4nx.so")

Q4NX_OK, E_ARG, E_CHUNK_KIND, E_SHAPE, E_SHORT, E_ALIGN, E_WORKSPACE, E_Q8_LAYOUT, E_HIP = range(9)
CHUNK_BYTES = {"q4_1": 5120, "q4_k": 4736, "q8": 8704}
Q8_LAYOUT = {None: -1, "A": 0, "B": 1}
GEMV_MAX_M = 8
GEMM_MAX_M = 64
BATCH_MAX_JOBS = 64

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")

_lib = ctypes.CDLL(LIB_PATH)


class Q4nxError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"q4nx status {status}: {detail}")
        self.status = status


class Weight(ctypes.Structure):
    _fields_ = [("chunks", ctypes.c_void_p), ("nbytes", ctypes.c_int64), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("chunk_bytes", ctypes.c_int32),
                ("q8_layout", ctypes.c_int32)]


class GemvJob(ctypes.Structure):
    _fields_ = [("w", Weight), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class GemmJob(ctypes.Structure):
    _fields_ = [("w", Weight), ("Y", ctypes.c_void_p)]


class MoeLayer(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_expert", ctypes.c_int32), ("d_shared", ctypes.c_int32),
                ("chunk_bytes", ctypes.c_int32), ("hot_tokens", ctypes.c_int32),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_stride", ctypes.c_int64), ("up_stride", ctypes.c_int64),
                ("down_stride", ctypes.c_int64), ("gate_bytes", ctypes.c_int64),
                ("up_bytes", ctypes.c_int64), ("down_bytes", ctypes.c_int64),
                ("sh_gate", Weight), ("sh_up", Weight), ("sh_down", Weight)]


class MoeDebug(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("d", ctypes.c_void_p), ("h_shared", ctypes.c_void_p),
                ("d_shared", ctypes.c_void_p)]


class ChunkLayout(ctypes.Structure):
    """q4nx_chunk_layout: where a q4_1 / Q4_K chunk keeps each field (see include/q4nx.h)."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "chunk_bytes", "code_off", "code_row", "code_group", "code_step", "code_pairing",
        "code_high_first", "f0_off", "f0_row", "f0_group", "f1_off", "f1_row", "f1_group",
        "s_off", "s_row", "m_off", "m_row")]


_P = ctypes.c_void_p
_I = ctypes.c_int
_lib.q4nx_weight_check.argtypes = [ctypes.POINTER(Weight)]
_lib.q4nx_gemv.argtypes = [ctypes.POINTER(Weight), _P, _P, _I, _P]
_lib.q4nx_gemv_batched.argtypes = [ctypes.POINTER(GemvJob), _I, _I, _P]
_lib.q4nx_gemm_block.argtypes = [ctypes.POINTER(Weight), _P, _P, _I, _P, ctypes.c_size_t, _P]
_lib.q4nx_gemm_block_ws.argtypes = [ctypes.POINTER(Weight)]
_lib.q4nx_gemm_block_ws.restype = ctypes.c_size_t
_lib.q4nx_plan_set_mode.argtypes = [_P, _I]
_lib.q4nx_gemm_block_noalloc.argtypes = [ctypes.POINTER(Weight), _P, _P, _I, _P]
_lib.q4nx_gemm_block_noalloc_max.argtypes = []
_lib.q4nx_gemm_block_noalloc_max.restype = ctypes.c_size_t
_lib.q4nx_gemm_batched.argtypes = [ctypes.POINTER(GemmJob), _I, _P, _I, _P, ctypes.c_size_t, _P]
_lib.q4nx_gemm_batched_ws.argtypes = [ctypes.POINTER(GemmJob), _I]
_lib.q4nx_gemm_batched_ws.restype = ctypes.c_size_t
_lib.q4nx_gemm_exchange_mode.argtypes = [_I]
_lib.q4nx_chunk_layout_default.argtypes = [_I, ctypes.POINTER(ChunkLayout)]
_lib.q4nx_chunk_layout_check.argtypes = [ctypes.POINTER(ChunkLayout)]
_lib.q4nx_relayout.argtypes = [ctypes.POINTER(ChunkLayout), ctypes.POINTER(Weight), _P, ctypes.c_size_t, _P]
_lib.q4nx_gemv_topk_ws.argtypes = [ctypes.POINTER(Weight), _I, _I]
_lib.q4nx_gemv_topk_ws.restype = ctypes.c_size_t
_lib.q4nx_gemv_topk.argtypes = [ctypes.POINTER(Weight), _P, _I, _I, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.q4nx_moe_ws.argtypes = [ctypes.POINTER(MoeLayer), _I, _I]
_lib.q4nx_moe_ws.restype = ctypes.c_size_t
_lib.q4nx_moe_experts.argtypes = [ctypes.POINTER(MoeLayer), _P, _P, _P, _I, _I, _P,
                                  ctypes.POINTER(MoeDebug), _P, ctypes.c_size_t, _P]
_lib.q4nx_unpack.argtypes = [ctypes.POINTER(Weight), _P, _P, _P, _P, _P]
_lib.q4nx_decode.argtypes = [ctypes.POINTER(Weight), _P, _P]
_lib.q4nx_repack_q4k_to_q41.argtypes = [ctypes.POINTER(Weight), _P, ctypes.c_size_t, _P]
_lib.q4nx_q8_rows.argtypes = [ctypes.POINTER(Weight), _P, _I, _P, _P]
_lib.q4nx_gguf_to_q41.argtypes = [_I, _P, ctypes.c_size_t, _I, _I, _P, ctypes.c_size_t, _P]
_lib.q4nx_gguf_bytes.argtypes = [_I, _I, _I]
_lib.q4nx_gguf_bytes.restype = ctypes.c_size_t
_lib.q4nx_argmax.argtypes = [_P, _I, _I, _I, _P, _P, _P, ctypes.c_size_t, _P]
_lib.q4nx_argmax_ws.argtypes = [_I, _I]
_lib.q4nx_argmax_ws.restype = ctypes.c_size_t
_lib.q4nx_moe_router.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P]
_lib.q4nx_plan_create.argtypes = [ctypes.POINTER(GemvJob), ctypes.POINTER(ctypes.c_int32), _I, _I,
                                  ctypes.POINTER(ctypes.c_void_p)]
_lib.q4nx_plan_run.argtypes = [_P, _P]
_lib.q4nx_plan_errors.argtypes = [_P, ctypes.POINTER(ctypes.c_uint32)]
_lib.q4nx_plan_bytes.argtypes = [_P]
_lib.q4nx_plan_bytes.restype = ctypes.c_size_t
_lib.q4nx_plan_destroy.argtypes = [_P]
_lib.q4nx_plan_destroy.restype = None
_lib.q4nx_status_str.argtypes = [_I]
_lib.q4nx_status_str.restype = ctypes.c_char_p
_lib.q4nx_last_error.restype = ctypes.c_char_p
for _f in ("q4nx_weight_check", "q4nx_gemv", "q4nx_gemv_batched", "q4nx_gemm_block", "q4nx_gemm_batched",
           "q4nx_moe_experts", "q4nx_unpack", "q4nx_decode", "q4nx_repack_q4k_to_q41", "q4nx_gguf_to_q41", "q4nx_q8_rows", "q4nx_argmax", "q4nx_moe_router", "q4nx_version", "q4nx_plan_create",
           "q4nx_plan_run", "q4nx_plan_errors", "q4nx_gemm_exchange_mode", "q4nx_gemv_topk",
           "q4nx_chunk_layout_default", "q4nx_chunk_layout_check", "q4nx_relayout", "q4nx_plan_set_mode",
           "q4nx_gemm_block_noalloc"):
    getattr(_lib, _f).restype = ctypes.c_int


def lib() -> ctypes.CDLL:
    """The loaded library (raw ctypes handle)."""
    return _lib


def last_error() -> str:
    return _lib.q4nx_last_error().decode()


def status_str(status: int) -> str:
    return _lib.q4nx_status_str(status).decode()


def version() -> int:
    return _lib.q4nx_version()


def _check(status: int):
    if status != Q4NX_OK:
        raise Q4nxError(status, last_error())


# ----------------------------------------------------------------------------
# descriptors
# ----------------------------------------------------------------------------
def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    if t is None or isinstance(t, int):
        return 0          # a raw address carries no size: the caller passes it explicitly
    return t.numel() * t.element_size()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def weight(chunks, rows: int, cols: int, kind: str, q8_layout: str | None = None,
           nbytes: int | None = None) -> Weight:
    """Descriptor of a Q4NX weight held in ``chunks`` (a device tensor or a raw address).

    The descriptor keeps a reference to a tensor, so the memory stays allocated
    for as long as the descriptor is alive.
    """
    w = Weight(_ptr(chunks), _nbytes(chunks) if nbytes is None else nbytes, rows, cols,
               CHUNK_BYTES[kind] if isinstance(kind, str) else int(kind),
               Q8_LAYOUT[q8_layout] if q8_layout in Q8_LAYOUT else int(q8_layout))
    if not isinstance(chunks, int) and chunks is not None:
        w._owner = chunks
    return w


def weight_check(w: Weight) -> int:
    """Host-only descriptor check; returns the status code (0 = ok)."""
    return _lib.q4nx_weight_check(ctypes.byref(w))


# ----------------------------------------------------------------------------
# calls
# ----------------------------------------------------------------------------
def gemv(w: Weight, x, y, M: int = 1, stream=None) -> None:
    """y[M, rows] (fp32) = x[M, cols] (bf16) @ W^T."""
    _check(_lib.q4nx_gemv(ctypes.byref(w), _ptr(x), _ptr(y), M, _stream(stream)))


def gemv_batched(jobs, M: int = 1, stream=None) -> None:
    """jobs: sequence of (Weight, x, y); runs them as independent GEMVs."""
    arr = (GemvJob * len(jobs))(*[GemvJob(w, _ptr(x), _ptr(y)) for w, x, y in jobs])
    _check(_lib.q4nx_gemv_batched(arr, len(jobs), M, _stream(stream)))


class Plan:
    """A device-resident GEMV plan (q4nx_plan_*): jobs in phases, one launch per run."""

    def __init__(self, jobs, phases, M: int = 1):
        self._jobs = (GemvJob * len(jobs))(*[GemvJob(w, _ptr(x), _ptr(y)) for w, x, y in jobs])
        self._keep = list(jobs)
        ph = (ctypes.c_int32 * len(jobs))(*phases)
        h = ctypes.c_void_p()
        _check(_lib.q4nx_plan_create(self._jobs, ph, len(jobs), M, ctypes.byref(h)))
        self.handle = h
        self.M = M

    def run(self, stream=None) -> None:
        _check(_lib.q4nx_plan_run(self.handle, _stream(stream)))

    def set_mode(self, mode: int) -> None:
        """0: one launch per phase (default); 1: persistent launches."""
        _check(_lib.q4nx_plan_set_mode(self.handle, mode))

    def errors(self) -> int:
        f = ctypes.c_uint32()
        _check(_lib.q4nx_plan_errors(self.handle, ctypes.byref(f)))
        return f.value

    def nbytes(self) -> int:
        return int(_lib.q4nx_plan_bytes(self.handle))

    def close(self) -> None:
        if self.handle:
            _lib.q4nx_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gemm_block_ws(w: Weight) -> int:
    """Workspace bytes q4nx_gemm_block needs for w (0 = none)."""
    return int(_lib.q4nx_gemm_block_ws(ctypes.byref(w)))


def gemm_block(w: Weight, X, Y, M: int, ws=None, stream=None, ws_bytes: int | None = None) -> None:
    """Y[M, rows] (fp32) = X[M, cols] (bf16) @ W^T for M <= 64.

    ws: a zero-initialised device buffer of gemm_block_ws(w) bytes (reused
    across calls; the library leaves it zeroed), or None when that size is 0.
    """
    _check(_lib.q4nx_gemm_block(ctypes.byref(w), _ptr(X), _ptr(Y), M, _ptr(ws),
                                _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream)))


def gemm_block_noalloc(w: Weight, X, Y, M: int, stream=None) -> None:
    """gemm_block with the library's static workspace: allocates nothing.
    Calls that may overlap on one GPU race (the workspace is shared)."""
    _check(_lib.q4nx_gemm_block_noalloc(ctypes.byref(w), _ptr(X), _ptr(Y), M, _stream(stream)))


def gemm_block_noalloc_max() -> int:
    """Bytes of gemm_block_noalloc's static workspace."""
    return int(_lib.q4nx_gemm_block_noalloc_max())


def gemv_topk_ws(w: Weight, M: int, k: int) -> int:
    """Workspace bytes of gemv_topk (0 = the shape does not fit it)."""
    return int(_lib.q4nx_gemv_topk_ws(ctypes.byref(w), M, k))


def gemv_topk(w: Weight, x, M: int, k: int, ids, ws, y=None, vals=None, stream=None,
              ws_bytes: int | None = None) -> None:
    """ids[M, k] (int32, best first) and optionally vals[M, k] and the logits y[M, rows]
    of y = x @ W^T, in one launch.  ws: zero-initialised, gemv_topk_ws(w, M, k) bytes."""
    _check(_lib.q4nx_gemv_topk(ctypes.byref(w), _ptr(x), M, k, _ptr(y), _ptr(ids), _ptr(vals),
                               _ptr(ws), _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream)))


def chunk_layout_default(kind) -> ChunkLayout:
    """The library's own in-chunk layout of q4_1 (5120) or Q4_K (4736) chunks."""
    L = ChunkLayout()
    _check(_lib.q4nx_chunk_layout_default(CHUNK_BYTES[kind] if isinstance(kind, str) else int(kind),
                                          ctypes.byref(L)))
    return L


def chunk_layout(**fields) -> ChunkLayout:
    """A layout descriptor from its field values (see include/q4nx.h)."""
    return ChunkLayout(**fields)


def chunk_layout_check(L: ChunkLayout) -> int:
    """Host-only check of a layout; returns the status code (0 = valid)."""
    return _lib.q4nx_chunk_layout_check(ctypes.byref(L))


def relayout(L: ChunkLayout, src: Weight, out, stream=None, out_bytes: int | None = None) -> None:
    """Chunks of src (in layout L) -> the same weight in the library's layout, into out."""
    _check(_lib.q4nx_relayout(ctypes.byref(L), ctypes.byref(src), _ptr(out),
                              _nbytes(out) if out_bytes is None else out_bytes, _stream(stream)))


def gemm_exchange_mode(mode: int) -> None:
    """Split-K exchange of every later block GEMM: 0 default, 1 odd groups act
    displaced (tests), 2 device-coherent exchange (tests)."""
    _check(_lib.q4nx_gemm_exchange_mode(mode))


GEMM_WS_DIAG_OFFSET = 3072   # uint32 in the GEMM workspace: workgroups that found their XCD slot taken


def _gemm_jobs(jobs):
    return (GemmJob * len(jobs))(*[GemmJob(w, _ptr(Y)) for w, Y in jobs])


def gemm_batched_ws(jobs) -> int:
    """Workspace bytes q4nx_gemm_batched needs for jobs = [(Weight, Y), ...] (0 = none)."""
    return int(_lib.q4nx_gemm_batched_ws(_gemm_jobs(jobs), len(jobs)))


def gemm_batched(jobs, X, M: int, ws=None, stream=None, ws_bytes: int | None = None) -> None:
    """Y_j = X @ W_j^T for jobs = [(Weight, Y_j), ...] sharing X (same kind and cols)."""
    _check(_lib.q4nx_gemm_batched(_gemm_jobs(jobs), len(jobs), _ptr(X), M, _ptr(ws),
                                  _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream)))


def moe_layer(n_experts: int, d_model: int, d_expert: int, kind: str, gate, up, down,
              gate_stride: int, up_stride: int, down_stride: int,
              shared=None, d_shared: int = 0, gate_bytes=None, up_bytes=None,
              down_bytes=None, hot_tokens: int = 0) -> MoeLayer:
    """MoE layer descriptor.  ``shared`` = (Weight gate, Weight up, Weight down) or None."""
    L = MoeLayer()
    L.n_experts, L.d_model, L.d_expert = n_experts, d_model, d_expert
    L.d_shared = d_shared if shared is not None else 0
    L.chunk_bytes = CHUNK_BYTES[kind]
    L.hot_tokens = hot_tokens
    L.gate, L.up, L.down = _ptr(gate), _ptr(up), _ptr(down)
    L.gate_stride, L.up_stride, L.down_stride = gate_stride, up_stride, down_stride
    L.gate_bytes = _nbytes(gate) if gate_bytes is None else gate_bytes
    L.up_bytes = _nbytes(up) if up_bytes is None else up_bytes
    L.down_bytes = _nbytes(down) if down_bytes is None else down_bytes
    if shared is not None:
        L.sh_gate, L.sh_up, L.sh_down = shared
    L._owners = (gate, up, down, shared)
    return L


def moe_ws(L: MoeLayer, T: int, k: int) -> int:
    return int(_lib.q4nx_moe_ws(ctypes.byref(L), T, k))


def moe_experts(L: MoeLayer, X, ids, p, Y, T: int, k: int, ws, dbg: dict | None = None,
                stream=None, ws_bytes: int | None = None) -> None:
    """Y[T, D] = MoE layer of X[T, D] with routing ids[T, k] / p[T, k]; ws from moe_ws()."""
    d = None
    if dbg:
        d = MoeDebug(_ptr(dbg.get("h")), _ptr(dbg.get("d")), _ptr(dbg.get("h_shared")),
                     _ptr(dbg.get("d_shared")))
    _check(_lib.q4nx_moe_experts(ctypes.byref(L), _ptr(X), _ptr(ids), _ptr(p), T, k, _ptr(Y),
                                 ctypes.byref(d) if d is not None else None, _ptr(ws),
                                 _nbytes(ws) if ws_bytes is None else ws_bytes,
                                 _stream(stream)))


GGUF_Q4_0, GGUF_Q4_1, GGUF_Q4_K = 2, 3, 12


def gguf_bytes(gguf_type: int, rows: int, cols: int) -> int:
    """Bytes of a rows x cols GGUF tensor of that type (0 if the type or cols is invalid)."""
    return int(_lib.q4nx_gguf_bytes(gguf_type, rows, cols))


def gguf_to_q41(gguf_type: int, src, rows: int, cols: int, out, stream=None,
                src_bytes: int | None = None, out_bytes: int | None = None) -> None:
    """GGUF Q4_0 / Q4_1 / Q4_K tensor bytes (device) -> q4_1 chunks in `out`."""
    _check(_lib.q4nx_gguf_to_q41(gguf_type, _ptr(src), _nbytes(src) if src_bytes is None else src_bytes,
                                 rows, cols, _ptr(out), _nbytes(out) if out_bytes is None else out_bytes,
                                 _stream(stream)))


def repack_q4k_to_q41(w: Weight, out, stream=None, out_bytes: int | None = None) -> None:
    """Q4_K weight -> q4_1 chunks in `out` (tiles * 5120 bytes), same tile order."""
    _check(_lib.q4nx_repack_q4k_to_q41(ctypes.byref(w), _ptr(out),
                                       _nbytes(out) if out_bytes is None else out_bytes,
                                       _stream(stream)))


def q8_rows(w: Weight, ids, T: int, out, stream=None) -> None:
    """out[t] = decoded row ids[t] of the Q8 weight w (fp32 [T][cols])."""
    _check(_lib.q4nx_q8_rows(ctypes.byref(w), _ptr(ids), T, _ptr(out), _stream(stream)))


def argmax_ws(n: int, M: int) -> int:
    return _lib.q4nx_argmax_ws(n, M)


def argmax(y, n: int, M: int, idx, val=None, ldy: int | None = None, ws=None, stream=None,
           ws_bytes: int | None = None) -> None:
    """idx[m] = index of the largest of y[m][:n] (lowest on ties, NaNs skipped);
    with a workspace (argmax_ws bytes) the rows are split over many workgroups."""
    _check(_lib.q4nx_argmax(_ptr(y), n, n if ldy is None else ldy, M, _ptr(idx), _ptr(val), _ptr(ws),
                            (_nbytes(ws) if ws is not None else 0) if ws_bytes is None else ws_bytes,
                            _stream(stream)))


def moe_router(R, X, T: int, D: int, E: int, k: int, ids, p, logits, renorm: bool = True,
               stream=None) -> None:
    """Router on the device: ids [T][k] int32, p [T][k] fp32 (and the fp32 logits [T][E]
    they are picked from) from bf16 R [E][D] and X [T][D]."""
    _check(_lib.q4nx_moe_router(_ptr(R), _ptr(X), T, D, E, k, 1 if renorm else 0, _ptr(ids),
                                _ptr(p), _ptr(logits), _stream(stream)))


def unpack(w: Weight, codes, meta0, meta1=None, row_meta=None, stream=None) -> None:
    _check(_lib.q4nx_unpack(ctypes.byref(w), _ptr(codes), _ptr(meta0), _ptr(meta1),
                            _ptr(row_meta), _stream(stream)))


def decode(w: Weight, out, stream=None) -> None:
    _check(_lib.q4nx_decode(ctypes.byref(w), _ptr(out), _stream(stream)))
