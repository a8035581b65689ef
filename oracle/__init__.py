"""CPU oracle for the Q4NX dequant-GEMV / block-GEMM / MoE path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package; the
library's own path never does, and it shares no code, table or constant with
the HIP kernels.  It is plain, slow and written to be checked by eye:

* ``decode``  -- chunk bytes -> logical fields -> exact weights (float64), plus
  a pure-Python scalar decoder used as brute force on tiny grids, and the same
  decode for chunks in another described in-chunk layout;
* ``ref``     -- float64 products y = W x with the per-output error scale
  a = sum |w x|, the tolerance test, SwiGLU, the MoE layer and its combine,
  the router (logits, softmax, top-k, renormalisation), the greedy / top-k
  pick from the head's logits, and the Q4_K -> q4_1 repack with its rounding
  bound;
* ``gguf``    -- GGUF Q4_0 / Q4_1 / Q4_K blocks decoded from their own
  definition, and the q4_1 fields the GGUF -> q4_1 conversion must give.

What it follows: the 1bit engine docs, page "NPU engine", section "Q4NX chunks"
(tile grid, chunk kinds, decode formulas, the two Q8 code layouts) and the
project's written chunk layout for the parts that page leaves to an unpublished
header (listed in each function that depends on them); for the GGUF
conversion, the same page's section "From a GGUF" and the public GGUF block
types (ggml's block_q4_0, block_q4_1, block_q4_K).

Parity unpinned: that in-chunk byte order of the q4_1 / Q4_K codes and of the
q4_1, Q4_K and Q8 metadata, against real model files (no header or real tile
is available to compare with), and the GGUF block layouts against a real GGUF
file (none is available; hand-worked blocks pin the reading instead).  Everything else here is pinned by tests that
do not reuse this code's formulas (tests/test_oracle_pins.py).
"""
from .decode import (KIND_BYTES, decode_fields, weights_exact, weights_f32, unpack_expected,
                     scalar_decode_chunk, default_layout, decode_fields_layout, weights_exact_layout)
from .ref import (gemv_ref, check_tol, tol_ratio, silu, swiglu, moe_layer_ref, moe_combine_ref,
                  repack_q4k_to_q41, repack_bound, router_topk, router_logits_ref, head_topk)
from .gguf import (GGUF_Q4_0, GGUF_Q4_1, GGUF_Q4_K, gguf_bytes, gguf_fields, gguf_dequant,
                   gguf_to_q41, gguf_to_q41_bound)

__all__ = [
    "KIND_BYTES", "decode_fields", "weights_exact", "weights_f32", "unpack_expected",
    "default_layout", "decode_fields_layout", "weights_exact_layout",
    "scalar_decode_chunk", "gemv_ref", "check_tol", "tol_ratio", "silu", "swiglu",
    "moe_layer_ref", "moe_combine_ref", "repack_q4k_to_q41", "repack_bound", "router_topk",
    "router_logits_ref", "head_topk", "GGUF_Q4_0", "GGUF_Q4_1", "GGUF_Q4_K", "gguf_bytes", "gguf_fields",
    "gguf_dequant", "gguf_to_q41", "gguf_to_q41_bound",
]
