"""The C ABI without a GPU: the library loads, exports what include/q4nx.h
declares, and every host-side check returns its status before anything is
enqueued (no call here reaches the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gemm_q4nx_chunk_amd", "libq4nx.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


@pytest.fixture(scope="module")
def q():
    import gemm_q4nx_chunk_amd as mod
    return mod


def _declared():
    text = open(os.path.join(ROOT, "include", "q4nx.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4nx_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(q):
    names = _declared()
    assert len(names) >= 11
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(q):
    assert q.version() == 100
    for s in range(9):
        assert q.status_str(s) and q.status_str(s) != "unknown status"
    assert q.status_str(99) == "unknown status"


def _w(q, rows=64, cols=512, kind="q4_1", layout=None, nbytes=None, ptr=0x100000):
    cb = q.CHUNK_BYTES[kind] if isinstance(kind, str) else kind
    need = (rows // 32) * (cols // 256) * cb if rows > 0 and cols > 0 else 0
    return q.weight(ptr, rows, cols, kind, layout, nbytes=need if nbytes is None else nbytes)


def test_weight_check_rules(q):
    assert q.weight_check(_w(q)) == q.Q4NX_OK and q.last_error() == ""
    assert q.weight_check(_w(q, kind="q4_k")) == q.Q4NX_OK
    assert q.weight_check(_w(q, kind="q8", layout="A")) == q.Q4NX_OK
    assert q.weight_check(_w(q, kind="q8", layout="B")) == q.Q4NX_OK
    assert q.weight_check(_w(q, ptr=0)) == q.E_ARG
    assert q.weight_check(_w(q, kind=5000, nbytes=10 ** 6)) == q.E_CHUNK_KIND
    assert "5000" in q.last_error()
    assert q.weight_check(_w(q, kind="q8", layout=None)) == q.E_Q8_LAYOUT
    assert q.weight_check(_w(q, rows=48, nbytes=10 ** 6)) == q.E_SHAPE
    assert q.weight_check(_w(q, cols=300, nbytes=10 ** 6)) == q.E_SHAPE
    assert q.weight_check(_w(q, rows=0, nbytes=10 ** 6)) == q.E_SHAPE
    assert q.weight_check(_w(q, nbytes=2 * 2 * 5120 - 1)) == q.E_SHORT
    assert q.weight_check(_w(q, ptr=0x100008)) == q.E_ALIGN
    assert q.weight_check(_w(q)) == q.Q4NX_OK and q.last_error() == ""


def test_null_descriptor(q):
    assert q.lib().q4nx_weight_check(None) == q.E_ARG


def _expect(q, status, fn, *a, **k):
    with pytest.raises(q.Q4nxError) as e:
        fn(*a, **k)
    assert e.value.status == status, str(e.value)


def test_gemv_argument_checks(q):
    w = _w(q)
    _expect(q, q.E_ARG, q.gemv, w, 0x2000, 0x3000, M=0, stream=0)
    _expect(q, q.E_ARG, q.gemv, w, 0x2000, 0x3000, M=9, stream=0)
    _expect(q, q.E_ARG, q.gemv, w, 0, 0x3000, M=1, stream=0)
    _expect(q, q.E_ALIGN, q.gemv, w, 0x2008, 0x3000, M=1, stream=0)
    _expect(q, q.E_ALIGN, q.gemv, w, 0x2000, 0x3002, M=1, stream=0)
    _expect(q, q.E_Q8_LAYOUT, q.gemv, _w(q, kind="q8"), 0x2000, 0x3000, M=1, stream=0)
    _expect(q, q.E_SHORT, q.gemv, _w(q, nbytes=100), 0x2000, 0x3000, M=1, stream=0)


def test_gemv_batched_checks_every_job_first(q):
    good = (_w(q), 0x2000, 0x3000)
    bad = (_w(q, kind=1234, nbytes=10 ** 6), 0x2000, 0x3000)
    _expect(q, q.E_CHUNK_KIND, q.gemv_batched, [good, good, bad], M=1, stream=0)
    assert "job 2" in q.last_error()
    arr = (q.GemvJob * 1)()
    assert q.lib().q4nx_gemv_batched(arr, 0, 1, None) == q.E_ARG
    assert q.lib().q4nx_gemv_batched(arr, q.BATCH_MAX_JOBS + 1, 1, None) == q.E_ARG


def test_gemm_block_checks(q):
    _expect(q, q.E_CHUNK_KIND, q.gemm_block, _w(q, kind="q8", layout="A"), 0x2000, 0x3000, 4, stream=0)
    _expect(q, q.E_ARG, q.gemm_block, _w(q), 0x2000, 0x3000, 65, stream=0)
    _expect(q, q.E_ARG, q.gemm_block, _w(q), 0x2000, 0x3000, 0, stream=0)
    _expect(q, q.E_ALIGN, q.gemm_block, _w(q), 0x2004, 0x3000, 8, stream=0)
    big = _w(q, rows=1024, cols=8192)
    need = q.gemm_block_ws(big)
    assert need > 0 and q.gemm_block_ws(_w(q, rows=14336, cols=4096)) > 0
    _expect(q, q.E_WORKSPACE, q.gemm_block, big, 0x2000, 0x3000, 64, stream=0)
    _expect(q, q.E_WORKSPACE, q.gemm_block, big, 0x2000, 0x3000, 64, ws=0x100000, ws_bytes=need - 1, stream=0)
    _expect(q, q.E_ALIGN, q.gemm_block, big, 0x2000, 0x3000, 64, ws=0x100010, ws_bytes=need, stream=0)


def test_gemm_batched_checks(q):
    a, b = _w(q, rows=1024, cols=4096), _w(q, rows=4096, cols=4096)
    jobs = [(a, 0x3000), (b, 0x4000)]
    need = q.gemm_batched_ws(jobs)
    # one workgroup row per 8 tile rows of each weight, K split over parts
    assert need == q.gemm_batched_ws([(b, 0x4000), (a, 0x3000)]) and need > 0
    _expect(q, q.E_SHAPE, q.gemm_batched, [(a, 0x3000), (_w(q, rows=1024, cols=2048), 0x4000)],
            0x2000, 64, stream=0)
    _expect(q, q.E_SHAPE, q.gemm_batched, [(a, 0x3000), (_w(q, kind="q4_k", rows=1024, cols=4096), 0x4000)],
            0x2000, 64, stream=0)
    _expect(q, q.E_CHUNK_KIND, q.gemm_batched, [(a, 0x3000), (_w(q, kind="q8", layout="A"), 0x4000)],
            0x2000, 64, stream=0)
    _expect(q, q.E_ARG, q.gemm_batched, [(a, 0x3000)] * 9, 0x2000, 64, stream=0)
    _expect(q, q.E_ARG, q.gemm_batched, [(a, 0)], 0x2000, 64, stream=0)
    _expect(q, q.E_ALIGN, q.gemm_batched, [(a, 0x3002)], 0x2000, 64, stream=0)
    _expect(q, q.E_WORKSPACE, q.gemm_batched, jobs, 0x2000, 64, ws=0x100000, ws_bytes=need - 1, stream=0)
    _expect(q, q.E_ALIGN, q.gemm_batched, jobs, 0x2000, 64, ws=0x100010, ws_bytes=need, stream=0)


def _layer(q, **over):
    D, De, Ds, n = 2048, 512, 1024, 512
    gu = (De // 32) * (D // 256) * 5120
    dn = (D // 32) * (De // 256) * 5120
    sh = (q.weight(0x200000, Ds, D, "q4_1"), q.weight(0x300000, Ds, D, "q4_1"),
          q.weight(0x400000, D, Ds, "q4_1"))
    for w in sh:
        w.nbytes = (w.rows // 32) * (w.cols // 256) * 5120
    args = dict(n_experts=n, d_model=D, d_expert=De, kind="q4_1", gate=0x10000000,
                up=0x20000000, down=0x30000000, gate_stride=gu, up_stride=gu, down_stride=dn,
                shared=sh, d_shared=Ds, gate_bytes=n * gu, up_bytes=n * gu, down_bytes=n * dn)
    args.update(over)
    return q.moe_layer(**args)


def test_moe_workspace_size_and_checks(q):
    L = _layer(q)
    ws1 = q.moe_ws(L, 1, 10)
    ws64 = q.moe_ws(L, 64, 10)
    assert 0 < ws1 < ws64
    # the fp32 down outputs alone need (T*k + T) * D * 4 bytes
    assert ws64 >= (640 + 64) * 2048 * 4
    assert q.moe_ws(L, 0, 10) == 0 and q.moe_ws(L, 512, 10) == 0 and q.moe_ws(L, 4, 17) == 0
    assert q.moe_ws(_layer(q, kind="q8"), 1, 10) == 0

    def call(L, T=1, k=10, ws=0x40000000, ws_bytes=None):
        return q.lib().q4nx_moe_experts(ctypes.byref(L), 0x1000, 0x2000, 0x3000, T, k, 0x4000,
                                        None, ws, ws1 if ws_bytes is None else ws_bytes, None)
    assert call(L, ws_bytes=ws1 - 1) == q.E_WORKSPACE
    assert call(L, ws=0) == q.E_WORKSPACE
    assert call(L, ws=0x40000010) == q.E_ALIGN
    assert call(L, T=0) == q.E_ARG
    assert call(L, T=4096, k=2) == q.E_ARG
    assert call(_layer(q, kind="q8")) == q.E_CHUNK_KIND
    assert call(_layer(q, d_expert=500)) == q.E_SHAPE
    assert call(_layer(q, gate_bytes=100)) == q.E_SHORT
    assert call(_layer(q, gate_stride=1000)) == q.E_ALIGN
    assert call(_layer(q, gate=0)) == q.E_ARG
    L3 = _layer(q)
    L3.sh_down.rows = 1024
    assert call(L3) in (q.E_SHAPE, q.E_SHORT)
    L4 = _layer(q)
    L4.n_experts = 0
    assert call(L4) == q.E_ARG


def test_unpack_decode_checks(q):
    _expect(q, q.E_ARG, q.unpack, _w(q), 0, 0x2000, stream=0)
    _expect(q, q.E_ALIGN, q.unpack, _w(q), 0x1000, 0x2001, stream=0)
    _expect(q, q.E_ARG, q.decode, _w(q), 0, stream=0)
    _expect(q, q.E_ALIGN, q.decode, _w(q), 0x1002, stream=0)


def test_repack_checks(q):
    wk = _w(q, rows=64, cols=512, kind="q4_k")
    need = 2 * 2 * 5120
    _expect(q, q.E_CHUNK_KIND, q.repack_q4k_to_q41, _w(q), 0x200000, stream=0, out_bytes=need)
    _expect(q, q.E_ARG, q.repack_q4k_to_q41, wk, 0, stream=0, out_bytes=need)
    _expect(q, q.E_ALIGN, q.repack_q4k_to_q41, wk, 0x200008, stream=0, out_bytes=need)
    _expect(q, q.E_SHORT, q.repack_q4k_to_q41, wk, 0x200000, stream=0, out_bytes=need - 1)


def test_gguf_sizes_and_checks(q):
    assert q.gguf_bytes(q.GGUF_Q4_0, 64, 512) == 64 * 16 * 18
    assert q.gguf_bytes(q.GGUF_Q4_1, 64, 512) == 64 * 16 * 20
    assert q.gguf_bytes(q.GGUF_Q4_K, 64, 512) == 64 * 2 * 144
    assert q.gguf_bytes(q.GGUF_Q4_K, 64, 500) == 0 and q.gguf_bytes(8, 64, 512) == 0
    need_out = 2 * 2 * 5120
    for t, al in ((q.GGUF_Q4_0, 2), (q.GGUF_Q4_1, 4), (q.GGUF_Q4_K, 16)):
        n = q.gguf_bytes(t, 64, 512)
        ok = dict(stream=0, src_bytes=n, out_bytes=need_out)
        _expect(q, q.E_ARG, q.gguf_to_q41, 6, 0x100000, 64, 512, 0x200000, **ok)       # Q5_0: not taken
        _expect(q, q.E_ARG, q.gguf_to_q41, t, 0, 64, 512, 0x200000, **ok)
        _expect(q, q.E_ARG, q.gguf_to_q41, t, 0x100000, 64, 512, 0, **ok)
        _expect(q, q.E_SHAPE, q.gguf_to_q41, t, 0x100000, 48, 512, 0x200000, **ok)
        _expect(q, q.E_SHAPE, q.gguf_to_q41, t, 0x100000, 64, 384, 0x200000, **ok)
        _expect(q, q.E_ALIGN, q.gguf_to_q41, t, 0x100000 + al // 2, 64, 512, 0x200000, **ok)
        _expect(q, q.E_ALIGN, q.gguf_to_q41, t, 0x100000, 64, 512, 0x200004, **ok)
        _expect(q, q.E_SHORT, q.gguf_to_q41, t, 0x100000, 64, 512, 0x200000, stream=0,
                src_bytes=n - 1, out_bytes=need_out)
        _expect(q, q.E_SHORT, q.gguf_to_q41, t, 0x100000, 64, 512, 0x200000, stream=0,
                src_bytes=n, out_bytes=need_out - 1)


def test_rows_and_argmax_checks(q):
    w8 = _w(q, kind="q8", layout="A")
    _expect(q, q.E_CHUNK_KIND, q.q8_rows, _w(q), 0x2000, 4, 0x3000, stream=0)
    _expect(q, q.E_ARG, q.q8_rows, w8, 0, 4, 0x3000, stream=0)
    _expect(q, q.E_ARG, q.q8_rows, w8, 0x2000, 0, 0x3000, stream=0)
    _expect(q, q.E_ALIGN, q.q8_rows, w8, 0x2002, 4, 0x3000, stream=0)
    _expect(q, q.E_ARG, q.argmax, 0, 10, 1, 0x3000, stream=0)
    _expect(q, q.E_ARG, q.argmax, 0x2000, 10, 1, 0x3000, ldy=9, stream=0)
    _expect(q, q.E_ARG, q.argmax, 0x2000, 10, 0, 0x3000, stream=0)
    _expect(q, q.E_ALIGN, q.argmax, 0x2002, 10, 1, 0x3000, stream=0)
    # split form: one 8-byte key per 4096-value slice per row
    assert q.argmax_ws(151936, 1) == 38 * 8
    assert q.argmax_ws(4096, 3) == 3 * 8 and q.argmax_ws(4097, 3) == 6 * 8
    assert q.argmax_ws(0, 1) == 0 and q.argmax_ws(10, 0) == 0
    _expect(q, q.E_WORKSPACE, q.argmax, 0x2000, 5000, 1, 0x3000, ws=0x4000, ws_bytes=15, stream=0)
    _expect(q, q.E_ALIGN, q.argmax, 0x2000, 5000, 1, 0x3000, ws=0x4004, ws_bytes=16, stream=0)


def test_router_checks(q):
    ok = dict(stream=0)
    _expect(q, q.E_ARG, q.moe_router, 0, 0x2000, 1, 2048, 512, 10, 0x3000, 0x4000, 0x5000, **ok)
    _expect(q, q.E_SHAPE, q.moe_router, 0x1000, 0x2000, 1, 2000, 512, 10, 0x3000, 0x4000, 0x5000, **ok)
    _expect(q, q.E_ARG, q.moe_router, 0x1000, 0x2000, 1, 2048, 2000, 10, 0x3000, 0x4000, 0x5000, **ok)
    _expect(q, q.E_ARG, q.moe_router, 0x1000, 0x2000, 1, 2048, 8, 10, 0x3000, 0x4000, 0x5000, **ok)
    _expect(q, q.E_ARG, q.moe_router, 0x1000, 0x2000, 0, 2048, 512, 10, 0x3000, 0x4000, 0x5000, **ok)
    _expect(q, q.E_ALIGN, q.moe_router, 0x1008, 0x2000, 1, 2048, 512, 10, 0x3000, 0x4000, 0x5000, **ok)
    _expect(q, q.E_ARG, q.moe_router, 0x1000, 0x2000, 1, 2048, 512, 10, 0x3000, 0x4000, None, **ok)


def test_plan_create_checks(q):
    good = (_w(q), 0x2000, 0x3000)
    lib = q.lib()

    def create(jobs, phases, M=1):
        arr = (q.GemvJob * len(jobs))(*[q.GemvJob(w, x, y) for w, x, y in jobs])
        ph = (ctypes.c_int32 * len(phases))(*phases)
        h = ctypes.c_void_p()
        return lib.q4nx_plan_create(arr, ph, len(jobs), M, ctypes.byref(h)), h
    assert create([good], [0], M=5)[0] == q.E_ARG
    assert create([good], [0], M=0)[0] == q.E_ARG
    assert create([good], [-1])[0] == q.E_ARG
    assert create([good, (_w(q, kind="q8", layout="A"), 0x2000, 0x3000)], [0, 0])[0] == q.E_CHUNK_KIND
    assert "mixes" in q.last_error()
    assert create([good, (_w(q, kind=77, nbytes=10 ** 6), 0x2000, 0x3000)], [0, 1])[0] == q.E_CHUNK_KIND
    assert lib.q4nx_plan_create(None, None, 0, 1, None) == q.E_ARG
    assert lib.q4nx_plan_run(None, None) == q.E_ARG
    assert lib.q4nx_plan_set_mode(None, 0) == q.E_ARG
    assert q.lib().q4nx_plan_bytes(None) == 0
    lib.q4nx_plan_destroy(None)


def test_descriptor_keeps_its_tensor_alive(q):
    torch = pytest.importorskip("torch")
    t = torch.zeros(2 * 2 * 5120, dtype=torch.uint8)
    w = q.weight(t, 64, 512, "q4_1")
    assert w._owner is t and q.weight_check(w) == q.Q4NX_OK


def test_chunk_layout_default_and_check(q):
    """The library's own layout passes its check; layouts that leave the chunk
    or overlap are refused with E_ARG (the fields' sizes add up to the chunk
    size, so no valid layout leaves a byte unused), other chunk sizes with
    E_CHUNK_KIND; relayout refuses before launching."""
    for kind in ("q4_1", "q4_k"):
        L = q.chunk_layout_default(kind)
        assert q.chunk_layout_check(L) == 0
    with pytest.raises(q.Q4nxError) as e:
        q.chunk_layout_default(8704)
    assert e.value.status == 2
    blocks = dict(chunk_bytes=5120, code_off=4, code_row=160, code_group=20, code_step=1, code_pairing=1,
                  code_high_first=0, f0_off=0, f0_row=160, f0_group=20, f1_off=2, f1_row=160, f1_group=20)
    assert q.chunk_layout_check(q.chunk_layout(**blocks)) == 0
    bad = [dict(blocks, f1_off=1),                 # zero overlaps the scale
           dict(blocks, code_off=5),               # codes leave the chunk
           dict(blocks, code_step=2),              # overlaps and leaves the chunk
           dict(blocks, code_pairing=2),           # not a pairing
           dict(blocks, chunk_bytes=4736)]         # a Q4_K chunk described with q4_1 records
    for b in bad:
        assert q.chunk_layout_check(q.chunk_layout(**b)) in (1, 2), b
    assert q.chunk_layout_check(q.chunk_layout(**dict(blocks, chunk_bytes=8704))) == 2
    w = _w(q, 64, 512, "q4_1")
    with pytest.raises(q.Q4nxError) as e:
        q.relayout(q.chunk_layout(**dict(blocks, f1_off=1)), w, 0x200000, stream=0, out_bytes=1 << 20)
    assert e.value.status == 1
    with pytest.raises(q.Q4nxError) as e:
        q.relayout(q.chunk_layout(**blocks), w, 0x200000, stream=0, out_bytes=100)
    assert e.value.status == 4
    with pytest.raises(q.Q4nxError) as e:
        q.relayout(q.chunk_layout_default("q4_k"), w, 0x200000, stream=0, out_bytes=1 << 20)
    assert e.value.status == 2
