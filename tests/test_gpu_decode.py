"""GPU decoders vs the CPU oracle, bit for bit (q4nx_unpack, q4nx_decode)."""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_u8, have_gpu, host, q, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

KINDS = [("q4_1", None), ("q4_k", None), ("q8", "A"), ("q8", "B")]


def _gen(kind, layout, N, K, tag):
    g = synth.rng("gpu-decode", tag, kind, layout or "-", N, K)
    if kind == "q4_1":
        return synth.gen_q4_1(g, N, K, zero="normal")
    if kind == "q4_k":
        return synth.gen_q4_k(g, N, K)
    return synth.gen_q8(g, N, K, layout)


def _unpack_gpu(ch_dev, N, K, kind, layout):
    codes = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    m0 = torch.zeros((N, K // 32), dtype=torch.int16, device="cuda")
    m1 = torch.zeros((N, K // 32), dtype=torch.int16, device="cuda")
    rm = torch.zeros((N, K // 256, 2), dtype=torch.int16, device="cuda")
    q().unpack(weight(ch_dev, N, K, kind, layout), codes, m0, m1, rm)
    return {"codes": host(codes), "meta0": host(m0).view(np.uint16),
            "meta1": host(m1).view(np.uint16), "row_meta": host(rm).view(np.uint16)}


def _decode_gpu(ch_dev, N, K, kind, layout):
    out = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    q().decode(weight(ch_dev, N, K, kind, layout), out)
    return host(out)


@pytest.mark.parametrize("kind,layout", KINDS)
@pytest.mark.parametrize("N,K", [(32, 256), (96, 1280), (160, 768)])
def test_unpack_and_decode_bit_exact(kind, layout, N, K):
    ch = _gen(kind, layout, N, K, "small")
    d = dev_u8(ch)
    got = _unpack_gpu(d, N, K, kind, layout)
    want = oracle.unpack_expected(ch, kind, N, K, layout)
    for name in ("codes", "meta0", "meta1", "row_meta"):
        np.testing.assert_array_equal(got[name], want[name], err_msg=name)
    w = _decode_gpu(d, N, K, kind, layout)
    np.testing.assert_array_equal(w.view(np.uint32), oracle.weights_f32(ch, kind, N, K, layout).view(np.uint32))


@pytest.mark.parametrize("kind,layout", KINDS)
def test_decode_random_bytes_including_subnormal_and_nan_metadata(kind, layout):
    """Every byte random: metadata covers subnormals, huge values, infinities and NaNs."""
    N, K = 64, 512
    g = synth.rng("gpu-decode", "raw", kind, layout or "-")
    ch = np.frombuffer(g.bytes(N // 32 * K // 256 * oracle.KIND_BYTES[kind]), np.uint8).copy()
    d = dev_u8(ch)
    got = _unpack_gpu(d, N, K, kind, layout)
    want = oracle.unpack_expected(ch, kind, N, K, layout)
    for name in ("codes", "meta0", "meta1", "row_meta"):
        np.testing.assert_array_equal(got[name], want[name], err_msg=name)
    w = _decode_gpu(d, N, K, kind, layout)
    with np.errstate(all="ignore"):
        ref = oracle.weights_f32(ch, kind, N, K, layout)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(w), nan)
    np.testing.assert_array_equal(w[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_single_gemv_weight_decodes_bit_exact():
    spec = synth.single_gemv_spec()
    ch = spec.generate()
    w = _decode_gpu(dev_u8(ch), spec.N, spec.K, "q4_1", None)
    np.testing.assert_array_equal(w.view(np.uint32),
                                  oracle.weights_f32(ch, "q4_1", spec.N, spec.K).view(np.uint32))


@pytest.mark.parametrize("kind,layout", [("q4_1", None), ("q8", "A"), ("q8", "B")])
def test_lm_head_sized_decode_sampled_tiles(kind, layout):
    """151936 x 2560 (the 4B lm_head shape): decode all of it, compare sampled tile rows."""
    N, K = 151936, 2560
    spec = (synth.qwen3_4b_decode_specs(0, True)[-1] if kind == "q4_1"
            else synth.mixed_decode_specs(0, layout)[-1])
    ch = spec.generate()
    if kind == "q8" and layout == "B":
        ch = synth.q8_relayout(ch, "A", "B")
    w = _decode_gpu(dev_u8(ch), N, K, kind, layout)
    TR = N // 32
    for tr in [0, 1, 777, TR // 2, TR - 1]:
        ref = oracle.weights_f32(ch[tr:tr + 1], kind, 32, K, layout)
        np.testing.assert_array_equal(w[32 * tr:32 * tr + 32].view(np.uint32), ref.view(np.uint32))
