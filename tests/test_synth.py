"""The seeded input generator: determinism, distributions and router properties."""
import numpy as np

import oracle
import synth


def test_same_key_same_bytes_and_different_keys_differ():
    a = synth.gen_q4_1(synth.rng("t", 1), 64, 512)
    b = synth.gen_q4_1(synth.rng("t", 1), 64, 512)
    c = synth.gen_q4_1(synth.rng("t", 2), 64, 512)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_q4_1_distributions():
    ch = synth.gen_q4_1(synth.rng("t", "dist"), 256, 1024, zero="minus8")
    f = oracle.decode_fields(ch, "q4_1", 256, 1024)
    counts = np.bincount(f["codes"].ravel(), minlength=16)
    assert counts.min() > 0.9 * counts.mean() and counts.max() < 1.1 * counts.mean()
    s = (f["scale"].astype(np.uint32) << 16).view(np.float32)
    z = (f["zero"].astype(np.uint32) << 16).view(np.float32)
    assert np.all(s >= 0) and abs(s.mean() - 0.02 * np.sqrt(2 / np.pi)) < 1e-3
    np.testing.assert_array_equal(z, -8 * s)


def test_q4_1_normal_zero_is_near_minus8_scale():
    ch = synth.gen_q4_1(synth.rng("t", "zn"), 128, 1024, zero="normal")
    f = oracle.decode_fields(ch, "q4_1", 128, 1024)
    s = (f["scale"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    z = (f["zero"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ok = s > 1e-4
    ratio = z[ok] / s[ok]
    assert abs(ratio.mean() + 8) < 0.02 and 0.08 < ratio.std() < 0.12


def test_q4_k_and_q8_ranges():
    f = oracle.decode_fields(synth.gen_q4_k(synth.rng("t", "k"), 64, 512), "q4_k", 64, 512)
    assert f["sc"].max() <= 63 and f["mn"].max() <= 63
    f8 = oracle.decode_fields(synth.gen_q8(synth.rng("t", "8"), 64, 512, "B"), "q8", 64, 512, "B")
    assert f8["codes"].min() >= -127 and f8["codes"].max() <= 127


def test_router_properties():
    ids, w = synth.gen_router(synth.rng("t", "router"), 4096, 512, 10, 1.1)
    assert ids.shape == (4096, 10) and w.dtype == np.float32
    assert all(len(set(row)) == 10 for row in ids.tolist())
    assert np.all((ids >= 0) & (ids < 512))
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)              # ordered by probability
    freq = np.bincount(ids.ravel(), minlength=512)
    top = np.sort(freq)[::-1]
    assert top[0] > 20 * max(1, top[255])               # skewed popularity


def test_union_of_a_64_token_block_is_a_few_hundred_experts():
    sizes = [len(np.unique(synth.moe_router(l, 64)[0])) for l in range(8)]
    assert 150 < np.mean(sizes) < 260
