"""GEMV plans (q4nx_plan_*): a decode step's dependent phases in one launch.

Checked in both modes (0: one launch per phase over the plan's device job
table; 1: persistent launches): every output against the float64 oracle; a
real dependency (phase 1 reads, as its activations, the bytes phase 0 writes);
repeated runs and HIP graph replays (the counters reset themselves); several
chunk kinds; no wait ever times out; a phase of more jobs than one batched
call takes, in one launch.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import dev_bf16, dev_u8, have_gpu, host, q, torch, weight

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _gen(kind, N, K, tag, layout=None):
    g = synth.rng("gpu-plan", tag, kind, N, K)
    if kind == "q4_1":
        return synth.gen_q4_1(g, N, K, zero="normal")
    if kind == "q4_k":
        return synth.gen_q4_k(g, N, K)
    return synth.gen_q8(g, N, K, layout)


class Job:
    def __init__(self, kind, N, K, tag, M, layout=None, x=None):
        self.kind, self.N, self.K, self.layout, self.M = kind, N, K, layout, M
        self.ch = _gen(kind, N, K, tag, layout)
        self.dw = dev_u8(self.ch)
        self.xb = synth.gen_x(synth.rng("gpu-plan", "x", tag), M, K) if x is None else x
        self.dx = dev_bf16(self.xb)
        self.dy = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        self.w = weight(self.dw, N, K, kind, layout)

    def job(self):
        return (self.w, self.dx, self.dy)

    def check(self):
        y = host(self.dy)
        yr, a = oracle.gemv_ref(oracle.weights_exact(self.ch, self.kind, self.N, self.K, self.layout), self.xb)
        r = oracle.tol_ratio(y, yr, a)
        assert r <= 1.0, (self.kind, self.N, self.K, r)
        return y


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M", [1, 2, 4])
def test_plan_matches_oracle_and_repeats(M, mode):
    jobs = [Job("q4_1", 4096, 2560, "q", M), Job("q4_1", 1024, 2560, "k", M),
            Job("q4_1", 2560, 4096, "o", M), Job("q4_1", 1920, 9728, "down", M),
            Job("q4_1", 32, 256, "tiny", M), Job("q4_1", 8192, 2560, "big", M)]
    phases = [0, 0, 1, 2, 2, 3]
    plan = q().Plan([j.job() for j in jobs], phases, M)
    plan.set_mode(mode)
    outs = []
    for _ in range(3):
        for j in jobs:
            j.dy.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        outs.append([j.check() for j in jobs])
    assert plan.errors() == 0
    for run in outs[1:]:
        for a, b in zip(run, outs[0]):
            np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    plan.close()


@pytest.mark.parametrize("mode", [0, 1])
def test_plan_honours_the_phase_dependency(mode):
    """Phase 1's activations are the bytes phase 0 writes (bf16-exact outputs by construction)."""
    M, N0, K0 = 2, 4096, 2560
    g = synth.rng("gpu-plan", "dep")
    codes = g.integers(0, 16, (N0, K0), dtype=np.uint8)
    exps = g.integers(-9, -3, (N0, K0 // 32))
    s_bits = synth.bf16_bits(np.ldexp(1.0, exps).astype(np.float32))
    z_bits = synth.bf16_bits(-8 * synth.bf16_to_f32(s_bits))
    ch0 = synth.pack_q4_1(codes, s_bits, z_bits)
    x0 = np.zeros((M, K0), np.uint16)
    ks = [17, 2000]
    for m, k in enumerate(ks):
        x0[m, k] = 0x3F80
    W0 = oracle.weights_exact(ch0, "q4_1", N0, K0)
    y0_expect = np.stack([W0[:, k] for k in ks]).astype(np.float32)     # exact in bf16
    assert np.all(synth.bf16_to_f32(synth.bf16_bits(y0_expect)) == y0_expect)

    d0 = dev_u8(ch0)
    dx0 = dev_bf16(x0)
    y0 = torch.empty((M, N0), dtype=torch.float32, device="cuda")
    K1, N1 = 2 * N0, 1024
    ch1 = _gen("q4_1", N1, K1, "dep1")
    d1 = dev_u8(ch1)
    x1_view = y0.view(torch.int16)                     # [M][2*N0] bf16 = the bytes of y0
    y1 = torch.empty((M, N1), dtype=torch.float32, device="cuda")
    plan = q().Plan([(weight(d0, N0, K0, "q4_1"), dx0, y0), (weight(d1, N1, K1, "q4_1"), x1_view, y1)],
                    [0, 1], M)
    plan.set_mode(mode)
    x1_bits = y0_expect.view(np.uint16).reshape(M, K1)
    yr, a = oracle.gemv_ref(oracle.weights_exact(ch1, "q4_1", N1, K1), x1_bits)
    stale = np.full((M, K1), 0x3F80, np.uint16)
    ys, _ = oracle.gemv_ref(oracle.weights_exact(ch1, "q4_1", N1, K1), stale)
    assert np.max(np.abs(ys - yr) / (2e-3 * a)) > 10    # stale activations would be caught
    for _ in range(4):
        y0.view(torch.int32).fill_(0x3F803F80)          # stale contents before every run
        y1.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y0), y0_expect)
        assert oracle.tol_ratio(host(y1), yr, a) <= 1.0
    assert plan.errors() == 0


@pytest.mark.parametrize("mode", [0, 1])
def test_plan_in_a_hip_graph_replays_correctly(mode):
    M = 1
    jobs = [Job("q4_1", 2048, 2560, "gq", M), Job("q4_1", 2560, 9728, "gd", M)]
    plan = q().Plan([j.job() for j in jobs], [0, 1], M)
    plan.set_mode(mode)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        plan.run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        plan.run()
    torch.cuda.synchronize()
    for rep in range(3):
        for i, j in enumerate(jobs):     # new activations between replays
            j.xb = synth.gen_x(synth.rng("gpu-plan", "replay", rep, i), M, j.K)
            j.dx.copy_(torch.from_numpy(j.xb.view(np.int16)))
            j.dy.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j in jobs:
            j.check()
    assert plan.errors() == 0


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("layout", ["A", "B"])
def test_plan_mixed_kinds_in_segments(layout, mode):
    M = 1
    jobs = [Job("q4_k", 4096, 2560, "kq", M), Job("q4_k", 1024, 2560, "kk", M),
            Job("q4_k", 2560, 9728, "kd", M), Job("q8", 8192, 2560, "head", M, layout)]
    plan = q().Plan([j.job() for j in jobs], [0, 0, 1, 2], M)
    plan.set_mode(mode)
    for _ in range(2):
        plan.run()
        torch.cuda.synchronize()
        for j in jobs:
            j.check()
    assert plan.errors() == 0


@pytest.mark.parametrize("mode", [0, 1])
def test_plan_of_a_qwen3_4b_layer_and_lm_head(mode):
    """The real decode-step shapes: one layer's four phases and the lm_head, M = 1."""
    specs = synth.qwen3_4b_decode_specs(1, True)
    jobs, phases = [], []
    ph = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3, "lm_head": 4}
    for s in specs:
        j = Job.__new__(Job)
        j.kind, j.N, j.K, j.layout, j.M = "q4_1", s.N, s.K, None, 1
        j.ch = s.generate()
        j.dw = dev_u8(j.ch)
        j.xb = synth.gen_x(synth.rng("gpu-plan", "4b", s.name), 1, s.K)
        j.dx = dev_bf16(j.xb)
        j.dy = torch.full((1, s.N), float("nan"), dtype=torch.float32, device="cuda")
        j.w = weight(j.dw, s.N, s.K, "q4_1")
        jobs.append(j)
        phases.append(ph[s.name.split(".")[-1]])
    plan = q().Plan([j.job() for j in jobs], phases, 1)
    plan.set_mode(mode)
    plan.run()
    torch.cuda.synchronize()
    assert plan.errors() == 0
    for j in jobs:
        if j.N > 50000:   # lm_head: sampled tile rows
            y = host(j.dy)
            tr = np.array([0, 5, 2000, j.N // 32 - 1])
            W = oracle.weights_exact(j.ch[tr], "q4_1", 32 * len(tr), j.K)
            yr, a = oracle.gemv_ref(W, j.xb)
            ysub = np.concatenate([y[:, 32 * t:32 * t + 32] for t in tr], axis=1)
            assert oracle.tol_ratio(ysub, yr, a) <= 1.0
        else:
            j.check()


@pytest.mark.parametrize("kind", ["q4_1", "q4_k"])
def test_one_phase_of_many_jobs_is_one_launch(kind):
    """200 independent GEMVs (more than one batched call takes) in one phase:
    mode 0 runs them as one launch over the device job table."""
    M, N, K = 1, 64, 512
    jobs = [Job(kind, N, K, f"many{i}", M) for i in range(200)]
    plan = q().Plan([j.job() for j in jobs], [0] * len(jobs), M)
    for _ in range(2):
        for j in jobs:
            j.dy.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        for j in jobs:
            j.check()
    assert plan.errors() == 0


def test_plan_mode_is_checked():
    plan = q().Plan([Job("q4_1", 64, 512, "modes", 1).job()], [0], 1)
    with pytest.raises(q().Q4nxError):
        plan.set_mode(2)
