#!/usr/bin/env python3
"""Throughput of the Q4NX dequant-GEMV / block-GEMM / MoE path on one MI355X.

Headline (value): weight GB/s of a Qwen3-4B-shaped decode step -- 36 layers of
distinct all-q4_1 weights (q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up
9728x2560, down 2560x9728) plus the 151936x2560 lm_head, batch 1, one bf16
N(0,1) activation vector per projection.  A step is launched the way a decode
engine has to: per layer one batched GEMV for q|k|v (one input), one for o,
one for gate|up (one input), one for down, then the lm_head -- 145 launches,
captured once in a HIP graph and replayed.  Weights are resident in HBM before
timing starts.

Also reported: the roofline of the GEMV kernel (the step's bytes per launch
over its average launch duration, HIP events around the timed region) with the
HBM traffic rocprofv3 counted for it; the CPU oracle timed on a bounded
sample; and, as legs, the same step as one persistent plan launch; the mixed Q4_K + Q8 lm_head decode step
(Q8 in each code layout); the 64-token block GEMM over 32 layers of 8B-dense
shapes (TFLOP/s) with its M = 1, 2, 4 GEMV variants; the MoE layer (512
experts, top-10, shared expert, 48 layers) at T = 1 and T = 64; the single
1024x1024 GEMV.  Inputs are synthetic and seeded (see synth).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "Q4NX dequant-GEMV weight GB/s (% of HBM peak); 64-tok block GEMM TFLOP/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Kernel sources whose rocprofv3 counter summary (under profiles/) stays valid
# while they are unchanged.
KERNEL_SOURCES = {
    "k_gemv_q4": ["gemv.hip", "gemv_core.h", "q4nx_dev.h", "topk.h"],
    "k_gemv_q8": ["gemv.hip", "gemv_core.h", "q4nx_dev.h", "topk.h"],
    "k_gemm_q4": ["gemm.hip", "gemm_args.h", "mfma_q4.h", "q4nx_dev.h"],
    "k_moe": ["moe.hip", "moe_args.h", "gemv_core.h", "mfma_q4.h", "q4nx_dev.h"],
    "k_router": ["router.hip", "q4nx_dev.h"],
    "k_step": ["step.hip", "plan_args.h", "gemv_core.h", "q4nx_dev.h"],
}
PROFILE_FILES = {   # the summaries whose FETCH/WRITE figures feed a roofline's "traffic"
    "k_gemv_q4": "k_gemv_q4__qwen3_4b_decode_step.md",
    "k_gemm_q4": "k_gemm_q4__dense_8b_block_m64.md",
}


def source_sha1(kernel: str) -> str:
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "gemm_q4nx_chunk_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", PROFILE_FILES[kernel])
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in ("traffic_bytes_per_launch", "source_sha1"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha1") != source_sha1(kernel) or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def summarize(trace_db, fetch_db, write_db, kernel, title, commands, counters_db=None):
    """Markdown summary of rocprofv3 results (kernel trace + FETCH_SIZE / WRITE_SIZE
    passes) for one kernel family; the counters are scaled by what they read for
    the 1 GiB copy of the copyref leg."""
    import sqlite3
    from collections import defaultdict
    out = [f"# {kernel}: {title}", "", "Commands (from the repository root, rocprofv3 output under gpurun_out/):", ""]
    out += [f"    {c}" for c in commands]
    db = sqlite3.connect(trace_db)
    per = defaultdict(list)
    for name, dur in db.execute("select name, duration from kernels"):
        per[name].append(dur)
    out += ["", "## Kernel trace (--kernel-trace --stats)", "",
            "| kernel | dispatches | avg us | total ms |", "|---|---:|---:|---:|"]
    fam = []
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{name[:70]}` | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | {sum(v) / 1e6:.2f} |")
        if kernel in name:
            fam += v
    out += ["", f"{kernel} (all template variants): {len(fam)} dispatches, "
                f"average {sum(fam) / len(fam) / 1e3:.2f} us"]

    def counters(path, counter):
        c = sqlite3.connect(path)
        rows = c.execute("select kernel_name, grid_size_x, value from counters_collection "
                         "where counter_name = ?", (counter,)).fetchall()
        return rows
    fr, wr = counters(fetch_db, "FETCH_SIZE"), counters(write_db, "WRITE_SIZE")
    copy_f = [v for n, g, v in fr if "copyBuffer" in n and v > 500000]
    copy_w = [v for n, g, v in wr if "copyBuffer" in n and v > 500000]
    gib_kib = float(1 << 20)
    sf = gib_kib / (sum(copy_f) / len(copy_f))
    sw = gib_kib / (sum(copy_w) / len(copy_w))
    out += ["", "## HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; KiB per dispatch)", "",
            f"Copy kernel moving 1 GiB (1048576 KiB each way): FETCH_SIZE {sum(copy_f) / len(copy_f):.0f} KiB, "
            f"WRITE_SIZE {sum(copy_w) / len(copy_w):.0f} KiB, so FETCH_SIZE is scaled by {sf:.3f} and "
            f"WRITE_SIZE by {sw:.3f}.", "",
            "| kernel | grid (threads) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---:|---:|---:|---:|"]
    agg = defaultdict(lambda: [0, 0.0, 0, 0.0])
    for n, g, v in fr:
        if kernel in n:
            a = agg[(n, g)]; a[0] += 1; a[1] += v
    for n, g, v in wr:
        if kernel in n:
            a = agg[(n, g)]; a[2] += 1; a[3] += v
    tf = tw = 0.0
    nf = nw = 0
    for (n, g), (cf, vf, cw, vw) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| `{n[:60]}` | {g} | {cf} | {vf / max(cf, 1):.1f} | {vw / max(cw, 1):.1f} |")
        tf += vf; nf += cf; tw += vw; nw += cw
    per_launch = (tf / nf * sf + tw / nw * sw) * 1024
    out += ["", f"Scaled HBM bytes per {kernel} dispatch (fetch + write, averaged over "
                f"{nf} dispatches): {per_launch / 1e6:.3f} MB"]
    if counters_db:
        c = sqlite3.connect(counters_db)
        rows = c.execute("select kernel_name, grid_size_x, counter_name, value from counters_collection").fetchall()
        names = sorted({r[2] for r in rows})
        acc = defaultdict(lambda: defaultdict(list))
        for n, g, cn, v in rows:
            if kernel in n:
                acc[(n, g)][cn].append(v)
        out += ["", "## Other counters (one --pmc pass; average per dispatch)", "",
                "| kernel | grid (threads) | dispatches | " + " | ".join(names) + " |",
                "|---|---:|---:|" + "---:|" * len(names)]
        for (n, g), d in sorted(acc.items(), key=lambda kv: -len(next(iter(kv[1].values())))):
            cnt = max(len(v) for v in d.values())
            out.append(f"| `{n[:60]}` | {g} | {cnt} | " +
                       " | ".join(f"{sum(d[cn]) / len(d[cn]):.4g}" if d.get(cn) else "" for cn in names) + " |")
    out += ["", f"traffic_bytes_per_launch: {per_launch:.0f}",
            f"source_sha1: `{source_sha1(kernel)}`"]
    return "\n".join(out) + "\n"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DB", "FETCH_DB", "WRITE_DB"),
                    help="print the markdown summary of rocprofv3 results for --kernel and exit")
    ap.add_argument("--kernel", default="k_gemv_q4", choices=sorted(KERNEL_SOURCES))
    ap.add_argument("--title", default="")
    ap.add_argument("--commands", default="", help="the rocprofv3 commands, separated by ';'")
    ap.add_argument("--counters", default=None, help="a further --pmc results database to tabulate")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="all",
                    help="comma list of: decode, mixed, gemm, moe, single, kinds, repack, gguf, greedy, cpu, copyref "
                         "(default all but copyref)")
    ap.add_argument("--no-graph", action="store_true", help="launch the step without a HIP graph")
    return ap.parse_args()


args = parse()
if args.summarize:
    print(summarize(*args.summarize, args.kernel, args.title,
                    [c.strip() for c in args.commands.split(";") if c.strip()], args.counters), end="")
    sys.exit(0)
if args.gpus != 1:
    print(json.dumps({"error": "one GPU only: the library has no multi-GPU path; --gpus must be 1",
                      "n_gpus": args.gpus}))
    sys.exit(2)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import gemm_q4nx_chunk_amd as q  # noqa: E402
import synth  # noqa: E402

LEGS = set(["decode", "mixed", "gemm", "moe", "single", "kinds", "repack", "gguf", "greedy", "cpu"]
           if args.legs == "all"
           else args.legs.split(","))
DEV = torch.device("cuda:0")
torch.cuda.set_device(DEV)
GEN_THREADS = min(16, len(os.sched_getaffinity(0)))


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.uint8)).to(DEV)


def bf16_dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(DEV)


def upload_specs(specs):
    """Generate on host threads and upload tensor by tensor (bounded host memory)."""
    out = []
    for i in range(0, len(specs), GEN_THREADS):
        chunk = specs[i:i + GEN_THREADS]
        for s, arr in zip(chunk, synth.generate_many(chunk, GEN_THREADS)):
            out.append(to_dev(arr))
    return out


def events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_calls(fn, steps: int, warmup: int, graph: bool):
    """ms per call of fn (a whole step), timed over `steps` calls after `warmup`."""
    if graph:
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        torch.cuda.synchronize()
        run = g.replay
    else:
        run = fn
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = events()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ms = e0.elapsed_time(e1) / steps
    return ms, wall


def per_launch_ms(calls, reps: int = 3):
    """Average duration of each launch, HIP events around it on the launch stream."""
    torch.cuda.synchronize()
    pairs = []
    for _ in range(reps):
        for c in calls:
            e0, e1 = events()
            e0.record()
            c()
            e1.record()
            pairs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


# ----------------------------------------------------------------------------
# GEMV decode steps (headline and mixed)
# ----------------------------------------------------------------------------
class DecodeStep:
    """Weights, activations and outputs of one decode step, launched in phases."""

    PHASES = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

    def __init__(self, specs, tag, M=1):
        self.specs = specs
        self.M = M
        self.bytes = sum(s.nbytes for s in specs)
        t0 = time.time()
        self.w = upload_specs(specs)
        log(f"[{tag}] generated+uploaded {self.bytes / 1e9:.2f} GB in {time.time() - t0:.1f} s")
        self.x, self.y, self.desc = {}, {}, {}
        by_name = {s.name: i for i, s in enumerate(specs)}
        self.calls = []
        self.plan_jobs, self.plan_phases = [], []
        layers = sorted({int(s.name.split(".")[0][1:]) for s in specs if s.name.startswith("L")})
        for l in layers:
            for pi, ph in enumerate(self.PHASES):
                idx = [by_name[f"L{l}.{n}"] for n in ph]
                K = specs[idx[0]].K
                x = bf16_dev(synth.gen_x(synth.rng(tag, "x", l, ph[0]), M, K))
                jobs = []
                for i in idx:
                    s = specs[i]
                    y = torch.empty((M, s.N), dtype=torch.float32, device=DEV)
                    w = q.weight(self.w[i], s.N, s.K, s.kind, s.q8_layout if s.kind == "q8" else None)
                    jobs.append((w, x, y))
                    self.y[s.name] = y
                    self.plan_jobs.append((w, x, y))
                    self.plan_phases.append(4 * l + pi)
                self.calls.append(self._batched(jobs))
        for s, dw in zip(specs, self.w):
            if not s.name.startswith("L"):
                x = bf16_dev(synth.gen_x(synth.rng(tag, "x", s.name), M, s.K))
                y = torch.empty((M, s.N), dtype=torch.float32, device=DEV)
                w = q.weight(dw, s.N, s.K, s.kind, s.q8_layout if s.kind == "q8" else None)
                self.y[s.name] = y
                self.calls.append(self._batched([(w, x, y)]))
                self.plan_jobs.append((w, x, y))
                self.plan_phases.append(4 * len(layers))
        self.plan = q.Plan(self.plan_jobs, self.plan_phases, M)

    def _batched(self, jobs):
        M = self.M
        arr = (q.GemvJob * len(jobs))(*[q.GemvJob(w, q._ptr(x), q._ptr(y)) for w, x, y in jobs])
        keep = jobs
        lib = q.lib()

        def call():
            st = lib.q4nx_gemv_batched(arr, len(keep), M, torch.cuda.current_stream().cuda_stream)
            if st:
                raise q.Q4nxError(st, q.last_error())
        return call

    def run(self):
        for c in self.calls:
            c()


def decode_leg(specs, tag, steps, warmup, graph, M=1):
    """The step as phased launches (one batched GEMV launch per dependent phase,
    each waiting for the previous one) and as one persistent plan launch."""
    step = DecodeStep(specs, tag, M)
    ms, wall = time_calls(step.run, steps, warmup, graph)
    gbs = step.bytes / (ms * 1e-3) / 1e9
    msp, _ = time_calls(step.plan.run, steps, warmup, graph)          # mode 0: one launch per phase
    step.plan.set_mode(1)
    msp1, _ = time_calls(step.plan.run, steps, warmup, graph)         # mode 1: persistent launches
    step.plan.set_mode(0)
    errs = step.plan.errors()
    if errs:
        raise RuntimeError(f"plan reported error flags {errs}")
    res = {"ms_per_step": ms, "wall_ms_per_step": wall, "weight_bytes": step.bytes,
           "GB_s": gbs, "pct_hbm_peak": 100 * gbs / HBM_PEAK_GBS,
           "launches": len(step.calls), "graph": graph,
           "plan": {"ms_per_step": msp, "GB_s": step.bytes / (msp * 1e-3) / 1e9,
                    "launches": max(step.plan_phases) + 1, "mode": "one launch per phase (device job tables)",
                    "persistent": {"ms_per_step": msp1, "GB_s": step.bytes / (msp1 * 1e-3) / 1e9,
                                   "launches": 1 + sum(1 for a, b in zip(specs, specs[1:]) if a.kind != b.kind)},
                    "phases": max(step.plan_phases) + 1, "device_bytes": step.plan.nbytes()}}
    return step, res


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ----------------------------------------------------------------------------
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_gemv_sample(specs, M, budget_s, tag):
    """float64 decode + product of the oracle over specs until budget_s; returns
    (bytes of chunks, decode s, product s, names, flops)."""
    import oracle
    done, t_dec, t_dot, names, flops = 0, 0.0, 0.0, [], 0
    t_start = time.time()
    for s in specs:
        ch = s.generate()
        x = synth.gen_x(synth.rng("cpu", tag, s.name), M, s.K)
        t0 = time.perf_counter()
        W = oracle.weights_exact(ch, s.kind, s.N, s.K, s.q8_layout if s.kind == "q8" else None)
        t1 = time.perf_counter()
        oracle.gemv_ref(W, x)
        t2 = time.perf_counter()
        t_dec += t1 - t0
        t_dot += t2 - t1
        done += s.nbytes
        flops += 2 * M * s.N * s.K
        names.append(s.name)
        del W, ch
        if time.time() - t_start > budget_s:
            break
    return done, t_dec, t_dot, names, flops


def cpu_baseline(specs, moe_check=None, budget_s=15.0):
    """The oracle, as it stands, on bounded samples of the workloads (host cores)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = 1
    done, t_dec, t_dot, names, _ = _oracle_gemv_sample(specs, 1, budget_s, "c2")
    tot = t_dec + t_dot
    out = {"value": done / tot / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"float64 decode + dot of {len(names)} q4_1 tensors of the decode step "
                     f"({names[0]}..{names[-1]}, {done / 1e6:.0f} MB of chunks)",
           "decode_s": t_dec, "dot_s": t_dot,
           "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
           "threads_note": "cores = the BLAS thread pool, which runs the products; the "
                           "oracle's decode is numpy elementwise work on one thread"}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1, a1, b1, n1, _ = _oracle_gemv_sample(specs, 1, 5.0, "c2")
        out["one_thread"] = {"value": d1 / (a1 + b1) / 1e9, "unit": "GB/s", "cores": 1,
                             "sample": f"the first {len(n1)} tensors of the same step, {d1 / 1e6:.0f} MB"}
    # mixed-kind decode (Q4_K projections of the first layers)
    mixed = [s for s in synth.mixed_decode_specs(q8_layout="A") if s.kind == "q4_k"]
    d3, a3, b3, n3, _ = _oracle_gemv_sample(mixed, 1, 5.0, "c3")
    out["mixed_decode_q4k"] = {"GB_s": d3 / (a3 + b3) / 1e9, "tensors": len(n3), "bytes": d3,
                               "s": a3 + b3}
    # 64-token block GEMM: one 8B-dense layer at M = 64, extrapolated to the 32-layer block
    dense = synth.dense_8b_block_specs(layers=1)
    d4, a4, b4, n4, f4 = _oracle_gemv_sample(dense, 64, 30.0, "c4")
    full = sum(s.nbytes for s in synth.dense_8b_block_specs())
    out["block_gemm_8b_m64"] = {"TFLOP_s": f4 / (a4 + b4) / 1e12, "layer_s": a4 + b4,
                                "tensors": len(n4),
                                "block_s_extrapolated": (a4 + b4) * full / d4,
                                "note": "one layer measured; the 32-layer figure is extrapolated by bytes"}
    # MoE layer 0 at T = 1 and T = 64: the oracle's time, and the GPU layer output
    # of the MoE leg against it (|y - y_ref| / (2e-3 * a), a = the layer's error scale)
    if moe_check:
        D, De, Ds = synth.MOE_D_MODEL, synth.MOE_D_EXPERT, synth.MOE_D_SHARED

        def wt(p_, e):
            sp = synth.moe_expert_spec(0, p_, e) if e != "shared" else synth.moe_shared_spec(0, p_)
            return oracle.weights_exact(sp.generate(), "q4_1", sp.N, sp.K)
        res5 = {}
        for T, (Xb, ids, pr, Yg) in sorted(moe_check.items()):
            t0 = time.perf_counter()
            ye, ae = oracle.moe_layer_ref(Xb, ids, pr, lambda e: (wt("gate", e), wt("up", e), wt("down", e)),
                                          (wt("gate", "shared"), wt("up", "shared"), wt("down", "shared")),
                                          n_experts=synth.MOE_EXPERTS, with_scale=True)
            dt = time.perf_counter() - t0
            res5[f"T{T}"] = {"oracle_layer_s": dt, "oracle_48_layers_s_extrapolated": 48 * dt,
                             "gpu_layer0_tol_ratio": oracle.tol_ratio(Yg, ye, ae)}
        out["moe_512x10"] = res5
    return out


# ----------------------------------------------------------------------------
# block GEMM
# ----------------------------------------------------------------------------
def gemm_leg(steps, warmup, graph):
    specs = synth.dense_8b_block_specs()
    t0 = time.time()
    w = upload_specs(specs)
    nbytes = sum(s.nbytes for s in specs)
    log(f"[gemm] generated+uploaded {nbytes / 1e9:.2f} GB in {time.time() - t0:.1f} s")
    Xs = {K: bf16_dev(synth.gen_x(synth.rng("dense_8b_block", "X", K), 64, K)) for K in (4096, 14336)}
    names = [n for n, _, _ in synth.DENSE_8B_LAYER]
    Ys = {n: torch.empty((64, N), dtype=torch.float32, device=DEV) for n, N, _ in synth.DENSE_8B_LAYER}
    descs = [q.weight(dw, s.N, s.K, "q4_1") for s, dw in zip(specs, w)]
    lib = q.lib()
    import ctypes
    # One launch per dependent phase of a layer: q/k/v share X, so do gate/up.
    PHASES = ((0, 1, 2), (3,), (4, 5), (6,))
    launches = []
    for l in range(synth.DENSE_8B_LAYERS):
        for ph in PHASES:
            jobs = [(descs[7 * l + i], Ys[names[i]]) for i in ph]
            launches.append((q._gemm_jobs(jobs), len(jobs), Xs[specs[7 * l + ph[0]].K]))
    ws_bytes = max(lib.q4nx_gemm_batched_ws(arr, n) for arr, n, _ in launches[:4])
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)

    def launch(arr, n, X):
        r = lib.q4nx_gemm_batched(arr, n, X.data_ptr(), 64, ws.data_ptr(), ws.numel(),
                                  torch.cuda.current_stream().cuda_stream)
        if r:
            raise q.Q4nxError(r, q.last_error())

    def run64():
        for arr, n, X in launches:
            launch(arr, n, X)
    flops = sum(2 * 64 * s.N * s.K for s in specs)
    ms, wall = time_calls(run64, steps, warmup, graph)
    res = {"M64": {"ms_per_block": ms, "TFLOP_s": flops / (ms * 1e-3) / 1e12, "flops": flops,
                   "weight_bytes": nbytes, "GB_s": nbytes / (ms * 1e-3) / 1e9,
                   "pct_mfma_peak": 100 * flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                   # attainable = min(MFMA peak, flops per weight byte x HBM peak)
                   "attainable_TFLOP_s": min(BF16_MFMA_PEAK_TFLOPS, flops / nbytes * HBM_PEAK_GBS / 1e3),
                   "pct_attainable": 100 * flops / (ms * 1e-3) / 1e12
                   / min(BF16_MFMA_PEAK_TFLOPS, flops / nbytes * HBM_PEAK_GBS / 1e3),
                   "pct_hbm_peak": 100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                   "launches": len(launches)}}
    # roofline of the block GEMM kernel: its launches run back to back, so the timed
    # region over the launch count is the average launch duration.  At 64 rows a
    # q4_1 weight byte carries 204.8 flops, under the MI355X ridge (~312), so the
    # bound is HBM; the bf16 matrix-core fraction is reported beside it.
    n_launch = len(launches)
    ach = nbytes / (ms * 1e-3) / 1e9
    res["M64"]["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": ach / HBM_PEAK_GBS, "traffic": profiled_traffic("k_gemm_q4"),
                              "kernel": "k_gemm_q4h<q4_1> (M = 64)",
                              "avg_launch_us": ms * 1e3 / n_launch,
                              "bytes_per_launch": nbytes / n_launch,
                              "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
    # M = 1, 2, 4 through the GEMV path (same weights)
    for M in (1, 2, 4):
        xm = {K: bf16_dev(synth.gen_x(synth.rng("dense_8b_block", "xm", K, M), M, K)) for K in (4096, 14336)}
        ym = {N: torch.empty((M, N), dtype=torch.float32, device=DEV) for N in (1024, 4096, 14336)}
        groups = []
        for l in range(synth.DENSE_8B_LAYERS):
            base = 7 * l
            for ph in ((0, 1, 2), (3,), (4, 5), (6,)):
                jobs = [(descs[base + i], xm[specs[base + i].K], ym[specs[base + i].N]) for i in ph]
                arr = (q.GemvJob * len(jobs))(*[q.GemvJob(a, q._ptr(b), q._ptr(c)) for a, b, c in jobs])
                groups.append((arr, len(jobs)))

        def runm(M=M, groups=groups):
            st = torch.cuda.current_stream().cuda_stream
            for arr, n in groups:
                r = lib.q4nx_gemv_batched(arr, n, M, st)
                if r:
                    raise q.Q4nxError(r, q.last_error())
        msm, _ = time_calls(runm, steps, warmup, graph)
        res[f"M{M}"] = {"ms_per_block": msm, "GB_s": nbytes / (msm * 1e-3) / 1e9,
                        "pct_hbm_peak": 100 * nbytes / (msm * 1e-3) / 1e9 / HBM_PEAK_GBS}
    # a verify window of M tokens against one token over the same weights
    res["window_cost_vs_M1"] = {f"M{M}": res[f"M{M}"]["ms_per_block"] / res["M1"]["ms_per_block"] for M in (2, 4)}
    del w
    return res


# ----------------------------------------------------------------------------
# MoE
# ----------------------------------------------------------------------------
MOE_CHECK = {}   # layer 0's inputs and GPU output per T, checked against the oracle in the cpu leg


def moe_leg(steps, warmup, graph):
    D, De, Ds, E, L = synth.MOE_D_MODEL, synth.MOE_D_EXPERT, synth.MOE_D_SHARED, synth.MOE_EXPERTS, synth.MOE_LAYERS
    gu = (De // 32) * (D // 256) * 5120
    dn = (D // 32) * (De // 256) * 5120
    res = {}
    routes = {T: [synth.moe_router(l, T) for l in range(L)] for T in (1, 64)}
    need = [set(np.concatenate([routes[1][l][0].ravel(), routes[64][l][0].ravel()]).tolist())
            for l in range(L)]
    t0 = time.time()
    layers = []
    for l in range(L):
        arenas = {p: torch.empty(E * (gu if p != "down" else dn), dtype=torch.uint8, device=DEV)
                  for p in ("gate", "up", "down")}
        specs, where = [], []
        for e in sorted(need[l]):
            for p in ("gate", "up", "down"):
                specs.append(synth.moe_expert_spec(l, p, e))
                where.append((p, e))
        for p in ("gate", "up", "down"):
            specs.append(synth.moe_shared_spec(l, p))
            where.append((p, "shared"))
        shared = {}
        for i in range(0, len(specs), GEN_THREADS):
            part = specs[i:i + GEN_THREADS]
            for (p, e), arr in zip(where[i:i + GEN_THREADS], synth.generate_many(part, GEN_THREADS)):
                t = torch.from_numpy(arr.reshape(-1))
                if e == "shared":
                    shared[p] = t.to(DEV)
                else:
                    stride = gu if p != "down" else dn
                    arenas[p][e * stride:(e + 1) * stride].copy_(t)
        sw = (q.weight(shared["gate"], Ds, D, "q4_1"), q.weight(shared["up"], Ds, D, "q4_1"),
              q.weight(shared["down"], D, Ds, "q4_1"))
        Ld = q.moe_layer(E, D, De, "q4_1", arenas["gate"], arenas["up"], arenas["down"], gu, gu, dn,
                         shared=sw, d_shared=Ds)
        layers.append((Ld, arenas, shared))
    log(f"[moe] arenas {3 * E * gu * L / 1e9:.1f} GB allocated, selected experts generated "
        f"in {time.time() - t0:.1f} s")
    lib = q.lib()
    import ctypes
    for T in (1, 64):
        k = synth.MOE_TOP_K
        ws_b = q.moe_ws(layers[0][0], T, k)
        wss = [torch.empty(ws_b, dtype=torch.uint8, device=DEV) for _ in range(L)]
        X = [bf16_dev(synth.gen_x(synth.rng("moe_512x10", l, "X", T), T, D)) for l in range(L)]
        ids = [torch.from_numpy(routes[T][l][0]).to(DEV) for l in range(L)]
        ps = [torch.from_numpy(routes[T][l][1]).to(DEV) for l in range(L)]
        Ys = [torch.empty((T, D), dtype=torch.float32, device=DEV) for _ in range(L)]

        def run(T=T, wss=wss, X=X, ids=ids, ps=ps, Ys=Ys, ws_b=ws_b, k=k):
            st = torch.cuda.current_stream().cuda_stream
            for l in range(L):
                r = lib.q4nx_moe_experts(ctypes.byref(layers[l][0]), X[l].data_ptr(), ids[l].data_ptr(),
                                         ps[l].data_ptr(), T, k, Ys[l].data_ptr(), None,
                                         wss[l].data_ptr(), ws_b, st)
                if r:
                    raise q.Q4nxError(r, q.last_error())
        ms, wall = time_calls(run, steps, warmup, graph)
        MOE_CHECK[T] = (X[0].cpu().numpy().view(np.uint16), routes[T][0][0], routes[T][0][1],
                        Ys[0].cpu().numpy())
        y_full = [y.clone() for y in Ys]
        # algorithmic bytes: every selected expert read once per layer, plus the shared expert
        uniq = sum(len(np.unique(routes[T][l][0])) for l in range(L))
        nbytes = uniq * (2 * gu + dn) + L * 3 * (Ds // 32) * (D // 256) * 5120
        flops = L * T * (synth.MOE_TOP_K * 3 * 2 * De * D + 3 * 2 * Ds * D)
        res[f"T{T}"] = {"ms_per_step": ms, "layers": L, "weight_bytes": nbytes,
                        "distinct_experts_per_layer": uniq / L, "GB_s": nbytes / (ms * 1e-3) / 1e9,
                        "pct_hbm_peak": 100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "TFLOP_s": flops / (ms * 1e-3) / 1e12,
                        # per layer: decode-sized gate/up, down + combine; or route, gate/up and
                        # down for one-token batches then for the rest, combine
                        "launches": (2 if T * k <= 64 else 6) * L}
        # tail skip: the picks ranked 7..10 dropped, the first six keep their weights
        # (no renormalisation); the layer outputs move by rel_l2 against all ten picks
        ks = 6
        ids6 = [i[:, :ks].contiguous() for i in ids]
        ps6 = [p_[:, :ks].contiguous() for p_ in ps]
        ms6, _ = time_calls(lambda: run(ids=ids6, ps=ps6, k=ks), steps, warmup, graph)
        uniq6 = sum(len(np.unique(routes[T][l][0][:, :ks])) for l in range(L))
        b6 = uniq6 * (2 * gu + dn) + L * 3 * (Ds // 32) * (D // 256) * 5120
        rel = [float(torch.linalg.vector_norm(y - yf) / torch.linalg.vector_norm(yf))
               for y, yf in zip(Ys, y_full)]
        res[f"T{T}"]["tail_skip_top6"] = {"ms_per_step": ms6, "speedup": ms / ms6, "weight_bytes": b6,
                                          "GB_s": b6 / (ms6 * 1e-3) / 1e9,
                                          "rel_l2_vs_top10_mean": sum(rel) / L, "rel_l2_vs_top10_max": max(rel)}
        del ids6, ps6, y_full
        if T * k > 64:
            # the same call with experts of 5 or more pairs (and the shared expert) on
            # the bf16 matrix cores instead of the batched dot2 kernels (the best
            # threshold measured at this block; the library's default keeps them off)
            for l in range(L):
                layers[l][0].hot_tokens = 5
            ms_hot, _ = time_calls(run, steps, warmup, graph)
            for l in range(L):
                layers[l][0].hot_tokens = 0
            res[f"T{T}"]["matrix_core_5"] = {"ms_per_step": ms_hot, "GB_s": nbytes / (ms_hot * 1e-3) / 1e9}
        # the router on the device in front of the layer (bf16 router rows 512 x 2048 per layer)
        Rs = [bf16_dev(synth.bf16_bits((synth.rng("moe_512x10", l, "R").standard_normal((E, D)) * 0.05)
                                       .astype(np.float32))) for l in range(L)]
        ids_d = [torch.empty((T, k), dtype=torch.int32, device=DEV) for _ in range(L)]
        p_d = [torch.empty((T, k), dtype=torch.float32, device=DEV) for _ in range(L)]
        lg_d = torch.empty((T, E), dtype=torch.float32, device=DEV)

        def run_router(T=T, Rs=Rs, X=X, ids_d=ids_d, p_d=p_d, lg_d=lg_d):
            st = torch.cuda.current_stream().cuda_stream
            for l in range(L):
                r = lib.q4nx_moe_router(Rs[l].data_ptr(), X[l].data_ptr(), T, D, E, k, 1,
                                        ids_d[l].data_ptr(), p_d[l].data_ptr(), lg_d.data_ptr(), st)
                if r:
                    raise q.Q4nxError(r, q.last_error())
        msr, _ = time_calls(run_router, steps, warmup, graph)
        rbytes = L * E * D * 2
        res[f"T{T}"]["router"] = {"ms_per_step": msr, "router_bytes": rbytes,
                                  "GB_s": rbytes / (msr * 1e-3) / 1e9, "launches": 2 * L}
        del wss, X, ids, ps, Ys, Rs, ids_d, p_d, lg_d
    del layers
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------
# weight preparation and the Q8 tied head's two ends
# ----------------------------------------------------------------------------
def repack_leg(steps, warmup, graph):
    """Q4_K -> q4_1 repack of one 8B-dense gate|up-sized weight (28672 x 4096)."""
    N, K = 2 * 14336, 4096
    spec = synth.TensorSpec("gate_up", "q4_k", N, K, ("repack_q4k", 0))
    src0 = to_dev(spec.generate())
    out_bytes = (N // 32) * (K // 256) * 5120
    n = n_copies(src0.numel() + out_bytes)   # source and destination pairs cycled past the cache
    srcs = [src0] + [src0.clone() for _ in range(n - 1)]
    ws = [q.weight(s_, N, K, "q4_k") for s_ in srcs]
    outs = [torch.empty(out_bytes, dtype=torch.uint8, device=DEV) for _ in range(n)]

    def run():
        for w, o in zip(ws, outs):
            q.repack_q4k_to_q41(w, o)
    ms, _ = time_calls(run, steps, warmup, graph)
    ms /= n
    moved = src0.numel() + out_bytes
    res = {"shape": [N, K], "bytes_read": src0.numel(), "bytes_written": out_bytes, "ms": ms,
           "copies_cycled": n, "working_set_bytes": n * moved,
           "GB_s_read_plus_write": moved / (ms * 1e-3) / 1e9,
           "pct_hbm_peak": 100 * moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del srcs, ws, outs, src0
    torch.cuda.empty_cache()
    return res


def gguf_leg(steps, warmup, graph):
    """GGUF Q4_0 / Q4_1 / Q4_K -> q4_1 conversion of one 8B-dense gate|up-sized
    tensor (28672 x 4096) each: bytes read plus written per second."""
    N, K = 2 * 14336, 4096
    out_bytes = (N // 32) * (K // 256) * 5120
    res = {}
    for name, gtype in (("q4_0", q.GGUF_Q4_0), ("q4_1", q.GGUF_Q4_1), ("q4_k", q.GGUF_Q4_K)):
        src0 = to_dev(synth.gen_gguf(synth.rng("gguf", name), gtype, N, K))
        n = n_copies(src0.numel() + out_bytes)
        srcs = [src0] + [src0.clone() for _ in range(n - 1)]
        outs = [torch.empty(out_bytes, dtype=torch.uint8, device=DEV) for _ in range(n)]

        def run(srcs=srcs, outs=outs, gtype=gtype):
            for s_, o in zip(srcs, outs):
                q.gguf_to_q41(gtype, s_, N, K, o)
        ms, _ = time_calls(run, steps, warmup, graph)
        ms /= n
        moved = src0.numel() + out_bytes
        res[name] = {"bytes_read": src0.numel(), "bytes_written": out_bytes, "ms": ms,
                     "copies_cycled": n, "working_set_bytes": n * moved,
                     "GB_s_read_plus_write": moved / (ms * 1e-3) / 1e9,
                     "pct_hbm_peak": 100 * moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del srcs, outs, src0
        torch.cuda.empty_cache()
    return {"shape": [N, K], **res}


ROTATE_BYTES = 1100 * 1000 * 1000   # working sets past the 256 MB Infinity Cache


def n_copies(nbytes: int) -> int:
    """Distinct device copies of a weight so that cycling through them moves at least ROTATE_BYTES."""
    return max(1, -(-ROTATE_BYTES // nbytes))


def kinds_leg(steps, warmup, graph):
    """One large decode GEMV per chunk kind at the lm_head shape (151936 x 2560,
    M = 1): q4_1, Q4_K and Q8 in both code layouts, HIP events around each call.
    Each timed run cycles through enough distinct copies of the weight (over
    1.1 GB) that every call reads HBM, not the Infinity Cache."""
    name, N, K = synth.QWEN3_4B_LM_HEAD
    x = bf16_dev(synth.gen_x(synth.rng("kinds", "x"), 1, K))
    y = torch.empty((1, N), dtype=torch.float32, device=DEV)
    res = {}
    for kind, lay, key in (("q4_1", None, ("qwen3_4b_decode", 10_000, name)),
                           ("q4_k", None, ("kinds", "q4_k")),
                           ("q8", "A", ("mixed_decode", 10_000, name)),
                           ("q8", "B", ("mixed_decode", 10_000, name))):
        spec = synth.TensorSpec(name, kind, N, K, key, q8_layout=lay or "A",
                                opts={"zero": "normal"} if kind == "q4_1" else {})
        ch = spec.generate()
        if lay == "B":
            ch = synth.q8_relayout(ch, "A", "B")
        d0 = to_dev(ch)
        del ch
        calls = n_copies(d0.numel())
        ds = [d0] + [d0.clone() for _ in range(calls - 1)]
        ws = [q.weight(d, N, K, kind, lay) for d in ds]

        def run(ws=ws):
            for w in ws:
                q.gemv(w, x, y, 1)
        ms, _ = time_calls(run, steps, warmup, graph)
        us = ms * 1e3 / calls
        res[kind if lay is None else f"q8_{lay}"] = {"bytes": d0.numel(), "us_per_call": us,
                                                      "copies_cycled": calls,
                                                      "working_set_bytes": calls * d0.numel(),
                                                      "GB_s": d0.numel() / (us * 1e-6) / 1e9,
                                                      "pct_hbm_peak": 100 * d0.numel() / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        del ds, ws, d0
        torch.cuda.empty_cache()
    return res


def greedy_leg(steps, warmup, graph):
    """The Q8 tied 151936 x 2560 head in both code layouts: embedding row gather
    for 1 and 64 tokens, greedy decode's lm_head GEMV + argmax (M = 1) as two
    launches, and the same head as one launch with its top-k pick (k = 1, 10)."""
    name, N, K = synth.QWEN3_4B_LM_HEAD
    chA = synth.TensorSpec(name, "q8", N, K, ("mixed_decode", 10_000, name), q8_layout="A").generate()
    reps = 50
    res = {}
    for lay in ("A", "B"):
        d = to_dev(chA if lay == "A" else synth.q8_relayout(chA, "A", "B"))
        w = q.weight(d, N, K, "q8", lay)
        r = {}
        for T in (1, 64):
            ids = [torch.from_numpy(synth.rng("greedy", "ids", T, i).integers(0, N, T).astype(np.int32)).to(DEV)
                   for i in range(reps)]
            out = torch.empty((T, K), dtype=torch.float32, device=DEV)

            def rows(ids=ids, out=out, T=T):
                for i in ids:
                    q.q8_rows(w, i, T, out)
            ms, _ = time_calls(rows, steps, warmup, graph)
            r[f"rows_T{T}_us"] = ms * 1e3 / reps
        x = bf16_dev(synth.gen_x(synth.rng("greedy", "x"), 1, K))
        y = torch.empty((1, N), dtype=torch.float32, device=DEV)
        idx = torch.empty(1, dtype=torch.int32, device=DEV)
        aws = torch.empty(q.argmax_ws(N, 1), dtype=torch.uint8, device=DEV)

        def head():
            q.gemv(w, x, y, 1)
            q.argmax(y, N, 1, idx, ws=aws)

        def argmax_split():
            for _ in range(reps):
                q.argmax(y, N, 1, idx, ws=aws)

        def argmax_one_wg():
            for _ in range(reps):
                q.argmax(y, N, 1, idx)
        # the same head in one launch: GEMV with its top-k pick, no logits written
        tk = {}
        for k in (1, 10):
            tids = torch.empty((1, k), dtype=torch.int32, device=DEV)
            tws = torch.zeros(q.gemv_topk_ws(w, 1, k), dtype=torch.uint8, device=DEV)

            def fused(tids=tids, tws=tws, k=k):
                q.gemv_topk(w, x, 1, k, tids, tws)
            msk, _ = time_calls(fused, steps, warmup, graph)
            tk[f"k{k}_us"] = msk * 1e3
            tk[f"k{k}_GB_s"] = d.numel() / (msk * 1e-3) / 1e9

        def gemv_only():
            q.gemv(w, x, y, 1)
        ms, _ = time_calls(head, steps, warmup, graph)
        msg, _ = time_calls(gemv_only, steps, warmup, graph)
        msa, _ = time_calls(argmax_split, steps, warmup, graph)
        ms1, _ = time_calls(argmax_one_wg, steps, warmup, graph)
        r.update({"head_gemv_argmax_us": ms * 1e3, "head_GB_s": d.numel() / (ms * 1e-3) / 1e9,
                  "gemv_alone_us": msg * 1e3, "head_one_launch_topk": tk,
                  "argmax_us": msa * 1e3 / reps, "argmax_one_workgroup_us": ms1 * 1e3 / reps})
        res[f"layout_{lay}"] = r
        del d
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------
# single 1024 x 1024 GEMV, rotated over distinct copies
# ----------------------------------------------------------------------------
def single_leg():
    spec = synth.single_gemv_spec()
    ch = spec.generate()
    copies = 2048
    big = torch.from_numpy(np.tile(ch.reshape(1, -1), (copies, 1)).reshape(-1)).to(DEV)
    x = bf16_dev(synth.gen_x(synth.rng("q4_1_gemv_1024", 0, "x"), 1, spec.K))
    y = torch.empty((1, spec.N), dtype=torch.float32, device=DEV)
    descs = [q.weight(big[i * spec.nbytes:(i + 1) * spec.nbytes], spec.N, spec.K, "q4_1") for i in range(copies)]
    lib = q.lib()
    import ctypes

    def run():
        st = torch.cuda.current_stream().cuda_stream
        for d in descs:
            lib.q4nx_gemv(ctypes.byref(d), x.data_ptr(), y.data_ptr(), 1, st)
    ms, _ = time_calls(run, 3, 1, graph=False)
    per = ms / copies * 1e3
    msg, _ = time_calls(run, 3, 1, graph=True)
    perg = msg / copies * 1e3
    hot = descs[0]

    def run_hot():
        st = torch.cuda.current_stream().cuda_stream
        for _ in range(copies):
            lib.q4nx_gemv(ctypes.byref(hot), x.data_ptr(), y.data_ptr(), 1, st)
    msh, _ = time_calls(run_hot, 3, 1, graph=True)
    # the same GEMVs, 64 independent ones (own weight copy, x and y) per batched launch
    nj = 64
    xs = bf16_dev(np.tile(synth.gen_x(synth.rng("q4_1_gemv_1024", 0, "x"), 1, spec.K), (nj, 1)))
    ys = torch.empty((nj, spec.N), dtype=torch.float32, device=DEV)
    arrs = []
    for b0 in range(0, copies, nj):
        arrs.append((q.GemvJob * nj)(*[q.GemvJob(descs[b0 + j], q._ptr(xs[j]), q._ptr(ys[j]))
                                       for j in range(nj)]))

    def run_batched():
        st = torch.cuda.current_stream().cuda_stream
        for arr in arrs:
            r = lib.q4nx_gemv_batched(arr, nj, 1, st)
            if r:
                raise q.Q4nxError(r, q.last_error())
    msb, _ = time_calls(run_batched, 5, 2, graph=True)
    perb = msb / copies * 1e3
    # all 2048 distinct copies in ONE launch: a plan whose single phase holds every GEMV
    yp = torch.empty((copies, spec.N), dtype=torch.float32, device=DEV)
    plan = q.Plan([(descs[i], x, yp[i]) for i in range(copies)], [0] * copies, 1)
    msp, _ = time_calls(plan.run, 5, 2, graph=True)
    if plan.errors():
        raise RuntimeError("plan of the 2048 copies reported an error flag")
    perp = msp / copies * 1e3
    plan.close()
    return {"weight_bytes": spec.nbytes, "rotated_copies": copies,
            "one_launch_2048_copies": {"launches": 1, "ms": msp, "us_per_gemv": perp,
                                       "GB_s": spec.nbytes / (perp * 1e-6) / 1e9,
                                       "pct_hbm_peak": 100 * spec.nbytes / (perp * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "us_per_call_stream": per, "us_per_call_graph": perg,
            "GB_s_graph_rotated": spec.nbytes / (perg * 1e-6) / 1e9,
            "us_per_call_graph_hot": msh / copies * 1e3,
            "batched_64_per_launch": {"us_per_gemv": perb, "GB_s": spec.nbytes / (perb * 1e-6) / 1e9,
                                      "pct_hbm_peak": 100 * spec.nbytes / (perb * 1e-6) / 1e9 / HBM_PEAK_GBS}}


# ----------------------------------------------------------------------------
def main():
    out = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "qwen3_4b_decode_step_q4_1", "layers": synth.QWEN3_4B_LAYERS,
                      "batch": 1, "lm_head": "151936x2560", "kind": "q4_1",
                      "phases": "per layer q|k|v, o, gate|up, down, then lm_head (145), each "
                                "waiting for the previous one; one batched launch per phase",
                      "hip_graph": not args.no_graph},
           "device": torch.cuda.get_device_name(0)}
    graph = not args.no_graph
    legs = {}
    specs = synth.qwen3_4b_decode_specs()
    if "decode" in LEGS:
        step, res = decode_leg(specs, "qwen3_4b_decode", args.steps, args.warmup, graph)
        out["value"] = res["GB_s"]
        out["ms_per_step"] = res["ms_per_step"]
        out["config"]["weight_bytes_per_step"] = res["weight_bytes"]
        out["pct_hbm_peak"] = res["pct_hbm_peak"]
        # roofline of the dominant kernel: the batched q4_1 M=1 GEMV kernel, which makes
        # every launch of the step.  The step's launches run back to back, so the
        # timed region (HIP events on the launch stream) over the launch count is the
        # average launch duration; bytes per launch = step bytes / launches.
        n_launch = len(step.calls)
        avg_ms = res["ms_per_step"] / n_launch
        per_launch_bytes = res["weight_bytes"] / n_launch
        ach = per_launch_bytes / (avg_ms * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS, "traffic": profiled_traffic("k_gemv_q4"),
                           "kernel": "k_gemv_q4x<q4_1, M=1> (k_gemv_q4 family)",
                           "avg_launch_us": avg_ms * 1e3, "bytes_per_launch": per_launch_bytes,
                           "launches_timed": n_launch * args.steps}
        legs["decode"] = res
        del step
        torch.cuda.empty_cache()
    if "mixed" in LEGS:
        for lay in ("A", "B"):
            ms = synth.mixed_decode_specs(q8_layout=lay)
            if lay == "B":   # the same logical lm_head, re-encoded in layout B
                head = ms[-1]
                orig = head.generate
                head.generate = lambda orig=orig: synth.q8_relayout(orig(), "A", "B")
            st, r = decode_leg(ms, f"mixed_decode", args.steps, args.warmup, graph)
            head_i = len(st.calls) - 1
            dur = per_launch_ms([st.calls[head_i]], reps=10)   # the Q8 lm_head GEMV alone
            r["q8_lm_head_us"] = 1e3 * sum(dur) / len(dur)
            r["q8_lm_head_GB_s"] = ms[-1].nbytes / (sum(dur) / len(dur) * 1e-3) / 1e9
            legs[f"mixed_q4k_q8{lay}"] = r
            del st
            torch.cuda.empty_cache()
    if "kinds" in LEGS:   # before the MoE leg, whose 48 GB of arenas come and go
        legs["lm_head_shape_per_kind"] = kinds_leg(max(3, args.steps // 2), 2, graph)
    if "gemm" in LEGS:
        legs["block_gemm_8b"] = gemm_leg(max(3, args.steps // 4), 2, graph)
        torch.cuda.empty_cache()
    if "moe" in LEGS:
        # eight untimed replays: the first MoE graph of a process can run about 20%
        # slow for its first few replays (measured), and the timed ones come after
        legs["moe_512x10"] = moe_leg(max(3, args.steps // 2), 8, graph)
    if "single" in LEGS:
        legs["single_gemv_1024"] = single_leg()
    if "repack" in LEGS:
        legs["repack_q4k_8b_gate_up"] = repack_leg(args.steps, 2, graph)
    if "gguf" in LEGS:
        legs["gguf_to_q41_8b_gate_up"] = gguf_leg(args.steps, 2, graph)
    if "greedy" in LEGS:
        legs["q8_head_151936x2560"] = greedy_leg(max(3, args.steps // 2), 2, graph)
    if "copyref" in LEGS:
        # a plain device copy of known size, for scaling the HBM byte counters
        a = torch.empty(1 << 30, dtype=torch.uint8, device=DEV)
        b = torch.empty_like(a)
        ms, _ = time_calls(lambda: b.copy_(a), 5, 1, graph=False)
        legs["copy_1GiB"] = {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "ms": ms,
                             "GB_s_read_plus_write": 2 * (1 << 30) / (ms * 1e-3) / 1e9}
        del a, b
    if "cpu" in LEGS:
        out["cpu_baseline"] = cpu_baseline(specs, MOE_CHECK)
    out["legs"] = legs
    print(json.dumps(out))


if __name__ == "__main__":
    main()
