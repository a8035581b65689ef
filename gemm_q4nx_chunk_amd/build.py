"""Build libq4nx.so in-tree with hipcc for gfx950.

Each HIP source compiles to its own object in parallel, then one link.  All
device code is built with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4nx.so")
OBJDIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["api.hip", "gemv.hip", "plan.hip", "step.hip", "gemm.hip", "decode.hip", "moe.hip", "router.hip"]
ARCH = os.environ.get("Q4NX_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libq4nx.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = _hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        jobs.append((obj, [cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[0] for j in jobs]])
    os.replace(tmp, LIB)
    return LIB


# The host-sanitised library: api.hip (every argument check of the C ABI) with
# its host code built under AddressSanitizer and UndefinedBehaviorSanitizer,
# linked with the other objects of build().  The device code is untouched
# (sanitisers are asked for the host side only).  Loading it needs the shared
# ASan runtime preloaded (asan_runtime()) and Q4NX_LIB set to its path.
SAN_DIR = os.path.join(OBJDIR, "asan")
SAN_LIB = os.path.join(SAN_DIR, "libq4nx.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime next to hipcc (may not exist)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    res = subprocess.run([clang, "-print-resource-dir"], capture_output=True, text=True).stdout.strip()
    return os.path.join(res, "lib", "linux", "libclang_rt.asan-x86_64.so")


def build_sanitized() -> str:
    """Build SAN_LIB (needs the objects of build()); returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    cc = _hipcc()
    others = [os.path.join(OBJDIR, s.replace(".hip", ".o")) for s in SOURCES if s != "api.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: {missing[0]} is missing")
    obj = os.path.join(SAN_DIR, "api.o")
    _run([cc, *[f for f in FLAGS if f != "-O3"], "-O1", "-g", *SAN_FLAGS, "-c", os.path.join(CSRC, "api.hip"),
          "-o", obj])
    tmp = SAN_LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS[:4], "-shared-libasan", "-o", tmp, obj,
          *others])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized())
    else:
        print(build(verbose=True))
