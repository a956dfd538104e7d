"""Build libqmm.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m gemm_qmm_gemv_amd.build``.  Every call compiles; the
library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqmm.so")
# (source, extra defines, object name); gemv_bits.hip is built once per width.
SOURCES = [("qmm_api.hip", [], "qmm_api.o"), ("gemm.hip", [], "gemm.o"), ("gemm_wl.hip", [], "gemm_wl.o"),
           ("unpack.hip", [], "unpack.o")] + [
    ("gemv_bits.hip", ["-DQMM_BITS=%d" % b], "gemv_b%d.o" % b) for b in (2, 3, 4, 5, 6, 8, 16)]
ARCH = os.environ.get("QMM_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=" + ARCH,
    # Keep the compiler from forming packed fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed: %s" % " ".join(cmd[-3:]))
    if verbose and msgs:
        print("\n".join(msgs))


def _stale(obj: str, src: str) -> bool:
    """An object is stale when it is missing or older than its source or any
    header it may include (csrc/*.h, include/*.h)."""
    if not os.path.exists(obj):
        return True
    deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + [
        os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose: bool = False, out: str | None = None, extra_flags=(), objdir: str | None = None,
          incremental: bool = False) -> str:
    """Compile every source (in parallel) and link libqmm.so.  Rebuilds every
    object unless ``incremental`` (then only objects older than their
    sources or headers; the library is always relinked).
    ``out``/``extra_flags``/``objdir`` produce variant builds (e.g. with a
    -D switch) next to the default one."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = objdir or os.path.join(ROOT, "_build", "qmm")
    out = out or LIB
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"] + list(extra_flags)
    jobs = []
    for src, defs, oname in SOURCES:
        obj = os.path.join(objdir, oname)
        jobs.append(([hipcc] + compile_flags + defs + ["-c", os.path.join(CSRC, src), "-o", obj], obj,
                     os.path.join(CSRC, src)))
    todo = [j for j in jobs if not incremental or _stale(j[1], j[2])]
    workers = max(1, min(len(todo), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), todo))
    tmp = out + ".tmp%d" % os.getpid()
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH] + [j[1] for j in jobs] + ["-o", tmp],
         verbose)
    os.replace(tmp, out)
    if out == LIB:
        build_ceiling(verbose)
    return out


CEILING_LIB = os.path.join(HERE, "libqmm_ceiling.so")


def build_ceiling(verbose: bool = False) -> str:
    """libqmm_ceiling.so: the streaming-read and MFMA-loop kernels whose
    measured rates bench.py reports beside the spec peaks."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = CEILING_LIB + ".tmp%d" % os.getpid()
    _run([hipcc] + FLAGS + [os.path.join(CSRC, "ceiling.hip"), "-o", tmp], verbose)
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv[1:]))
