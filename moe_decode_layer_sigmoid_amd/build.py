"""Compiles the HIP sources of the MoE decode layer into libmoe_decode.so
(gfx950, in-tree, next to this file).

    python -m moe_decode_layer_sigmoid_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_decode.so")
SOURCES = ["api.hip", "router.hip", "experts_gemv.hip", "experts_mfma.hip", "epilogue.hip",
           "experts_chain.hip", "probe.hip"]
# experts_chain.hip is also compiled once per w13 chunk count (the first
# template argument of its kernels), each into its own object, in parallel.
CHAIN_NJG = range(1, 9)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # hipcc -O3 forms packed fp32 instructions on its own; keep them off.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    return res.returncode, out


def build(verbose: bool = False) -> str:
    """Always compiles (a stale library is never reused by this call): every
    source to an object in parallel, then one link."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append((obj, [hipcc(), *FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj]))
    for nj in CHAIN_NJG:
        obj = os.path.join(objdir, "experts_chain_njg%d.o" % nj)
        jobs.append((obj, [hipcc(), *FLAGS, *inc, "-DMOE_CHAIN_NJG=%d" % nj, "-c",
                           os.path.join(CSRC, "experts_chain.hip"), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    for (obj, cmd), (rc, out) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (os.path.basename(obj), out))
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp%d" % os.getpid()
    rc, out = _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC",
                    *[j[0] for j in jobs], "-o", tmp])
    if rc != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("link failed:\n" + out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
