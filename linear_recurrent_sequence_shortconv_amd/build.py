"""Compile the HIP kernels and the C ABI into libprism.so (in-tree).

    python -m linear_recurrent_sequence_shortconv_amd.build

Every source is compiled for gfx950 with hipcc, in parallel, into _build/,
then linked into linear_recurrent_sequence_shortconv_amd/libprism.so.  The
library is written to a temporary name and renamed, so a process that has
the old one open never sees a partial file.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libprism.so")

# slowest first, so the parallel compile finishes early
SOURCES = [
    "chunk_bwd_solve.hip",
    "chunk_bwd_pairs.hip",
    "chunk_bwd_state.hip",
    "chunk_fwd.hip",
    "chunk_fused_gelu.hip",
    "chunk_fused_identity.hip",
    "refine_bwd_gelu.hip",
    "refine_bwd_gelu_past.hip",
    "refine_bwd_identity.hip",
    "refine_bwd_identity_past.hip",
    "refine_fwd.hip",
    "state.hip",
    "step.hip",
    "refine_bwd.hip",
    "noalloc.hip",
    "chunk_bwd.hip",
    "prism_api.cpp",
]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, jobs=None):
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + f".tmp{os.getpid()}"
    _run([hipcc] + FLAGS + ["-shared", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
