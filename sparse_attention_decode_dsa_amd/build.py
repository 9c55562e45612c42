"""Build libdsa.so in-tree: every HIP source in csrc/ for gfx950 plus the host ABI.

    python -m sparse_attention_decode_dsa_amd.build

Each source is compiled on its own (in parallel) and the objects are linked
with hipcc.  The library lands next to this file, where the binding loads it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")

SOURCES = ["dsa_api.cpp", "quantize_q.hip", "index_scores.hip", "topk.hip", "topk_noalloc.hip",
           "sparse_mla.hip", "lse_merge.hip", "cache_write.hip", "merge_project.hip"]
# The benchmark's plain bandwidth kernels, in a library of their own.
BW_SOURCES = ["bandwidth.hip"]
BW_LIB = os.path.join(PKG, "libdsa_bw.so")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libdsa.so")


def flags() -> list[str]:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wextra", "-Werror",
        # Keep the compiler from forming packed fp32 instructions.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in VGPRs: no AGPR copies around accumulator updates.
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", INCLUDE,
    ]


def _compile(src: str) -> tuple[str, str]:
    os.makedirs(OBJDIR, exist_ok=True)
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + flags() + lang + ["-c", path, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (p.stdout + p.stderr).splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{err}")
    return obj, err


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{' '.join(cmd)}\n{p.stdout}{p.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source for gfx950 and link libdsa.so (and the benchmark's
    libdsa_bw.so); returns the path of libdsa.so."""
    srcs = SOURCES + BW_SOURCES
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = dict(zip(srcs, ex.map(_compile, srcs)))
    for obj, msg in results.values():
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
    _link([results[s][0] for s in SOURCES], LIB)
    _link([results[s][0] for s in BW_SOURCES], BW_LIB)
    if verbose:
        print(f"built {LIB} and {BW_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
