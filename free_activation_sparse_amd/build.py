"""Builds libsparse_linear.so (HIP, gfx950) in-tree with hipcc, and beside
it libsparse_linear_timeline.so: the same library with fused.hip compiled with
SL_TIMELINE, whose fused forward records per-workgroup timestamps
(sparse_linear_set_timeline; measurement only).

    python -m free_activation_sparse_amd.build        # always recompiles
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsparse_linear.so")
LIB_TIMELINE = os.path.join(HERE, "libsparse_linear_timeline.so")
SOURCES = ["api.cpp", "layout.hip", "gate.hip", "product.hip", "fused.hip", "union_product.hip", "ffn.hip", "double_sparse.hip", "ceiling.hip"]

HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU forms.
# Denormals are preserved (scores may be subnormal); no fp contraction except
# where a kernel calls fmaf explicitly.
CFLAGS = [
    "-x", "hip", "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


def _compile(job) -> str:
    src, defines, suffix = job
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [HIPCC, *CFLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link both shared libraries; returns the path
    of the regular one."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = [(s, [], "") for s in srcs] + [("fused.hip", ["-DSL_TIMELINE"], "_timeline")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    regular, timeline = objs[:len(srcs)], objs[len(srcs):]
    _link(regular, LIB)
    _link([o for o, s in zip(regular, srcs) if s != "fused.hip"] + timeline, LIB_TIMELINE)
    if verbose:
        print(f"built {LIB} and {LIB_TIMELINE}")
    return LIB


def is_stale() -> bool:
    """True when the library is missing or older than a source or header."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    deps += [os.path.join(os.path.dirname(HERE), "include", f) for f in ("sparse_linear.h", "double_sparse.h")]
    return any(os.path.getmtime(d) > t for d in deps if os.path.exists(d))


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
