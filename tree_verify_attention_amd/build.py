"""Compile the HIP sources of the library into ``libtreeverify.so`` (gfx950).

Usage: ``python -m tree_verify_attention_amd.build`` or ``build()`` from
Python.  The library is built in-tree, next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtreeverify.so")
# the benchmark's streaming-read probe (not part of the library)
PROBE_SRC = os.path.join(CSRC, "probe", "tv_probe.hip")
PROBE_LIB = os.path.join(HERE, "libtvprobe.so")
SOURCES = ["tv_api.hip", "tv_mask.hip", "tv_walk.hip", "tv_attn.hip", "tv_gdn.hip", "tv_commit.hip",
           "tv_tree.hip"]
ARCH = os.environ.get("TV_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-result",
        # keep the compiler from emitting packed fp32 arithmetic
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


# per-source additions.  The attention kernels take row maxima of matrix-core
# results, which no NaN reaches unless the inputs hold one: without NaN
# semantics the compiler drops the quieting of each operand before a max.
EXTRA_FLAGS = {"tv_attn.hip": ["-fno-honor-nans"]}


def _compile(src: str, obj: str, verbose: bool):
    cmd = [hipcc(), *flags(), *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", "-o", obj, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel, one process per file),
    then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(srcs, objs)))
    # only show warnings that are not the host pass ignoring the target feature
    noise = "is not a recognized feature for this target"
    failed = False
    for r in results:
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and noise not in ln]
        if r.returncode != 0:
            failed = True
            sys.stderr.write("\n".join(msgs) + "\n")
        elif msgs and verbose:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("HIP build failed")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("HIP link failed")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), *flags(), "-shared", "-o", tmp, PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("probe build failed")
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
