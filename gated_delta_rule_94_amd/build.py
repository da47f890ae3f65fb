"""Build libkda.so (HIP, gfx950) in-tree with hipcc, and its debug build libkda_debug.so.

The library is compiled for gfx950 only.  The debug build is the same library with the C ABI's
translation unit compiled with KDA_DEBUG_CHECKS: every entry point first checks g and beta against
the documented input envelope on the GPU (include/kda.h).  Every HIP source is built with
packed fp32 instructions disabled (``-Xclang -target-feature -Xclang
-packed-fp32-ops``); hipcc's host pass warns that it does not know the feature,
which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
DEBUG_LIB = os.path.join(HERE, "libkda_debug.so")
SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_prefill.hip", "kda_intra.hip", "kda_chain.hip", "kda_backward.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, out_dir: str, extra=(), suffix: str = "") -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source, link libkda.so and libkda_debug.so next to this file; returns the
    path of libkda.so."""
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    jobs = [(s, (), "") for s in SOURCES] + [("kda_api.hip", ("-DKDA_DEBUG_CHECKS",), "_debug")]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], out_dir, j[1], j[2]), jobs))
    release, debug_api = objs[:len(SOURCES)], objs[len(SOURCES)]
    _link(release, LIB)
    _link([debug_api if s == "kda_api.hip" else o for s, o in zip(SOURCES, release)], DEBUG_LIB)
    if verbose:
        print("built", LIB, "and", DEBUG_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
