"""Builds the HIP library libtsd_attn.so in-tree for gfx950 with hipcc.

    python -m transformer_scaled_dot_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtsd_attn.so")
SOURCES = ["attn_fwd_bf16.hip", "attn_bwd_bf16.hip", "attn_fwd_f32.hip", "attn_weights.hip", "gemm_bf16.hip",
           "capi.hip"]
# the benchmark's clock probe: a library of its own, outside the attention library and its C ABI
PROBE_LIB = os.path.join(HERE, "libtsd_probe.so")
PROBE_SOURCES = [os.path.join("probe", "clock_probe.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


COMMON_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-I" + INCLUDE, "-I" + CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, out: str) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libtsd_attn.so (and the benchmark's libtsd_probe.so) next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
