"""Builds libkda.so (the C-ABI library of include/kda.h) and libkda_probe.so (the
measurement-only HBM probes of include/kda_probe.h) for gfx950 with hipcc.

    python -m kimi_delta_attention_conv_amd.build      # or build() from Python

Cross-compiles without a GPU. The libraries land next to this file, where the
Python bindings load them.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
PROBE_LIB = os.path.join(PKG, "libkda_probe.so")
SOURCES = [os.path.join(CSRC, f) for f in ("kda_core.hip", "kda_linear.hip", "kda_api.cpp",
                                            "kda_noalloc.hip")]
PROBE_SOURCES = [os.path.join(CSRC, "hbm_probe.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 arithmetic (v_pk_*_f32) is disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _link(sources, lib, build_dir, verbose):
    objs = []
    for src in sources:
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c", src, "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compiles every source to an object and links both libraries; returns
    the product library's path."""
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    _link(SOURCES, LIB, build_dir, verbose)
    _link(PROBE_SOURCES, PROBE_LIB, build_dir, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
