"""ctypes binding of libkda_probe.so, the HBM stream probes of include/kda_probe.h.

Measurement only: plain read / write / copy streams (the achievable HBM rates
and the counter calibration) and the core kernel's state traffic replayed
without its arithmetic (the ceiling of its access pattern). Nothing in the
product path loads this library.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda_probe.so")

BARRIER = 1            # KDA_PROBE_BARRIER
CORE_OCCUPANCY = 2     # KDA_PROBE_CORE_OCCUPANCY

_lib = None


def load_probe_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m kimi_delta_attention_conv_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.kda_probe_copy.argtypes = [vp, vp, i64, vp]
    lib.kda_probe_write.argtypes = [vp, i64, ctypes.c_float, vp]
    lib.kda_probe_read.argtypes = [vp, i64, vp, vp]
    lib.kda_probe_copy_runs.argtypes = [vp, vp, i64, vp]
    lib.kda_probe_write_runs.argtypes = [vp, i64, ctypes.c_float, vp]
    lib.kda_probe_state_stream.argtypes = [vp, i64, i32, vp, i64, vp, i32, i32, i32, i32, vp]
    for f in (lib.kda_probe_copy, lib.kda_probe_write, lib.kda_probe_read, lib.kda_probe_copy_runs,
              lib.kda_probe_write_runs, lib.kda_probe_state_stream):
        f.restype = ctypes.c_int
    lib.kda_probe_sink_floats.argtypes = []
    lib.kda_probe_sink_floats.restype = i32
    _lib = lib
    return lib
