"""ctypes binding of the CPU oracle (oracle/kda_oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline use this module. It never imports the GPU package, and the GPU
package never imports it.

`Oracle(path)` binds one build of the oracle library (the mutation tests bind
deliberately broken copies); the module-level functions use the default build
`oracle/libkda_oracle.so`. Step functions take and return float64 numpy
arrays; the whole-call runner takes bf16 data as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda_oracle.so")

HEAD_DIM = 128
FA_RANK = 128


class Problem(ctypes.Structure):
    _fields_ = [
        ("heads", ctypes.c_int32), ("width", ctypes.c_int32),
        ("requests", ctypes.c_int32), ("tokens", ctypes.c_int32),
        ("projected", ctypes.c_void_p), ("pitch", ctypes.c_int64),
        ("slots", ctypes.c_void_p), ("slots_row_stride", ctypes.c_int64),
        ("accepted", ctypes.c_void_p), ("num_slots", ctypes.c_int32),
        ("conv", ctypes.c_void_p), ("conv_slot_stride", ctypes.c_int64),
        ("conv_dim_stride", ctypes.c_int64), ("conv_pos_stride", ctypes.c_int64),
        ("state", ctypes.c_void_p), ("state_slot_stride", ctypes.c_int64),
        ("conv_weight", ctypes.c_void_p), ("conv_bias", ctypes.c_void_p),
        ("f_b", ctypes.c_void_p), ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("norm_weight", ctypes.c_void_p), ("norm_head_stride", ctypes.c_int32),
        ("gate_lower_bound", ctypes.c_double), ("q_scale", ctypes.c_double),
        ("norm_eps", ctypes.c_double), ("l2_eps", ctypes.c_double),
        ("core_out", ctypes.c_void_p), ("core_out_f64", ctypes.c_void_p),
        ("handoff_bf16", ctypes.c_int32), ("check_distinct", ctypes.c_int32),
    ]


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    assert a.dtype == np.uint16, a.dtype
    return np.ascontiguousarray(a)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (a bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Oracle:
    def __init__(self, path: str = LIB_PATH):
        if path == LIB_PATH and not os.path.exists(path):
            from . import build as _build  # compiling the checker, not a fallback
            _build.build()
        lib = ctypes.CDLL(path)
        d, p, i32 = ctypes.c_double, ctypes.c_void_p, ctypes.c_int32
        lib.kda_ref_sigmoid.argtypes = [d]
        lib.kda_ref_sigmoid.restype = d
        lib.kda_ref_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.kda_ref_bf16_to_double.restype = d
        lib.kda_ref_double_to_bf16.argtypes = [d]
        lib.kda_ref_double_to_bf16.restype = ctypes.c_uint16
        lib.kda_ref_conv_token.argtypes = [i32, i32, p, p, p, p, p]
        lib.kda_ref_conv_token.restype = None
        lib.kda_ref_gate.argtypes = [i32, p, p, p, p, d, i32, p]
        lib.kda_ref_gate.restype = None
        lib.kda_ref_l2norm.argtypes = [i32, p, d, d, p]
        lib.kda_ref_l2norm.restype = None
        lib.kda_ref_recur_token.argtypes = [i32, i32, p, p, p, p, p, d, p]
        lib.kda_ref_recur_token.restype = None
        lib.kda_ref_gated_rmsnorm.argtypes = [i32, p, p, p, d, p]
        lib.kda_ref_gated_rmsnorm.restype = None
        lib.kda_ref_run.argtypes = [ctypes.POINTER(Problem)]
        lib.kda_ref_run.restype = i32
        lib.kda_ref_handoff_ties.argtypes = [ctypes.POINTER(Problem), p, p]
        lib.kda_ref_handoff_ties.restype = i32
        i64 = ctypes.c_int64
        lib.kda_ref_linear.argtypes = [i32, i32, i32, p, i64, p, p, i64, p]
        lib.kda_ref_linear.restype = None
        lib.kda_ref_linear_entries.argtypes = [i32, p, i64, p, i32, p, p, p]
        lib.kda_ref_linear_entries.restype = None
        self.lib = lib
        self.path = path

    # ------------------------------------------------------------ formats
    def bf16_to_f64(self, bits: int) -> float:
        return self.lib.kda_ref_bf16_to_double(int(bits))

    def f64_to_bf16_bits(self, x) -> np.ndarray:
        flat = np.asarray(x, dtype=np.float64).ravel()
        f = self.lib.kda_ref_double_to_bf16
        out = np.fromiter((f(float(v)) for v in flat), dtype=np.uint16, count=flat.size)
        return out.reshape(np.shape(x))

    def sigmoid(self, x: float) -> float:
        return self.lib.kda_ref_sigmoid(float(x))

    # ------------------------------------------------------------ steps
    def conv_token(self, w, bias, win, x):
        """One token of the conv update + SiLU. w [C][W], bias [C] or None,
        win [C][W-1] (oldest first), x [C]. Returns (y [C], new window)."""
        w = _f64(w)
        C, W = w.shape
        win = _f64(win).reshape(C, W - 1).copy()
        x = _f64(x)
        b = None if bias is None else _f64(bias)
        y = np.zeros(C)
        self.lib.kda_ref_conv_token(C, W, _ptr(w), _ptr(b), _ptr(win), _ptr(x), _ptr(y))
        return y, win

    def gate(self, f_b, f_a, A_log, dt_bias, lb, round_g1=False):
        """Decay gate g [D] of one token; f_b [D][128], f_a [128], A_log [H], dt_bias [D].
        With round_g1, g1 = f_b f_a is rounded to bf16 first (the hand-off mode)."""
        f_b, f_a, A_log, dt_bias = _f64(f_b), _f64(f_a), _f64(A_log), _f64(dt_bias)
        H = A_log.size
        assert f_b.shape == (H * HEAD_DIM, FA_RANK) and f_a.size == FA_RANK
        g = np.zeros(H * HEAD_DIM)
        self.lib.kda_ref_gate(H, _ptr(f_b), _ptr(f_a), _ptr(A_log), _ptr(dt_bias), float(lb),
                              int(bool(round_g1)), _ptr(g))
        return g

    def l2norm(self, x, eps, scale=1.0):
        x = _f64(x)
        out = np.zeros_like(x)
        self.lib.kda_ref_l2norm(x.size, _ptr(x), float(eps), float(scale), _ptr(out))
        return out

    def recur_token(self, S, g, k, q, v, beta):
        """One recurrence token on S stored [dv][dk]. Returns (new S, o [dv])."""
        S = _f64(S).copy()
        dv, dk = S.shape
        g, k, q, v = _f64(g), _f64(k), _f64(q), _f64(v)
        o = np.zeros(dv)
        self.lib.kda_ref_recur_token(dk, dv, _ptr(S), _ptr(g), _ptr(k), _ptr(q), _ptr(v),
                                     float(beta), _ptr(o))
        return S, o

    def gated_rmsnorm(self, o, gate_raw, w, eps):
        o, gate_raw, w = _f64(o), _f64(gate_raw), _f64(w)
        y = np.zeros_like(o)
        self.lib.kda_ref_gated_rmsnorm(o.size, _ptr(o), _ptr(gate_raw), _ptr(w), float(eps),
                                       _ptr(y))
        return y

    # ------------------------------------------------------------ projections
    def linear(self, x_bits, w_bits, x_pitch=None, with_f64=True):
        """y = x w^T for bf16 bit patterns x [M][>=K] (rows x_pitch apart) and
        w [N][K]. Returns (y bf16 bits [M][N], y float64 [M][N] or None)."""
        x_bits, w_bits = _u16(x_bits), _u16(w_bits)
        N, K = w_bits.shape
        M = x_bits.shape[0]
        x_pitch = x_bits.shape[1] if x_pitch is None else x_pitch
        y = np.zeros((M, N), np.uint16)
        y64 = np.zeros((M, N), np.float64) if with_f64 else None
        self.lib.kda_ref_linear(M, N, K, _ptr(x_bits), x_pitch, _ptr(w_bits), _ptr(y), N,
                                _ptr(y64))
        return y, y64

    def linear_entries(self, x_bits, w_bits, ms, ns, x_pitch=None):
        """Entries (ms[i], ns[i]) of x w^T in float64."""
        x_bits, w_bits = _u16(x_bits), _u16(w_bits)
        K = w_bits.shape[1]
        x_pitch = x_bits.shape[1] if x_pitch is None else x_pitch
        ms = np.ascontiguousarray(ms, dtype=np.int32)
        ns = np.ascontiguousarray(ns, dtype=np.int32)
        out = np.zeros(ms.size, np.float64)
        self.lib.kda_ref_linear_entries(K, _ptr(x_bits), x_pitch, _ptr(w_bits), ms.size,
                                        _ptr(ms), _ptr(ns), _ptr(out))
        return out

    # ------------------------------------------------------------ whole call
    def run(self, *, heads, width, requests, tokens, projected, pitch, slots, slots_row_stride,
            accepted, num_slots, conv, conv_strides, state, state_slot_stride, conv_weight,
            conv_bias, f_b, A_log, dt_bias, norm_weight, norm_head_stride, gate_lower_bound,
            norm_eps, l2_eps, core_out, q_scale=HEAD_DIM ** -0.5, core_out_f64=None,
            handoff_bf16=False, check_distinct=False, ties=None,
            tie_margins=(0.0, 0.0, 0.0, 0.0)) -> int:
        """One decode (accepted=None) or verify call, in place on host arrays.

        bf16 arrays are uint16 bit patterns. `conv`, `state` (whole pools) and
        `core_out` must be C-contiguous numpy arrays; they are updated in
        place. Returns the number of skipped requests.

        handoff_bf16 rounds conv out, g1 and o to bf16 where produced. A slot
        named as a destination twice makes the call undefined (ValueError,
        nothing written) unless check_distinct, which skips and counts every
        request involved. `ties` (checker instrumentation, hand-off mode only),
        an int32 array [R, H, 4] zeroed by the caller, receives per (request,
        head) the near-tie counts of conv out, g1, o and core_out under the
        relative margins `tie_margins` (conv, g1, o, core_out); they are
        counted by a separate read-only replay before the call runs."""
        projected = _u16(projected)
        slots = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
        acc = None if accepted is None else np.ascontiguousarray(
            np.asarray(accepted, dtype=np.int32))
        for name, arr in (("conv", conv), ("state", state), ("core_out", core_out)):
            assert isinstance(arr, np.ndarray) and arr.flags.c_contiguous, name
        assert conv.dtype == np.uint16 and state.dtype == np.float32
        assert core_out.dtype == np.uint16
        conv_weight = _u16(conv_weight)
        conv_bias = None if conv_bias is None else _u16(conv_bias)
        f_b = _u16(f_b)
        A_log = np.ascontiguousarray(np.asarray(A_log, dtype=np.float32))
        dt_bias = np.ascontiguousarray(np.asarray(dt_bias, dtype=np.float32))
        norm_weight = np.ascontiguousarray(np.asarray(norm_weight, dtype=np.float32))
        if core_out_f64 is not None:
            assert core_out_f64.dtype == np.float64 and core_out_f64.flags.c_contiguous
        if ties is not None:
            assert ties.dtype == np.int32 and ties.flags.c_contiguous
            assert ties.size == requests * heads * 4
        pr = Problem(
            heads=heads, width=width, requests=requests, tokens=tokens,
            projected=_ptr(projected), pitch=pitch, slots=_ptr(slots),
            slots_row_stride=slots_row_stride, accepted=_ptr(acc), num_slots=num_slots,
            conv=_ptr(conv), conv_slot_stride=conv_strides[0], conv_dim_stride=conv_strides[1],
            conv_pos_stride=conv_strides[2], state=_ptr(state),
            state_slot_stride=state_slot_stride, conv_weight=_ptr(conv_weight),
            conv_bias=_ptr(conv_bias), f_b=_ptr(f_b), A_log=_ptr(A_log),
            dt_bias=_ptr(dt_bias), norm_weight=_ptr(norm_weight),
            norm_head_stride=norm_head_stride, gate_lower_bound=gate_lower_bound,
            q_scale=q_scale, norm_eps=norm_eps, l2_eps=l2_eps, core_out=_ptr(core_out),
            core_out_f64=_ptr(core_out_f64), handoff_bf16=int(bool(handoff_bf16)),
            check_distinct=int(bool(check_distinct)))
        if ties is not None:
            assert handoff_bf16, "near ties are counted for the hand-off mode"
            rel = np.ascontiguousarray(np.asarray(tie_margins, dtype=np.float64))
            assert rel.size == 4
            if self.lib.kda_ref_handoff_ties(ctypes.byref(pr), _ptr(rel), _ptr(ties)) < 0:
                raise ValueError("oracle rejected the problem description")
        rc = self.lib.kda_ref_run(ctypes.byref(pr))
        if rc < 0:
            raise ValueError("oracle rejected the problem description")
        return rc


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
