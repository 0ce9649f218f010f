"""Python binding of libkda.so, the gfx950 KDA decode / spec-verify core.

The functions below carry the C ABI's names (include/kda.h) and only marshal
arguments; all work runs in the library's HIP kernels. `KdaCore` wraps them
for torch tensors (device memory and the current HIP stream come from torch;
nothing is computed by torch).

The library must have been built (`python -m kimi_delta_attention_conv_amd.build`):
there is no fallback path, and loading fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "KdaError", "KdaWeights", "KdaCaches", "load_library", "kda_prepare", "kda_decode",
    "kda_verify", "kda_device_errors", "kda_destroy", "kda_status_string", "KdaCore",
    "kda_linear", "kda_linear_workspace_bytes", "kda_in_proj", "kda_o_proj", "linear",
    "kda_linear_noalloc", "kda_noalloc_scratch_bytes",
    "HEAD_DIM", "FA_RANK", "CONV_WIDTH", "MAX_TOKENS", "ROUNDING",
]

HEAD_DIM = 128
FA_RANK = 128
CONV_WIDTH = 4
MAX_TOKENS = 8
# kda_rounding: fused (fp32 intermediates) or bf16 at the unfused path's hand-offs
ROUNDING = {"fused": 0, "bf16_handoff": 1}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

STATUS = {0: "KDA_OK", -1: "KDA_ERR_NULL", -2: "KDA_ERR_SHAPE", -3: "KDA_ERR_ALIGN",
          -4: "KDA_ERR_UNSUPPORTED", -5: "KDA_ERR_HIP", -6: "KDA_ERR_NOMEM", -7: "KDA_ERR_DEVICE",
          -8: "KDA_ERR_SCRATCH"}


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        name = STATUS.get(status, str(status))
        msg = f"{where}: {name}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


class KdaWeights(ctypes.Structure):
    _fields_ = [
        ("heads", ctypes.c_int32), ("conv_width", ctypes.c_int32),
        ("conv_weight", ctypes.c_void_p), ("conv_bias", ctypes.c_void_p),
        ("f_b", ctypes.c_void_p), ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("norm_weight", ctypes.c_void_p), ("norm_head_stride", ctypes.c_int32),
        ("gate_lower_bound", ctypes.c_float), ("norm_eps", ctypes.c_float),
        ("l2_eps", ctypes.c_float), ("rounding", ctypes.c_int32),
        ("A_log_dtype", ctypes.c_int32), ("dt_bias_dtype", ctypes.c_int32),
        ("norm_weight_dtype", ctypes.c_int32),
    ]


class KdaCaches(ctypes.Structure):
    _fields_ = [
        ("conv", ctypes.c_void_p), ("conv_slot_stride", ctypes.c_int64),
        ("conv_dim_stride", ctypes.c_int64), ("conv_pos_stride", ctypes.c_int64),
        ("state", ctypes.c_void_p), ("state_slot_stride", ctypes.c_int64),
        ("num_slots", ctypes.c_int32), ("check_distinct", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libkda.so once; raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built: run `python -m kimi_delta_attention_conv_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.kda_prepare.argtypes = [ctypes.POINTER(KdaWeights), ctypes.POINTER(KdaCaches), vp,
                                ctypes.POINTER(vp)]
    lib.kda_decode.argtypes = [vp, vp, i64, i32, vp, vp, vp]
    lib.kda_verify.argtypes = [vp, vp, i64, i32, i32, vp, i64, vp, vp, vp]
    lib.kda_device_errors.argtypes = [vp, ctypes.POINTER(i32), vp]
    lib.kda_destroy.argtypes = [vp]
    for f in (lib.kda_prepare, lib.kda_decode, lib.kda_verify, lib.kda_device_errors,
              lib.kda_destroy):
        f.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_hip_error.argtypes = []
    lib.kda_last_hip_error.restype = ctypes.c_char_p
    sz = ctypes.c_size_t
    lib.kda_linear.argtypes = [vp, i64, vp, vp, i64, i32, i32, i32, vp, sz, vp]
    lib.kda_in_proj.argtypes = [vp, i64, vp, vp, i64, i32, i32, i32, vp, sz, vp]
    lib.kda_o_proj.argtypes = [vp, i64, vp, vp, i64, i32, i32, i32, vp, sz, vp]
    for f in (lib.kda_linear, lib.kda_in_proj, lib.kda_o_proj):
        f.restype = ctypes.c_int
    lib.kda_linear_workspace_bytes.argtypes = [i32, i32, i32]
    lib.kda_linear_workspace_bytes.restype = sz
    lib.kda_linear_noalloc.argtypes = [vp, i64, vp, vp, i64, i32, i32, i32, vp]
    lib.kda_linear_noalloc.restype = ctypes.c_int
    lib.kda_noalloc_scratch_bytes.argtypes = []
    lib.kda_noalloc_scratch_bytes.restype = sz
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        lib = load_library()
        detail = lib.kda_status_string(status).decode()
        if status == -5:
            detail += ": " + lib.kda_last_hip_error().decode()
        raise KdaError(status, where, detail)


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(status).decode()


def kda_prepare(weights: KdaWeights, caches: KdaCaches, stream: int = 0) -> int:
    """Returns the handle (an opaque integer)."""
    h = ctypes.c_void_p()
    _check(load_library().kda_prepare(ctypes.byref(weights), ctypes.byref(caches),
                                      ctypes.c_void_p(stream), ctypes.byref(h)), "kda_prepare")
    return h.value


def kda_decode(handle: int, projected: int, pitch: int, batch: int, slots: int, core_out: int,
               stream: int = 0) -> None:
    _check(load_library().kda_decode(handle, projected, pitch, batch, slots, core_out, stream),
           "kda_decode")


def kda_verify(handle: int, projected: int, pitch: int, requests: int, tokens: int, slots: int,
               slots_row_stride: int, accepted: int, core_out: int, stream: int = 0) -> None:
    _check(load_library().kda_verify(handle, projected, pitch, requests, tokens, slots,
                                     slots_row_stride, accepted, core_out, stream), "kda_verify")


def kda_linear(x: int, x_pitch: int, w: int, y: int, y_pitch: int, M: int, N: int, K: int,
               workspace: int = 0, workspace_bytes: int = 0, stream: int = 0) -> None:
    _check(load_library().kda_linear(x, x_pitch, w, y, y_pitch, M, N, K, workspace,
                                     workspace_bytes, stream), "kda_linear")


def kda_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load_library().kda_linear_workspace_bytes(M, N, K))


def kda_linear_noalloc(x: int, x_pitch: int, w: int, y: int, y_pitch: int, M: int, N: int,
                       K: int, stream: int = 0) -> None:
    _check(load_library().kda_linear_noalloc(x, x_pitch, w, y, y_pitch, M, N, K, stream),
           "kda_linear_noalloc")


def kda_noalloc_scratch_bytes() -> int:
    return int(load_library().kda_noalloc_scratch_bytes())


def kda_in_proj(x: int, x_pitch: int, w_in: int, projected: int, pitch: int, rows: int,
                hidden: int, heads: int, workspace: int = 0, workspace_bytes: int = 0,
                stream: int = 0) -> None:
    _check(load_library().kda_in_proj(x, x_pitch, w_in, projected, pitch, rows, hidden, heads,
                                      workspace, workspace_bytes, stream), "kda_in_proj")


def kda_o_proj(core: int, core_pitch: int, w_o: int, out: int, out_pitch: int, rows: int,
               heads: int, hidden: int, workspace: int = 0, workspace_bytes: int = 0,
               stream: int = 0) -> None:
    _check(load_library().kda_o_proj(core, core_pitch, w_o, out, out_pitch, rows, heads, hidden,
                                     workspace, workspace_bytes, stream), "kda_o_proj")


def _stream_of(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def linear(x, w, y=None, stream=None, workspace="auto"):
    """y = x w^T for bf16 device tensors x [M, >=K] (unit column stride), w [N, K]
    (dense); y [M, >=N] is allocated when not given. `workspace`: "auto"
    allocates the split-K workspace kda_linear_workspace_bytes asks for (none for
    shapes that do not split), None passes none (the unsplit kernel), a device
    tensor is used as given. Returns y."""
    import torch
    M, N, K = x.shape[0], w.shape[0], w.shape[1]
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("x and w must be bfloat16")
    if not (x.is_cuda and w.is_cuda and (y is None or y.is_cuda)) or w.device != x.device or \
            (y is not None and y.device != x.device):
        raise TypeError("x, w and y must be tensors on one GPU")
    if x.stride(1) != 1 or not w.is_contiguous() or x.shape[1] < K:
        raise ValueError("x needs unit column stride and >= K columns; w must be dense [N, K]")
    if y is None:
        y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
    if y.dtype != torch.bfloat16 or y.stride(1) != 1 or y.shape[0] < M or y.shape[1] < N:
        raise ValueError("y must be bfloat16 [>= M, >= N] with unit column stride")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a device tensor')
        nbytes = kda_linear_workspace_bytes(M, N, K) if M > 0 else 0
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
    if workspace is not None and (not workspace.is_cuda or workspace.device != x.device or
                                  not workspace.is_contiguous()):
        raise TypeError("workspace must be a contiguous tensor on x's GPU")
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(x.device):   # launch on the tensors' device (its current stream)
        kda_linear(x.data_ptr(), x.stride(0), w.data_ptr(), y.data_ptr(), y.stride(0), M, N, K,
                   ws_ptr, ws_bytes, _stream_of(stream))
    return y


def kda_device_errors(handle: int, stream: int = 0) -> int:
    n = ctypes.c_int32()
    _check(load_library().kda_device_errors(handle, ctypes.byref(n), stream), "kda_device_errors")
    return n.value


def kda_destroy(handle: int) -> None:
    _check(load_library().kda_destroy(handle), "kda_destroy")


class KdaCore:
    """One KDA layer's core bound to its weights and slot caches (torch tensors).

    conv   : bf16 logical view [slots, 3D, 3] of the conv window cache (dim
             first, or the transposed view of [slots, 3, 3D] storage).
    state  : fp32 [slots, H, 128, 128] (slot stride may exceed H*128*128).
    Weights: conv_weight bf16 [3D, 1, 4]; conv_bias bf16 [3D] or None; f_b bf16
             [D, 128]; A_log [H], dt_bias [D], norm_weight [128] or [H, 128], each
             fp32 or bf16 (converted to fp32 at prepare time).
    rounding: "fused" (default) or "bf16_handoff" (kda_rounding in kda.h).
    check_distinct: make every call skip and count requests whose destination
             slots collide (kda_caches.check_distinct in kda.h).
    """

    def __init__(self, *, conv_weight, conv_bias, f_b, A_log, dt_bias, norm_weight,
                 gate_lower_bound, norm_eps, conv, state, l2_eps=1e-6, stream=None,
                 rounding="fused", check_distinct=False):
        import torch

        self._torch = torch
        H = int(A_log.numel())
        D = H * HEAD_DIM
        for name, t, dt in (("conv_weight", conv_weight, torch.bfloat16),
                            ("f_b", f_b, torch.bfloat16),
                            ("conv", conv, torch.bfloat16), ("state", state, torch.float32)):
            if t.dtype != dt or not t.is_cuda:
                raise TypeError(f"{name} must be a {dt} device tensor")
        small_dtypes = {torch.float32: 0, torch.bfloat16: 1}   # kda_dtype
        for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("norm_weight", norm_weight)):
            if t.dtype not in small_dtypes or not t.is_cuda:
                raise TypeError(f"{name} must be a float32 or bfloat16 device tensor")
        if conv_bias is not None and (conv_bias.dtype != torch.bfloat16 or not conv_bias.is_cuda):
            raise TypeError("conv_bias must be a bfloat16 device tensor or None")
        for name, t in (("conv_weight", conv_weight), ("f_b", f_b), ("A_log", A_log),
                        ("dt_bias", dt_bias), ("norm_weight", norm_weight)):
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if conv_weight.numel() != 3 * D * CONV_WIDTH or f_b.shape != (D, FA_RANK):
            raise ValueError("weight shapes do not match A_log's head count")
        if conv.dim() != 3 or conv.shape[1] != 3 * D or conv.shape[2] != CONV_WIDTH - 1:
            raise ValueError("conv must be a [slots, 3D, 3] view")
        if state.dim() != 4 or tuple(state.shape[1:]) != (H, HEAD_DIM, HEAD_DIM) or \
                state.stride()[1:] != (HEAD_DIM * HEAD_DIM, HEAD_DIM, 1):
            raise ValueError("state must be [slots, H, 128, 128] with dense slots")
        if norm_weight.numel() not in (HEAD_DIM, D):
            raise ValueError("norm_weight must have 128 or H*128 elements")
        self.heads, self.dim = H, D
        self.device = state.device
        for name, t in (("conv_weight", conv_weight), ("f_b", f_b), ("A_log", A_log),
                        ("dt_bias", dt_bias), ("norm_weight", norm_weight), ("conv", conv)):
            if t.device != self.device:
                raise TypeError(f"{name} is on {t.device}, the state pool on {self.device}")
        self.conv, self.state = conv, state
        w = KdaWeights(heads=H, conv_width=CONV_WIDTH, conv_weight=conv_weight.data_ptr(),
                       conv_bias=None if conv_bias is None else conv_bias.data_ptr(),
                       f_b=f_b.data_ptr(), A_log=A_log.data_ptr(), dt_bias=dt_bias.data_ptr(),
                       norm_weight=norm_weight.data_ptr(),
                       norm_head_stride=0 if norm_weight.numel() == HEAD_DIM else HEAD_DIM,
                       gate_lower_bound=float(gate_lower_bound), norm_eps=float(norm_eps),
                       l2_eps=float(l2_eps), rounding=ROUNDING[rounding],
                       A_log_dtype=small_dtypes[A_log.dtype], dt_bias_dtype=small_dtypes[dt_bias.dtype],
                       norm_weight_dtype=small_dtypes[norm_weight.dtype])
        cs = conv.stride()
        c = KdaCaches(conv=conv.data_ptr(), conv_slot_stride=cs[0], conv_dim_stride=cs[1],
                      conv_pos_stride=cs[2], state=state.data_ptr(),
                      state_slot_stride=state.stride(0), num_slots=int(state.shape[0]),
                      check_distinct=int(bool(check_distinct)))
        if conv.shape[0] != state.shape[0]:
            raise ValueError("conv and state pools must have the same slot count")
        # the handle belongs to the device current at prepare time: the pools' device
        with torch.cuda.device(self.device):
            self.handle = kda_prepare(w, c, self._stream(stream))
            torch.cuda.synchronize()   # the caller's weights may be released from here on

    def _stream(self, stream):
        if stream is None:
            return self._torch.cuda.current_stream().cuda_stream
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)

    def _on_device(self, **tensors):
        for name, t in tensors.items():
            if not t.is_cuda or t.device != self.device:
                raise TypeError(f"{name} must be on {self.device} (the core's device)")

    def _rows(self, projected, out):
        torch = self._torch
        if projected.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
            raise TypeError("projected and out must be bfloat16")
        self._on_device(projected=projected, out=out)
        if projected.dim() == 2 and projected.shape[1] < 4 * self.dim + FA_RANK + self.heads:
            raise ValueError("projected rows hold fewer than 4D + 128 + H columns")
        if projected.dim() != 2 or projected.stride(1) != 1 or out.dim() != 2 or \
                out.stride(1) != 1 or out.shape[1] != self.dim or out.stride(0) != self.dim:
            raise ValueError("projected [S, pitch] and out [S, D] must be row-major")
        if out.shape[0] < projected.shape[0]:
            raise ValueError("out has fewer rows than projected")
        return projected.stride(0)

    def decode(self, projected, out, slots, stream=None):
        """projected bf16 [B, pitch], out bf16 [B, D], slots int32 [B] (in place)."""
        pitch = self._rows(projected, out)
        self._on_device(slots=slots)
        if slots.dtype != self._torch.int32 or slots.dim() != 1 or slots.stride(0) != 1:
            raise ValueError("slots must be a dense int32 [B] tensor")
        B = projected.shape[0]
        if slots.shape[0] < B:
            raise ValueError("fewer slots than rows")
        kda_decode(self.handle, projected.data_ptr(), pitch, B, slots.data_ptr(), out.data_ptr(),
                   self._stream(stream))
        return out

    def verify(self, projected, out, slots, accepted, stream=None):
        """projected bf16 [R*L, pitch], out bf16 [R*L, D], slots int32 [>= R, L] (row
        stride >= L, unit column stride), accepted int32 [>= R]."""
        pitch = self._rows(projected, out)
        torch = self._torch
        self._on_device(slots=slots, accepted=accepted)
        if slots.dtype != torch.int32 or slots.dim() != 2 or slots.stride(1) != 1:
            raise ValueError("slots must be int32 [R, L] with unit column stride")
        if accepted.dtype != torch.int32 or accepted.dim() != 1 or accepted.stride(0) != 1:
            raise ValueError("accepted must be a dense int32 [R] tensor")
        L = slots.shape[1]
        if projected.shape[0] % L != 0:
            raise ValueError("projected rows are not a multiple of the verify length")
        R = projected.shape[0] // L
        if slots.shape[0] < R or accepted.shape[0] < R:
            raise ValueError("slots / accepted cover fewer requests than projected")
        kda_verify(self.handle, projected.data_ptr(), pitch, R, L, slots.data_ptr(),
                   slots.stride(0), accepted.data_ptr(), out.data_ptr(), self._stream(stream))
        return out

    def device_errors(self, stream=None) -> int:
        return kda_device_errors(self.handle, self._stream(stream))

    def close(self):
        if getattr(self, "handle", None):
            kda_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
