"""Runs a seeded case from kda_inputs through the HIP library (test infrastructure).

Device tensors are plain copies of the case's CPU tensors; every view (the
transposed conv cache, a strided block-table slice of slots) is rebuilt on the
device with the same strides, so the library sees the same layout the oracle
walks."""
from __future__ import annotations

import numpy as np
import torch

import kimi_delta_attention_conv_amd as kda
from kda_inputs import Case

_FROM_CASE = object()
OUT_SENTINEL = 0x7FC1  # a NaN pattern no kernel result can equal by accident


def _strided_to_device(t: torch.Tensor) -> torch.Tensor:
    """Copies the storage span a strided view walks, and re-views it on the device."""
    if t.is_contiguous():
        return t.cuda()
    span = 1 + sum((s - 1) * st for s, st in zip(t.shape, t.stride()))
    flat = torch.as_strided(t, (span,), (1,), t.storage_offset()).contiguous().cuda()
    return torch.as_strided(flat, t.shape, t.stride(), 0)


class GpuCase:
    """Device copies of a case and a KdaCore bound to them."""

    def __init__(self, case: Case, *, projected=None, conv_storage=None, state=None,
                 norm_weight=None, dt_bias=None, gate_lower_bound=None, rounding="fused",
                 check_distinct=False):
        self.case = case
        self.projected = (case.projected if projected is None else projected).cuda()
        st = case.conv_storage if conv_storage is None else conv_storage
        self.conv_storage = st.cuda()
        self.conv = self.conv_storage if case.conv_dim_first else self.conv_storage.transpose(-1, -2)
        self.state = (case.state if state is None else state).cuda()
        self.core = kda.KdaCore(
            conv_weight=case.conv_weight.cuda(),
            conv_bias=None if case.conv_bias is None else case.conv_bias.cuda(),
            f_b=case.f_b.cuda(), A_log=case.A_log.cuda(),
            dt_bias=(case.dt_bias if dt_bias is None else torch.as_tensor(dt_bias)).cuda(),
            norm_weight=(case.norm_weight if norm_weight is None else torch.as_tensor(norm_weight)).cuda(),
            gate_lower_bound=case.gate_lower_bound if gate_lower_bound is None else gate_lower_bound,
            norm_eps=case.norm_eps, l2_eps=case.l2_eps, conv=self.conv, state=self.state,
            rounding=rounding, check_distinct=check_distinct)
        self.out = torch.full((case.S, case.D), OUT_SENTINEL, dtype=torch.int16).view(
            torch.bfloat16).cuda()

    def run(self, *, slots=None, accepted=_FROM_CASE, projected=None, decode=None):
        c = self.case
        slots = _strided_to_device(c.slots if slots is None else slots)
        acc = c.accepted if accepted is _FROM_CASE else accepted
        proj = self.projected if projected is None else projected.cuda()
        use_decode = (acc is None) if decode is None else decode
        if use_decode:
            self.core.decode(proj, self.out, slots.reshape(-1) if slots.dim() == 2 else slots)
        else:
            if slots.dim() == 1:
                slots = slots.view(-1, 1)
            self.core.verify(proj, self.out, slots, torch.as_tensor(acc, dtype=torch.int32).cuda())
        torch.cuda.synchronize()
        return self

    def host(self):
        torch.cuda.synchronize()
        return dict(
            out=self.out.cpu().view(torch.int16).numpy().view(np.uint16).copy(),
            conv=self.conv_storage.cpu().view(torch.int16).numpy().view(np.uint16).copy(),
            state=self.state.cpu().numpy().copy(),
            errors=self.core.device_errors(),
        )

    def close(self):
        self.core.close()


def run_gpu(case: Case, **kw) -> dict:
    run_kw = {k: kw.pop(k) for k in ("slots", "accepted", "decode") if k in kw}
    g = GpuCase(case, **kw)
    try:
        g.run(**run_kw)
        return g.host()
    finally:
        g.close()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)
