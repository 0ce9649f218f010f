"""Runs the CPU oracle on a seeded case from kda_inputs (test infrastructure)."""
from __future__ import annotations

import numpy as np
import torch

import oracle as oracle_mod
from kda_inputs import Case


def bf16_np(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (same shape, contiguous copy)."""
    return t.detach().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def slots_flat(case: Case) -> np.ndarray:
    """The slots operand as the flat int32 span the row stride walks over."""
    s = case.slots
    if s.dim() == 1:
        return s.contiguous().numpy().copy()
    R, L = s.shape
    span = (R - 1) * s.stride(0) + L if R > 0 else 0
    flat = torch.as_strided(s, (span,), (1,), s.storage_offset())
    return flat.contiguous().numpy().copy()


_FROM_CASE = object()


def run_oracle(case: Case, orc: oracle_mod.Oracle | None = None, *, projected=None,
               accepted=_FROM_CASE, conv_storage=None, state=None, with_f64=True, **overrides):
    """Runs one call of the case on copies of its pools.

    Returns dict(out [S, D] uint16, out_f64, conv (storage layout, uint16),
    state (float32 pool), skipped)."""
    orc = orc or oracle_mod.default()
    D = case.D
    S = case.S
    conv = bf16_np(case.conv_storage if conv_storage is None else conv_storage)
    st = (case.state if state is None else state).numpy().copy()
    out = np.zeros((S, D), dtype=np.uint16)
    out64 = np.zeros((S, D), dtype=np.float64) if with_f64 else None
    acc = case.accepted if accepted is _FROM_CASE else accepted
    kw = dict(
        heads=case.H, width=case.W, requests=case.R, tokens=case.L,
        projected=bf16_np(case.projected if projected is None else projected),
        pitch=case.pitch, slots=slots_flat(case), slots_row_stride=case.slots_row_stride(),
        accepted=None if acc is None else np.asarray(acc, dtype=np.int32),
        num_slots=case.num_slots, conv=conv.reshape(-1), conv_strides=case.conv_strides(),
        state=st.reshape(-1), state_slot_stride=case.H * 128 * 128,
        conv_weight=bf16_np(case.conv_weight),
        conv_bias=None if case.conv_bias is None else bf16_np(case.conv_bias),
        f_b=bf16_np(case.f_b), A_log=case.A_log.numpy(), dt_bias=case.dt_bias.numpy(),
        norm_weight=case.norm_weight.numpy(), norm_head_stride=0,
        gate_lower_bound=case.gate_lower_bound, norm_eps=case.norm_eps, l2_eps=case.l2_eps,
        core_out=out, core_out_f64=out64)
    kw.update(overrides)
    skipped = orc.run(**kw)
    return dict(out=out, out_f64=out64, conv=conv, state=st, skipped=skipped)
