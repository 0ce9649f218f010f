"""Seeded synthetic inputs for the KDA decode / spec-verify core.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the CPU oracle's tests and the GPU path's tests (and
the benchmark) take their inputs from here, so the two sides see identical
bytes.

Shapes follow the pages: one tensor-parallel rank's share of 12 heads of 128
channels, f_a rank 128, a width-4 conv over the packed q|k|v channels, and a
packed projection row q|k|v (3D) | gate (D) | f_a (128) | beta (H)
(page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.prepared",
PreparedKda._operands).

Draw order for one case, from one CPU torch.Generator seeded with the case's
seed (fp32 draws; bf16 by round-to-nearest-even cast):
  1. projected [S, pitch]            ~ N(0, 1)
  2. conv weight [3D, W]             ~ N(0, 0.5^2)   -> bf16, viewed [3D, 1, W]
  3. conv bias [3D]                  ~ N(0, 0.1^2)   -> bf16
  4. conv cache pool                 ~ N(0, 1)       -> bf16, stored [slots, 3D, W-1]
                                                        or [slots, W-1, 3D] (transposed)
  5. state pool [slots, H, 128, 128] ~ N(0, 0.05^2)  fp32
  6. f_b [D, 128]                    ~ N(0, 0.09^2)  -> bf16
  7. A_log [H]                       ~ U(a_lo, a_hi) fp32
  8. dt_bias [D]                     ~ U(-1, 1)      fp32
  9. o_norm weight [128]             ~ U(0.5, 1.5)   fp32
 10. slots: a random permutation of the pool (distinct slots), or a fixed slot
 11. accepted [R]                    ~ U{1 .. L}     int32 (verify only)
 12. beta_raw columns [S, H]         ~ N(0, beta_std^2), written over the
                                       projected beta columns (only when
                                       beta_std != 1)

 13. coarse gate operands (only with coarse_gate): f_b [D, 128] = k 2^-8 and the
     projected f_a columns [S, 128] = k 2^-4, k ~ U{-31 .. 31} (f_b first). Every
     product is a multiple of 2^-12 and a sum of 128 of them stays below 2^12, so
     g1 = f_b f_a is exact in fp32 in any summation order.

With `pool_device` set (pools of many gigabytes), steps 4 and 5 are drawn instead
on that device, from a generator of that device seeded with the case's seed
(conv pool first, then state pool), and the CPU generator goes on at step 6.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

HEAD_DIM = 128
FA_RANK = 128
CONV_WIDTH = 4


@dataclasses.dataclass
class Case:
    name: str
    seed: int
    R: int
    L: int
    H: int
    W: int
    num_slots: int
    pitch: int
    verify: bool
    projected: torch.Tensor          # bf16 [S, pitch]
    conv_weight: torch.Tensor        # bf16 [3D, 1, W]
    conv_bias: Optional[torch.Tensor]  # bf16 [3D] or None
    conv_storage: torch.Tensor       # bf16, [slots, 3D, W-1] or [slots, W-1, 3D]
    conv_dim_first: bool
    state: torch.Tensor              # fp32 [slots, H, 128, 128]
    f_b: torch.Tensor                # bf16 [D, 128]
    A_log: torch.Tensor              # fp32 [H]
    dt_bias: torch.Tensor            # fp32 [D]
    norm_weight: torch.Tensor        # fp32 [128]
    slots: torch.Tensor              # int32 [R] (decode) or [R, L] view (verify)
    accepted: Optional[torch.Tensor]  # int32 [R] or None
    gate_lower_bound: float = -5.0
    norm_eps: float = 1e-6
    l2_eps: float = 1e-6

    @property
    def D(self) -> int:
        return self.H * HEAD_DIM

    @property
    def S(self) -> int:
        return self.R * self.L

    def conv_view(self) -> torch.Tensor:
        """The conv cache as a logical [slots, 3D, W-1] view (dim first)."""
        return self.conv_storage if self.conv_dim_first else self.conv_storage.transpose(-1, -2)

    def conv_strides(self):
        return tuple(self.conv_view().stride())

    def slots_row_stride(self) -> int:
        return self.slots.stride(0) if self.slots.dim() == 2 else 1


# name, R, L, H, pool slots, seed, and per-config options
CONFIGS = {
    0: dict(name="tiny_decode_r1_h2", R=1, L=1, H=2, num_slots=4, seed=0, fixed_slot=2),
    1: dict(name="decode_r64", R=64, L=1, H=12, num_slots=128, seed=1),
    2: dict(name="verify_r16_l4", R=16, L=4, H=12, num_slots=128, seed=2, verify=True),
    3: dict(name="verify_r64_l8", R=64, L=8, H=12, num_slots=1024, seed=3, verify=True,
            block_table_cols=16),
    4: dict(name="decode_r256", R=256, L=1, H=12, num_slots=1024, seed=4,
            conv_dim_first=False, beta_std=2.0, a_log_range=(-3.0, 2.0)),
}


def default_pitch(H: int) -> int:
    """4D + 128 + H elements: the packed row with no padding (odd for odd H)."""
    return 4 * H * HEAD_DIM + FA_RANK + H


def make_case(R: int, L: int, H: int, num_slots: int, seed: int, *, name: str = "custom",
              verify: Optional[bool] = None, pitch: Optional[int] = None,
              conv_dim_first: bool = True, with_bias: bool = True, beta_std: float = 1.0,
              a_log_range=(-1.0, 1.0), fixed_slot: Optional[int] = None,
              block_table_cols: Optional[int] = None, W: int = CONV_WIDTH,
              pool_device: Optional[str] = None, coarse_gate: bool = False) -> Case:
    if verify is None:
        verify = L > 1
    if not verify and L != 1:
        raise ValueError("a decode case has one token a request")
    D = H * HEAD_DIM
    C = 3 * D
    S = R * L
    pitch = default_pitch(H) if pitch is None else pitch
    gen = torch.Generator().manual_seed(seed)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32)

    def rand(*shape):
        return torch.rand(*shape, generator=gen, dtype=torch.float32)

    projected = randn(S, pitch).to(torch.bfloat16)
    conv_weight = (randn(C, W) * 0.5).to(torch.bfloat16).view(C, 1, W)
    bias_draw = (randn(C) * 0.1).to(torch.bfloat16)
    conv_bias = bias_draw if with_bias else None
    conv_shape = (num_slots, C, W - 1) if conv_dim_first else (num_slots, W - 1, C)
    if pool_device is None:
        conv_storage = randn(*conv_shape).to(torch.bfloat16)
        state = randn(num_slots, H, HEAD_DIM, HEAD_DIM) * 0.05
    else:
        dgen = torch.Generator(device=pool_device).manual_seed(seed)
        conv_storage = torch.randn(conv_shape, generator=dgen, device=pool_device).to(torch.bfloat16)
        state = torch.randn((num_slots, H, HEAD_DIM, HEAD_DIM), generator=dgen,
                            device=pool_device).mul_(0.05)
    f_b = (randn(D, FA_RANK) * 0.09).to(torch.bfloat16)
    lo, hi = a_log_range
    A_log = rand(H) * (hi - lo) + lo
    dt_bias = rand(D) * 2.0 - 1.0
    norm_weight = rand(HEAD_DIM) + 0.5

    if fixed_slot is not None:
        if S != 1:
            raise ValueError("a fixed slot serves one row")
        slots = torch.tensor([fixed_slot], dtype=torch.int32)
    elif block_table_cols is not None:
        if R * block_table_cols > num_slots or block_table_cols < L:
            raise ValueError("block table does not fit the pool")
        table = torch.randperm(num_slots, generator=gen)[: R * block_table_cols]
        table = table.to(torch.int32).view(R, block_table_cols)
        slots = table[:, :L]
    else:
        if S > num_slots:
            raise ValueError("more rows than pool slots")
        perm = torch.randperm(num_slots, generator=gen)[:S].to(torch.int32)
        slots = perm.view(R, L) if verify else perm
    accepted = torch.randint(1, L + 1, (R,), generator=gen, dtype=torch.int32) if verify else None
    if beta_std != 1.0:
        beta = (randn(S, H) * beta_std).to(torch.bfloat16)
        projected[:, 4 * D + FA_RANK: 4 * D + FA_RANK + H] = beta
    if coarse_gate:
        f_b = (torch.randint(-31, 32, (D, FA_RANK), generator=gen).float() * 2.0 ** -8).to(torch.bfloat16)
        f_a = (torch.randint(-31, 32, (S, FA_RANK), generator=gen).float() * 2.0 ** -4).to(torch.bfloat16)
        projected[:, 4 * D: 4 * D + FA_RANK] = f_a

    return Case(name=name, seed=seed, R=R, L=L, H=H, W=W, num_slots=num_slots, pitch=pitch,
                verify=verify, projected=projected, conv_weight=conv_weight,
                conv_bias=conv_bias, conv_storage=conv_storage, conv_dim_first=conv_dim_first,
                state=state, f_b=f_b, A_log=A_log, dt_bias=dt_bias, norm_weight=norm_weight,
                slots=slots, accepted=accepted)


def make_config(index: int) -> Case:
    """One of the five workload configurations, with its own seed."""
    cfg = dict(CONFIGS[index])
    name, R, L, H, num_slots, seed = (cfg.pop(k) for k in ("name", "R", "L", "H", "num_slots",
                                                           "seed"))
    return make_case(R, L, H, num_slots, seed, name=name, **cfg)


# Projections around the core: the hidden size of the model the pages serve
# (the back page's o_proj produces 448 x 16 = 7168 rows) and one
# tensor-parallel rank's 12 heads.
HIDDEN = 7168


def make_linear(M: int, N: int, K: int, seed: int, x_pitch: Optional[int] = None):
    """x bf16 [M, x_pitch] ~ N(0, 1) and an nn.Linear-scaled weight w bf16 [N, K]
    ~ N(0, 1/K), drawn in that order from one generator seeded with `seed`."""
    x_pitch = K if x_pitch is None else x_pitch
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(M, x_pitch, generator=gen).to(torch.bfloat16)
    w = (torch.randn(N, K, generator=gen) * K ** -0.5).to(torch.bfloat16)
    return x, w
