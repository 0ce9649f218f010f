"""Parity at the largest shapes: a decode grid of 196,608 workgroups (16,384
requests x 12 heads, a 12.9 GB state pool) checked on sampled requests, and the
most heads the ABI accepts (4096, D = 524,288 channels) checked in full.

The pools of these cases are drawn on the device (kda_inputs, `pool_device`).
For the sampled check, the oracle runs a sub-problem made of the sampled
requests only: their projected rows, the pre-call contents of the slots they
read and write (gathered into a small pool of their own), and the same weights.
Requests are independent of one another, so the sub-problem's results are the
full call's results for those requests."""
import dataclasses

import numpy as np
import pytest
import torch

import kimi_delta_attention_conv_amd as kda
from gpu_cases import OUT_SENTINEL
from kda_inputs import make_case
from oracle_cases import bf16_np, run_oracle
from parity import assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _core(case):
    conv = case.conv_storage if case.conv_dim_first else case.conv_storage.transpose(-1, -2)
    return kda.KdaCore(conv_weight=case.conv_weight.cuda(),
                       conv_bias=None if case.conv_bias is None else case.conv_bias.cuda(),
                       f_b=case.f_b.cuda(), A_log=case.A_log.cuda(), dt_bias=case.dt_bias.cuda(),
                       norm_weight=case.norm_weight.cuda(), gate_lower_bound=case.gate_lower_bound,
                       norm_eps=case.norm_eps, l2_eps=case.l2_eps, conv=conv, state=case.state)


def _run(case, core):
    out = torch.full((case.S, case.D), OUT_SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    proj = case.projected.cuda()
    slots = case.slots.contiguous().cuda()
    if case.verify:
        core.verify(proj, out, slots, case.accepted.cuda())
    else:
        core.decode(proj, out, slots)
    torch.cuda.synchronize()
    return out


def test_large_decode_grid_sampled():
    R, H = 16384, 12
    case = make_case(R, 1, H, R, seed=900, pool_device="cuda")
    rng = np.random.default_rng(901)
    sample = np.sort(rng.choice(R, 64, replace=False))
    sample[0], sample[-1] = 0, R - 1            # the first and last workgroups' units too
    used = case.slots[torch.as_tensor(sample)].long()
    conv_before = case.conv_storage[used.cuda()].cpu()
    state_before = case.state[used.cuda()].cpu()

    core = _core(case)
    try:
        out = _run(case, core)
        errors = core.device_errors()
    finally:
        core.close()
    assert errors == 0
    assert not torch.any(out.view(torch.int16) == OUT_SENTINEL), "a core_out row was not written"
    assert bool(torch.isfinite(out.float()).all()), "non-finite core_out"

    n = len(sample)
    sub = dataclasses.replace(
        case, name="large_decode_sample", R=n, num_slots=n,
        projected=case.projected[torch.as_tensor(sample)].clone(),
        conv_storage=conv_before, state=state_before,
        slots=torch.arange(n, dtype=torch.int32))
    ref = run_oracle(sub)
    got = dict(out=out[torch.as_tensor(sample).cuda()].cpu().view(torch.int16).numpy().view(np.uint16).copy(),
               conv=bf16_np(case.conv_storage[used.cuda()].cpu()),
               state=case.state[used.cuda()].cpu().numpy().copy(),
               errors=0)
    assert_parity(sub, ref, got, state_before.numpy(), label=f"decode R={R} H={H}, {n} sampled")


def test_max_heads_verify_full():
    H = 4096
    case = make_case(2, 2, H, 4, seed=910, verify=True, pool_device="cuda")
    host = dataclasses.replace(case, conv_storage=case.conv_storage.cpu(), state=case.state.cpu())
    ref = run_oracle(host)

    core = _core(case)
    try:
        out = _run(case, core)
        errors = core.device_errors()
    finally:
        core.close()
    got = dict(out=out.cpu().view(torch.int16).numpy().view(np.uint16).copy(),
               conv=bf16_np(case.conv_storage.cpu()),
               state=case.state.cpu().numpy(),
               errors=errors)
    assert_parity(host, ref, got, host.state.numpy(), label=f"verify R=2 L=2 H={H}")
