"""HIP path vs the CPU oracle, element by element, through the C ABI.

Full-size workload configurations (tiny decode, decode R=64, verify 16x4,
verify 64x8 with a block-table slice, decode R=256 with the transposed conv
layout and decay extremes), ragged small cases for every verify length, and
several chained steps on the same pools."""
import numpy as np
import pytest
import torch

from kda_inputs import CONFIGS, make_case, make_config
from oracle_cases import run_oracle
from parity import assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpu_cases import run_gpu  # noqa: F401  (loads the library early, loudly)


@pytest.mark.parametrize("index", sorted(CONFIGS))
def test_config_parity(index):
    from gpu_cases import run_gpu
    case = make_config(index)
    print(f"[case] config {index} {case.name} R={case.R} L={case.L} H={case.H} "
          f"slots={case.num_slots}", flush=True)
    before = case.state.numpy().copy()
    ref = run_oracle(case)
    got = run_gpu(case)
    assert_parity(case, ref, got, before, label=case.name)


@pytest.mark.parametrize("L", range(1, 9))
def test_ragged_verify_every_length(L):
    from gpu_cases import run_gpu
    case = make_case(R=5, L=L, H=3, num_slots=48, seed=100 + L, verify=True)
    print(f"[case] ragged verify R=5 L={L} H=3", flush=True)
    before = case.state.numpy().copy()
    assert_parity(case, run_oracle(case), run_gpu(case), before, label=f"ragged L={L}")


@pytest.mark.parametrize("R,H", [(1, 1), (7, 2), (33, 5)])
def test_ragged_decode(R, H):
    from gpu_cases import run_gpu
    case = make_case(R=R, L=1, H=H, num_slots=2 * R + 3, seed=200 + R, verify=False,
                     conv_dim_first=(R % 2 == 1))
    print(f"[case] ragged decode R={R} H={H}", flush=True)
    before = case.state.numpy().copy()
    assert_parity(case, run_oracle(case), run_gpu(case), before, label=f"decode R={R} H={H}")


def test_chained_verify_steps():
    """Four verify steps in a row on the same pools, with new accepted counts each step."""
    from gpu_cases import GpuCase
    case = make_case(R=6, L=4, H=2, num_slots=64, seed=300, verify=True)
    print("[case] chained verify steps R=6 L=4 H=2", flush=True)
    g = GpuCase(case)
    conv = case.conv_storage.clone()
    state = case.state.clone()
    gen = torch.Generator().manual_seed(301)
    try:
        for step in range(4):
            proj = torch.randn(case.S, case.pitch, generator=gen).to(torch.bfloat16)
            acc = torch.randint(1, case.L + 1, (case.R,), generator=gen, dtype=torch.int32)
            stepcase = make_case(R=6, L=4, H=2, num_slots=64, seed=300, verify=True)
            stepcase.accepted = acc
            before = state.numpy().copy()
            ref = run_oracle(stepcase, projected=proj, conv_storage=conv, state=state)
            g.run(projected=proj, accepted=acc)
            got = g.host()
            assert_parity(stepcase, ref, got, before, label=f"step {step}")
            # both sides carry the oracle's pools forward
            state = torch.from_numpy(ref["state"])
            conv = torch.from_numpy(ref["conv"]).view(torch.int16).view(torch.bfloat16)
            g.state.copy_(state)
            g.conv_storage.copy_(conv)
    finally:
        g.close()


@pytest.mark.parametrize("variant", ["saturated", "strong_decay_large_inputs"])
def test_extreme_parameters(variant):
    """Saturating and extreme values: a gate sigmoid driven far into saturation
    (A_log up to 4, so exp(A_log) ~ 55), a lower bound of -30 (decays down to
    e^-30 per token over 8 tokens), beta_raw ~ N(0, 4^2) (beta near 0 or 1), and
    inputs 4x larger (exact in bf16). The fast exp / sigmoid / rsqrt paths must
    stay finite and match the oracle within the usual bars."""
    import dataclasses
    from gpu_cases import run_gpu
    if variant == "saturated":
        case = make_case(R=12, L=4, H=4, num_slots=64, seed=950, verify=True, beta_std=4.0,
                         a_log_range=(2.0, 4.0))
    else:
        base = make_case(R=12, L=8, H=4, num_slots=128, seed=951, verify=True, beta_std=4.0,
                         a_log_range=(-3.0, 4.0))
        case = dataclasses.replace(base, projected=(base.projected.float() * 4.0).to(torch.bfloat16),
                                   gate_lower_bound=-30.0)
    before = case.state.numpy().copy()
    ref = run_oracle(case)
    got = run_gpu(case)
    assert np.all(np.isfinite(got["state"])), "non-finite state"
    assert_parity(case, ref, got, before, label=f"extreme: {variant}")
