"""The bf16 hand-off rounding mode on the GPU against the oracle's hand-off mode
(bars and margins in handoff_bars.py)."""
import numpy as np
import pytest
import torch

from gpu_cases import run_gpu
from handoff_bars import MARGINS, assert_handoff_parity
from kda_inputs import make_case
from oracle_cases import run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(case, min_clean):
    ties = np.zeros((case.R, case.H, 4), np.int32)
    ref = run_oracle(case, handoff_bf16=True, ties=ties, tie_margins=MARGINS)
    got = run_gpu(case, rounding="bf16_handoff")
    return assert_handoff_parity(case, ref, got, ties, case.state.numpy(), min_clean=min_clean,
                                 label=case.name)


@pytest.mark.parametrize("R,L,min_clean", [(64, 1, 100), (64, 2, 30), (16, 8, 0)])
def test_handoff_parity_coarse_gate(R, L, min_clean):
    case = make_case(R, L, 12, 1024, seed=700 + L, verify=L > 1, coarse_gate=True,
                     name=f"handoff_coarse_r{R}_l{L}")
    _check(case, min_clean)


def test_handoff_parity_general_inputs():
    """Ordinary gate operands: g1 values near a rounding boundary are common, so
    few units are clean; the flip-tolerant bars still hold everywhere."""
    case = make_case(64, 1, 12, 128, seed=720, name="handoff_general_r64")
    _check(case, 0)


def test_handoff_transposed_pool_and_verify_ragged():
    case = make_case(5, 3, 3, 32, seed=721, verify=True, conv_dim_first=False, coarse_gate=True,
                     name="handoff_ragged_transposed")
    _check(case, 0)


def test_fused_mode_unchanged_by_handoff_build():
    """The fused mode still meets its own bars (a guard on the mode switch)."""
    from parity import assert_parity
    case = make_case(16, 4, 12, 128, seed=722, verify=True, name="fused_after_handoff")
    ref = run_oracle(case)
    got = run_gpu(case)
    assert_parity(case, ref, got, case.state.numpy(), label=case.name)
