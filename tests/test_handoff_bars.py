"""The hand-off bars tell the two rounding modes apart (CPU, oracle only): the
oracle's fused-mode results, offered as if a kernel had ignored the hand-off
mode, fail them, while the hand-off results themselves pass."""
import numpy as np
import pytest

from handoff_bars import CLEAN_RTOL, MARGINS, assert_handoff_parity, clean_units
from kda_inputs import make_case
from oracle_cases import run_oracle


def _as_got(res):
    return dict(out=res["out"], conv=res["conv"], state=res["state"], errors=res["skipped"])


def test_fused_results_fail_the_handoff_bars():
    case = make_case(16, 1, 12, 64, seed=730, coarse_gate=True)
    ties = np.zeros((case.R, case.H, 4), np.int32)
    hand = run_oracle(case, handoff_bf16=True, ties=ties, tie_margins=MARGINS)
    fused = run_oracle(case)
    assert_handoff_parity(case, hand, _as_got(hand), ties, case.state.numpy(), label="self")
    with pytest.raises(AssertionError):
        assert_handoff_parity(case, hand, _as_got(fused), ties, case.state.numpy(), label="fused")
    # every clean tile is far outside the clean bar, not just the worst one
    clean = clean_units(ties)
    assert clean.sum() >= 20
    for r in range(case.R):
        slot = int(case.slots[r])
        for h in range(case.H):
            if clean[r, h]:
                a = hand["state"][slot, h].astype(np.float64)
                b = fused["state"][slot, h].astype(np.float64)
                assert np.abs(a - b).max() / np.abs(a).max() > 20 * CLEAN_RTOL, (r, h)
    assert np.mean(hand["out"] != fused["out"]) > 0.3
