"""Decode grids of more (request, head) units than the device has compute units
(several rounds of workgroups a compute unit), with every option the core
takes: checked against the oracle, and bit for bit against the same requests
issued as calls of at most 21 requests (252 units; a whole MI355X has 256
compute units), so that a result never depends on how a batch is split into
calls or how many rounds of workgroups it takes."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_cases import GpuCase, OUT_SENTINEL, run_gpu
from kda_inputs import make_case
from oracle_cases import run_oracle
from parity import assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    props = torch.cuda.get_device_properties(0)
    if props.multi_processor_count != 256:
        pytest.skip("the 21-request split assumes 256 compute units")


def _chunked(case, chunk=21, **kw):
    """The same decode call issued as calls of at most `chunk` requests."""
    g = GpuCase(case, **kw)
    try:
        slots = case.slots.cuda()
        for r0 in range(0, case.R, chunk):
            r1 = min(case.R, r0 + chunk)
            g.core.decode(g.projected[r0:r1], g.out[r0:r1], slots[r0:r1])
        torch.cuda.synchronize()
        return g.host()
    finally:
        g.close()


CASES = {
    "r40_dim_first": dict(R=40, seed=1100),
    "r24_transposed_no_bias_odd_pitch": dict(R=24, seed=1101, conv_dim_first=False, with_bias=False,
                                             pitch=4 * 1536 + 128 + 12 + 1),
    "r33_extremes": dict(R=33, seed=1102, beta_std=2.0, a_log_range=(-3.0, 2.0)),
    "r25_h11_ragged": dict(R=25, H=11, seed=1103),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_large_decode_grid_against_oracle_and_split_calls(name):
    kw = dict(CASES[name])
    H = kw.pop("H", 12)
    R = kw.pop("R")
    case = make_case(R, 1, H, 2 * R + 8, verify=False, name=name, **kw)
    assert case.R * case.H > 256
    print(f"[case] large decode grid {name}: {case.R * case.H} units", flush=True)
    got = run_gpu(case)
    ref = run_oracle(case)
    assert_parity(case, ref, got, case.state.numpy(), label=name)
    split = _chunked(case)
    for k in ("out", "conv", "state"):
        assert np.array_equal(got[k], split[k]), (name, k, int(np.count_nonzero(got[k] != split[k])))


def test_large_decode_grid_per_head_norm_weights_and_handoff():
    from handoff_bars import MARGINS, assert_handoff_parity
    case = make_case(30, 1, 12, 64, seed=1104, verify=False, coarse_gate=True,
                     name="large_grid_handoff")
    ties = np.zeros((case.R, case.H, 4), np.int32)
    ref = run_oracle(case, handoff_bf16=True, ties=ties, tie_margins=MARGINS)
    got = run_gpu(case, rounding="bf16_handoff")
    assert_handoff_parity(case, ref, got, ties, case.state.numpy(), min_clean=40, label=case.name)
    split = _chunked(case, rounding="bf16_handoff")
    for k in ("out", "conv", "state"):
        assert np.array_equal(got[k], split[k]), k
    nw = torch.rand(case.H * 128, generator=torch.Generator().manual_seed(5)) + 0.5
    got = run_gpu(case, norm_weight=nw)
    ref = run_oracle(case, norm_weight=nw.numpy(), norm_head_stride=128)
    assert_parity(case, ref, got, case.state.numpy(), label="large_grid_per_head_norm")


def test_large_decode_grid_skips_invalid_and_colliding_requests():
    """Skipped requests across rounds of workgroups: out-of-range slots, and
    (with check_distinct) two requests naming one slot; the others are exact."""
    base = make_case(36, 1, 12, 96, seed=1105, verify=False)
    s = base.slots.clone()
    s[3] = base.num_slots + 1       # out of range
    s[17] = -4                      # negative
    s[30] = s[8]                    # duplicate destination (requests 8 and 30)
    case = dataclasses.replace(base, slots=s)
    ref = run_oracle(case, check_distinct=True)
    assert ref["skipped"] == 4
    got = run_gpu(case, check_distinct=True)
    assert_parity(case, ref, got, case.state.numpy(), skip={8, 30}, label="large_grid_skips")
    for r in (3, 8, 17, 30):
        assert np.all(got["out"][r] == OUT_SENTINEL), r
