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


@pytest.mark.parametrize("R", [16, 32])
def test_handoff_verify_equals_chained_decodes_bit_exact(R):
    """Hand-off mode: a verify call over 8 tokens (12 heads; 16 requests take the
    16-wave unit form, 32 the 8-wave one) equals 8 decode calls chained on one slot
    a request, bit for bit: every core_out row, every per-token state and conv
    window. Each token's arithmetic does not depend on L, so the L = 1 bars of the
    hand-off mode carry over to every token of a long verify."""
    import dataclasses

    from gpu_cases import GpuCase
    from parity import request_slots

    L = 8
    case = make_case(R, L, 12, R * L, seed=730 + R, verify=True, coarse_gate=True,
                     name=f"handoff_chain_r{R}")
    print(f"[case] {case.name}: verify", flush=True)
    g = GpuCase(case, rounding="bf16_handoff").run()
    full = g.host()
    g.close()
    assert full["errors"] == 0
    reqs = request_slots(case)
    tmp = [dst[0] for _, _, dst in reqs]
    state = case.state.clone()
    conv = case.conv_storage.clone()
    for r, (_, src, _) in enumerate(reqs):
        state[tmp[r]] = case.state[src]
        conv[tmp[r]] = case.conv_storage[src]
    dec = dataclasses.replace(case, L=1, verify=False, accepted=None, state=state,
                              conv_storage=conv, slots=torch.tensor(tmp, dtype=torch.int32),
                              projected=case.projected[0::L].contiguous())
    gd = GpuCase(dec, rounding="bf16_handoff")
    try:
        for t in range(L):
            print(f"[case] {case.name}: chained decode token {t}", flush=True)
            gd.run(projected=case.projected[t::L].contiguous())
            h = gd.host()
            assert h["errors"] == 0
            for r in range(R):
                d = reqs[r][2][t]
                assert np.array_equal(h["out"][r], full["out"][r * L + t]), (r, t, "core_out")
                assert np.array_equal(h["state"][tmp[r]], full["state"][d]), (r, t, "state")
                assert np.array_equal(h["conv"][tmp[r]], full["conv"][d]), (r, t, "conv")
    finally:
        gd.close()


def test_handoff_l8_each_token_against_oracle_from_gpu_state():
    """Hand-off mode at 16 x 8, 12 heads, token by token: for token t of every
    request the oracle runs one decode step from the GPU's own state and conv window
    after token t - 1 (the carried ones for t = 0), so both sides start every step
    from identical inputs, and the GPU's state written for token t and its core_out
    row must meet the one-token bars: conv windows bit-exact, state tiles of units
    with no conv-out or g1 near tie in that step within 2e-5 of the tile maximum
    (1e-2 otherwise), core_out within 2e-2 + 2^-7 |ref| with at most 2 % of the
    values differing."""
    import dataclasses

    from gpu_cases import bf16_bits_to_f32
    from handoff_bars import (CLEAN_RTOL, FLIP_RTOL, OUT_ATOL, OUT_MISMATCH_FRAC, OUT_RTOL,
                              clean_units)
    from oracle_cases import bf16_np
    from parity import request_slots

    R, L, H = 16, 8, 12
    case = make_case(R, L, H, R * L, seed=740, verify=True, coarse_gate=True,
                     name="handoff_l8_stepwise")
    print(f"[case] {case.name}", flush=True)
    got = run_gpu(case, rounding="bf16_handoff")
    assert got["errors"] == 0
    reqs = request_slots(case)
    state0 = case.state.numpy()
    conv0 = bf16_np(case.conv_storage)
    n_clean = 0
    worst = {True: 0.0, False: 0.0}
    mism = []
    for t in range(L):
        prev = [src if t == 0 else dst[t - 1] for _, src, dst in reqs]
        st = np.stack([state0[s] if t == 0 else got["state"][s] for s in prev])
        cv = np.stack([conv0[s] if t == 0 else got["conv"][s] for s in prev])
        step = dataclasses.replace(
            case, L=1, verify=False, accepted=None, num_slots=R,
            slots=torch.arange(R, dtype=torch.int32), projected=case.projected[t::L].contiguous(),
            state=torch.from_numpy(st.copy()),
            conv_storage=torch.from_numpy(cv.view(np.int16).copy()).view(torch.bfloat16))
        ties = np.zeros((R, H, 4), np.int32)
        ref = run_oracle(step, handoff_bf16=True, ties=ties, tie_margins=MARGINS)
        assert ref["skipped"] == 0
        clean = clean_units(ties)
        for r, (_, _, dst) in enumerate(reqs):
            assert np.array_equal(got["conv"][dst[t]], ref["conv"][r]), (r, t, "conv window")
            for h in range(H):
                g = got["state"][dst[t], h].astype(np.float64)
                rr = ref["state"][r, h].astype(np.float64)
                rel = np.abs(g - rr).max() / np.abs(rr).max()
                c = bool(clean[r, h])
                n_clean += c
                worst[c] = max(worst[c], rel)
                assert rel <= (CLEAN_RTOL if c else FLIP_RTOL), (r, t, h, c, rel)
        rows = np.arange(R) * L + t
        go = bf16_bits_to_f32(got["out"][rows]).astype(np.float64)
        ro = bf16_bits_to_f32(ref["out"]).astype(np.float64)
        assert np.all(np.isfinite(go))
        assert (np.abs(go - ro) - (OUT_ATOL + OUT_RTOL * np.abs(ro))).max() <= 0, t
        mism.append(float(np.mean(got["out"][rows] != ref["out"])))
        assert mism[-1] <= OUT_MISMATCH_FRAC, (t, mism[-1])
    print(f"[handoff] stepwise 16x8: clean unit-steps {n_clean}/{R * H * L}, state rel clean "
          f"{worst[True]:.2e} other {worst[False]:.2e}, core_out mismatch max {max(mism):.4f}",
          flush=True)
    assert n_clean >= 150, n_clean
