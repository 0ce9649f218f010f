"""Parity bars of the bf16 hand-off rounding mode (test infrastructure).

Both the kernel and the oracle round conv out, g1 and o to bf16 where they are
produced, but each computes the value it rounds in its own precision (fp32 on
the GPU, double in the oracle). A value lying within the kernel's error of a
bf16 rounding boundary may therefore round differently on the two sides, and
the flip then propagates. The oracle reports, per (request, head), how many
rounded values lie within a margin of a boundary (its near-tie counters); the
margins below bound the kernel's fp32 error:

  conv out  y = SiLU(pre), pre from four fused multiply-adds of exact bf16
            products: |d pre| <= 4 * 2^-24 * sum|terms| = 2^-22 sum|terms|,
            reaching y through SiLU's slope; SiLU in fp32 rounds the exponent's
            argument (|pre| 2^-24 relative in e^-pre) and adds ~2^-22.4 relative
            for exp2, 1 + e, the reciprocal and the products. The oracle's margin
            mu (|SiLU'| sum|terms| + (1 + |pre|) |y|) covers both for any
            mu >= 2^-22; mu = 2^-20 leaves a factor of 4.
  g1        f_b f_a on MFMA: with the coarse gate operands of kda_inputs every
            term is a multiple of 2^-12 and the sum stays below 2^12, so any fp32
            summation is exact; the oracle certifies that per channel and uses
            a zero margin. For other operands, 2^-16 sum|terms| (twice the
            worst case of a sequential fp32 sum of 128 terms).
  o, y      reported (2^-18, 2^-19) but not used to pick units: o near ties are
            common, and their effect is bounded on core_out instead.

Bars:
  - conv pool bit-exact (windows are copies of bf16 inputs), untouched slots and
    skipped rows as in the fused mode;
  - "clean" units, with no conv-out or g1 near tie in any of their tokens: both
    sides round identical values, so only fp32-versus-double arithmetic
    separates them (measured <= 6e-7 of the tile maximum in the fused mode):
    every written state tile within max|d| / max|ref| <= 2e-5. The fused and
    hand-off modes differ by 1.6e-3 or more on such tiles.
  - other units: <= 1e-2 (one flipped bf16 input moves a tile by a few 1e-3);
  - core_out: |d| <= 2e-2 + 2^-7 |ref| everywhere, and at most 2 % of the bf16
    values differ (a flipped o moves its output by about one bf16 step; the
    fused mode differs from the hand-off mode in about half of them).
"""
from __future__ import annotations

import numpy as np

from gpu_cases import OUT_SENTINEL, bf16_bits_to_f32
from parity import request_slots

MARGINS = (2.0 ** -20, 2.0 ** -16, 2.0 ** -18, 2.0 ** -19)
CLEAN_RTOL = 2e-5
FLIP_RTOL = 1e-2
OUT_ATOL = 2e-2
OUT_RTOL = 2.0 ** -7
OUT_MISMATCH_FRAC = 0.02


def clean_units(ties: np.ndarray) -> np.ndarray:
    """[R, H] bool: no conv-out or g1 near tie in the unit's tokens."""
    return (ties[:, :, 0] == 0) & (ties[:, :, 1] == 0)


def assert_handoff_parity(case, ref, got, ties, state_before, *, min_clean=0, label=""):
    reqs = request_slots(case)
    n_bad = sum(1 for ok, _, _ in reqs if not ok)
    assert got["errors"] == n_bad == ref["skipped"], (label, got["errors"], n_bad, ref["skipped"])
    if not np.array_equal(got["conv"], ref["conv"]):
        raise AssertionError(f"{label}: conv pool differs at {np.count_nonzero(got['conv'] != ref['conv'])}")

    clean = clean_units(ties)
    n_clean = int(sum(clean[r].sum() for r, (ok, _, _) in enumerate(reqs) if ok))
    assert n_clean >= min_clean, (label, "too few clean units", n_clean, min_clean)
    worst = {True: 0.0, False: 0.0}
    written = set()
    for r, (ok, _, dst) in enumerate(reqs):
        if not ok:
            continue
        for slot in dst:
            written.add(slot)
            for h in range(case.H):
                rr = ref["state"][slot, h].astype(np.float64)
                g = got["state"][slot, h].astype(np.float64)
                assert np.all(np.isfinite(g)), (label, slot, h)
                rel = np.abs(g - rr).max() / np.abs(rr).max()
                c = bool(clean[r, h])
                worst[c] = max(worst[c], rel)
                assert rel <= (CLEAN_RTOL if c else FLIP_RTOL), (label, r, h, "clean" if c else "tie", rel)
    untouched = np.array([s for s in range(case.num_slots) if s not in written], dtype=np.int64)
    if untouched.size:
        assert np.array_equal(got["state"][untouched], state_before[untouched]), (label, "untouched")

    L = case.L
    rows = np.array([r * L + t for r, (ok, _, _) in enumerate(reqs) if ok for t in range(L)], np.int64)
    bad = np.array([r * L + t for r, (ok, _, _) in enumerate(reqs) if not ok for t in range(L)], np.int64)
    if bad.size:
        assert np.all(got["out"][bad] == OUT_SENTINEL), (label, "skipped rows written")
    g = bf16_bits_to_f32(got["out"][rows]).astype(np.float64)
    rr = bf16_bits_to_f32(ref["out"][rows]).astype(np.float64)
    assert np.all(np.isfinite(g)), (label, "non-finite core_out")
    excess = np.abs(g - rr) - (OUT_ATOL + OUT_RTOL * np.abs(rr))
    assert excess.max() <= 0, (label, "core_out", float(np.abs(g - rr).max()))
    mism = float(np.mean(got["out"][rows] != ref["out"][rows]))
    assert mism <= OUT_MISMATCH_FRAC, (label, "core_out mismatch fraction", mism)
    print(f"[handoff] {label}: clean units {n_clean}/{clean.size}, state rel clean {worst[True]:.2e} "
          f"other {worst[False]:.2e}, core_out max abs {float(np.abs(g - rr).max()):.2e}, "
          f"mismatch {mism:.4f}", flush=True)
    return dict(n_clean=n_clean, worst_clean=worst[True], worst_other=worst[False], mismatch=mism)
