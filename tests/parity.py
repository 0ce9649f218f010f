"""Element-by-element comparison of the HIP path with the oracle.

Bars:
  - conv cache pool: bit-exact everywhere (written windows are copies of bf16
    inputs; untouched slots must not change);
  - state pool: every (written slot, head) tile within max|d| / max|ref| <= 1e-3;
    every other slot bit-exact (untouched);
  - core_out: max |gpu - oracle| <= 2e-2 over all outputs of valid requests,
    compared as floats from the bf16 values; rows of skipped requests untouched;
  - the device error counter equals the oracle's skipped-request count.
"""
from __future__ import annotations

import numpy as np

from gpu_cases import OUT_SENTINEL, bf16_bits_to_f32

OUT_ATOL = 2e-2
STATE_RTOL = 1e-3


def request_slots(case, slots=None, accepted="case", skip=()):
    """Per request: (valid, src, [dst per token]) under the oracle's rules; the
    requests in `skip` (e.g. colliding destinations under check_distinct) count
    as invalid."""
    s = (case.slots if slots is None else slots).numpy()
    acc = case.accepted if isinstance(accepted, str) else accepted
    acc = None if acc is None else np.asarray(acc)
    if s.ndim == 1:
        s = s[:, None]
    res = []
    for r in range(case.R):
        dst = [int(x) for x in s[r, :case.L]]
        ok = all(0 <= d < case.num_slots for d in dst)
        if acc is None:
            src = dst[0]
        else:
            a = int(acc[r])
            ok = ok and 1 <= a <= case.L
            src = dst[a - 1] if ok else -1
        res.append((ok and r not in skip, src, dst))
    return res


def assert_parity(case, ref, got, state_before, *, slots=None, accepted="case", label="",
                  skip=()):
    reqs = request_slots(case, slots, accepted, skip)
    n_bad = sum(1 for ok, _, _ in reqs if not ok)
    assert got["errors"] == n_bad == ref["skipped"], (label, got["errors"], n_bad, ref["skipped"])

    # conv windows: bit-exact over the whole pool
    if not np.array_equal(got["conv"], ref["conv"]):
        diff = np.argwhere(got["conv"] != ref["conv"])
        raise AssertionError(f"{label}: conv pool differs at {len(diff)} elements, first {diff[:4]}")

    # states
    written = sorted({d for ok, _, dst in reqs if ok for d in dst})
    wset = set(written)
    H = case.H
    worst = 0.0
    for slot in written:
        for h in range(H):
            r = ref["state"][slot, h].astype(np.float64)
            g = got["state"][slot, h].astype(np.float64)
            assert np.all(np.isfinite(g)), (label, slot, h, "non-finite state")
            scale = np.abs(r).max()
            rel = np.abs(g - r).max() / scale if scale > 0 else np.abs(g).max()
            worst = max(worst, rel)
            assert rel <= STATE_RTOL, (label, "state tile", slot, h, rel)
    untouched = np.array([s for s in range(case.num_slots) if s not in wset], dtype=np.int64)
    if untouched.size:
        assert np.array_equal(got["state"][untouched], state_before[untouched]), \
            (label, "an untouched state slot changed")

    # core_out
    S, L = case.S, case.L
    valid_rows = np.array([r * L + t for r, (ok, _, _) in enumerate(reqs) if ok for t in range(L)],
                          dtype=np.int64)
    bad_rows = np.array([r * L + t for r, (ok, _, _) in enumerate(reqs) if not ok
                         for t in range(L)], dtype=np.int64)
    if bad_rows.size:
        assert np.all(got["out"][bad_rows] == OUT_SENTINEL), (label, "skipped rows written")
    out_err = 0.0
    ulps = 0
    if valid_rows.size:
        g = bf16_bits_to_f32(got["out"][valid_rows]).astype(np.float64)
        r = bf16_bits_to_f32(ref["out"][valid_rows]).astype(np.float64)
        assert np.all(np.isfinite(g)), (label, "non-finite core_out")
        err = np.abs(g - r)
        out_err = float(err.max())
        ulps = int(np.count_nonzero(got["out"][valid_rows] != ref["out"][valid_rows]))
        if out_err > OUT_ATOL:
            i = np.unravel_index(int(np.argmax(err)), err.shape)
            raise AssertionError(f"{label}: core_out err {out_err} at row {valid_rows[i[0]]} col "
                                 f"{i[1]}: gpu {g[i]} oracle {r[i]}")
    print(f"[parity] {label}: state rel {worst:.3e}, core_out max abs {out_err:.3e}, "
          f"bf16 mismatches {ulps}/{valid_rows.size * case.D}, skipped {n_bad}", flush=True)
    return dict(state_rel=worst, out_err=out_err, out_mismatch=ulps)
