"""Seeded random combinations of the options the explicit parity cases set one or
two at a time: request count, verify length (1..8, decode or verify), heads,
pool size, slots from a block-table slice or a permutation, conv layout, bias,
padded pitch, per-head norm weights and decay / beta extremes for the core; row
count, column count, K, pitches and workspace for the projection GEMM. Every
case is checked against the oracle in full. The draws come from fixed seeds, so
a failing case is reproducible from its printed parameters."""
import numpy as np
import pytest
import torch

from kda_inputs import default_pitch, make_case, make_linear
from oracle_cases import run_oracle
from parity import assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpu_cases import run_gpu  # noqa: F401  (loads the library early, loudly)


def _core_params(i):
    rng = np.random.default_rng(7000 + i)
    L = 1 if i % 4 == 0 else int(rng.integers(1, 9))
    verify = i % 4 != 0
    R = int(rng.integers(1, 10))
    H = int(rng.integers(1, 5))
    use_table = verify and bool(rng.integers(0, 2))
    cols = L + int(rng.integers(0, 4)) if use_table else None
    rows = R * (cols if use_table else L)
    return dict(R=R, L=L, H=H, verify=verify, block_table_cols=cols,
                num_slots=rows + int(rng.integers(0, 9)),
                conv_dim_first=bool(rng.integers(0, 2)), with_bias=bool(rng.integers(0, 2)),
                extra_pitch=int(rng.choice([0, 1, 2, 63])), per_head_norm=bool(rng.integers(0, 2)),
                beta_std=float(rng.choice([1.0, 2.0, 4.0])),
                a_log_range=[(-1.0, 1.0), (-3.0, 2.0)][int(rng.integers(0, 2))])


@pytest.mark.parametrize("i", range(48))
def test_core_random_combination(i):
    from gpu_cases import run_gpu
    prm = _core_params(i)
    print(f"[case] core sweep {i}: {prm}", flush=True)
    case = make_case(prm["R"], prm["L"], prm["H"], prm["num_slots"], seed=7100 + i,
                     verify=prm["verify"], pitch=default_pitch(prm["H"]) + prm["extra_pitch"],
                     conv_dim_first=prm["conv_dim_first"], with_bias=prm["with_bias"],
                     beta_std=prm["beta_std"], a_log_range=prm["a_log_range"],
                     block_table_cols=prm["block_table_cols"])
    before = case.state.numpy().copy()
    if prm["per_head_norm"]:
        nw = torch.rand(case.H, 128, generator=torch.Generator().manual_seed(7200 + i)) + 0.5
        ref = run_oracle(case, norm_weight=nw.numpy().reshape(-1), norm_head_stride=128)
        got = run_gpu(case, norm_weight=nw)
    else:
        ref = run_oracle(case)
        got = run_gpu(case)
    assert_parity(case, ref, got, before, label=f"core sweep {i}")


def _linear_params(i):
    rng = np.random.default_rng(8000 + i)
    if i % 3 == 2:   # shapes that take the K split with a workspace
        M = int(rng.integers(33, 257))
        K = 256 * int(rng.integers(16, 20))
    else:            # up to 64 rows, or any row count
        M = int(rng.integers(1, 65 if i % 3 == 0 else 300))
        K = 8 * int(rng.integers(1, 160))
    N = int(rng.integers(1, 300))
    return dict(M=M, N=N, K=K, x_extra=8 * int(rng.integers(0, 3)),
                y_extra=int(rng.integers(0, 5)), workspace=bool(rng.integers(0, 2)) or i % 3 == 2)


@pytest.mark.parametrize("i", range(48))
def test_linear_random_shape(i):
    import kimi_delta_attention_conv_amd as kda
    import oracle
    from oracle_cases import bf16_np
    prm = _linear_params(i)
    M, N, K = prm["M"], prm["N"], prm["K"]
    print(f"[case] linear sweep {i}: {prm}", flush=True)
    x, w = make_linear(M, N, K, seed=8100 + i, x_pitch=K + prm["x_extra"])
    y_pitch = N + prm["y_extra"]
    sent = 0x7FC1
    xd, wd = x.cuda(), w.cuda()
    y = torch.full((M, y_pitch), sent, dtype=torch.int16).view(torch.bfloat16).cuda()
    nbytes = kda.kda_linear_workspace_bytes(M, N, K) if prm["workspace"] else 0
    work = torch.full((max(nbytes, 16) // 4,), float("nan"), device="cuda")
    kda.kda_linear(xd.data_ptr(), xd.stride(0), wd.data_ptr(), y.data_ptr(), y_pitch, M, N, K,
                   work.data_ptr() if nbytes else 0, nbytes,
                   stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = bf16_np(y.cpu())
    assert np.all(got[:, N:] == sent), "columns beyond N were written"
    _, ref = oracle.default().linear(bf16_np(x), bf16_np(w))
    xf = oracle.bf16_bits_to_f64(bf16_np(x)[:, :K])
    wf = oracle.bf16_bits_to_f64(bf16_np(w))
    lim = 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -23 * (np.abs(xf) @ np.abs(wf).T)
    g = (got[:, :N].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.isfinite(g))
    worst = float(np.max(np.abs(g - ref) / np.maximum(lim, 1e-300)))
    print(f"[linear] sweep {i}: split={nbytes > 0} max err/limit {worst:.3f}", flush=True)
    assert worst <= 1.0
