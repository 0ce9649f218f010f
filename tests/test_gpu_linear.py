"""The projection kernel (kda_linear / kda_in_proj / kda_o_proj) vs the oracle.

Bar (derived from the arithmetic): bf16 x bf16 products are exact in fp32, so
the kernel's only error before the output rounding is fp32 accumulation, at
most K u sum_k |x_k w_k| with u = 2^-24 for round-to-nearest sums. The matrix
cores' internal rounding of their fp32 sums is not documented, so u = 2^-23
(the unit of directed rounding) is used; it also covers the accumulation
error's share of the output rounding. The bf16 output adds at most half an
ulp, which is up to 2^-8 |y| when |y| lies just above a power of two (so
measured ratios near 1 come from the output rounding). Each element must
satisfy |y_gpu - y| <= 2^-8 |y| + K 2^-23 sum|x w| with y the oracle's
double-precision value. Untouched output columns (pitch > N)
must stay bit-exact, and two runs must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from kda_inputs import HIDDEN, make_linear
from oracle_cases import bf16_np

pytestmark = pytest.mark.gpu

SENT = 0x7FC1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(x, w, y_pitch=None, M=None, fn="linear", heads=None, workspace=None):
    """workspace: None (no workspace: the unsplit kernel), "auto" (the size the
    library asks for), or a byte count."""
    import kimi_delta_attention_conv_amd as kda
    M = x.shape[0] if M is None else M
    N, K = w.shape
    y_pitch = N if y_pitch is None else y_pitch
    xd, wd = x.cuda(), w.cuda()
    y = torch.full((max(M, 1), y_pitch), SENT, dtype=torch.int16).view(torch.bfloat16).cuda()
    s = torch.cuda.current_stream().cuda_stream
    nbytes = kda.kda_linear_workspace_bytes(M, N, K) if workspace == "auto" else (workspace or 0)
    # the workspace starts as NaN patterns: no result may depend on its contents
    work = torch.full((max(nbytes, 16) // 2,), SENT, dtype=torch.int16, device="cuda")
    wp = work.data_ptr() if workspace is not None else 0
    if fn == "linear":
        kda.kda_linear(xd.data_ptr(), xd.stride(0), wd.data_ptr(), y.data_ptr(), y_pitch, M, N, K,
                       wp, nbytes, stream=s)
    elif fn == "in_proj":
        kda.kda_in_proj(xd.data_ptr(), xd.stride(0), wd.data_ptr(), y.data_ptr(), y_pitch, M, K,
                        heads, wp, nbytes, stream=s)
    else:
        kda.kda_o_proj(xd.data_ptr(), xd.stride(0), wd.data_ptr(), y.data_ptr(), y_pitch, M,
                       heads, N, wp, nbytes, stream=s)
    torch.cuda.synchronize()
    return bf16_np(y.cpu())


def _check(x, w, got, ms=None, ns=None, label=""):
    orc = oracle.default()
    xb, wb = bf16_np(x), bf16_np(w)
    N, K = wb.shape
    M = xb.shape[0]
    if ms is None:
        _, ref = orc.linear(xb, wb)
        ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        ms, ns = ms.ravel(), ns.ravel()
        ref = ref.ravel()
    else:
        ref = orc.linear_entries(xb, wb, ms, ns)
    xf = oracle.bf16_bits_to_f64(xb[:, :K])
    wf = oracle.bf16_bits_to_f64(wb)
    absdot = np.einsum("ik,ik->i", np.abs(xf[ms]), np.abs(wf[ns]))
    g = (got[ms, ns].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(g - ref)
    lim = 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -23 * absdot
    assert np.all(np.isfinite(g)), label
    worst = float(np.max(err / np.maximum(lim, 1e-300)))
    print(f"[linear] {label}: {ms.size} entries, max err/limit {worst:.3f}, "
          f"max abs err {err.max():.3e}", flush=True)
    assert worst <= 1.0, label


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (5, 37, 136), (16, 16, 128), (17, 33, 264),
                                   (33, 100, 1024), (64, 48, 520), (70, 129, 384),
                                   (100, 77, 520), (256, 65, 64), (257, 130, 192),
                                   (300, 200, 256), (20, 45, 128), (40, 65, 192), (17, 31, 64),
                                   (9, 40, 192), (7, 70, 1152), (24, 97, 896), (1, 300, 256),
                                   (64, 200, 1280)])
def test_ragged_shapes(M, N, K):
    x, w = make_linear(M, N, K, seed=M * 1000 + N + K, x_pitch=K + 8)
    got = _run(x, w, y_pitch=N + 3)
    _check(x, w, got[:, :N], label=f"M={M} N={N} K={K}")
    assert np.all(got[:, N:] == SENT), "columns beyond N were written"


@pytest.mark.parametrize("rows", [1, 16, 32, 64, 256, 512])
def test_in_proj_full_shape(rows):
    heads = 12
    N = 4 * 128 * heads + 128 + heads
    x, w = make_linear(rows, N, HIDDEN, seed=rows)
    got = _run(x, w, fn="in_proj", heads=heads)
    rng = np.random.default_rng(rows)
    ms, ns = rng.integers(0, rows, 3000), rng.integers(0, N, 3000)
    _check(x, w, got, ms, ns, label=f"in_proj rows={rows}")
    again = _run(x, w, fn="in_proj", heads=heads)
    assert np.array_equal(got, again), "not deterministic"


@pytest.mark.parametrize("rows", [33, 48, 64, 65, 128, 192, 256])
def test_in_proj_split_k(rows):
    """33 to 256 rows with a workspace: K split over 4 slices, then the ordered sum."""
    import kimi_delta_attention_conv_amd as kda
    heads = 12
    N = 4 * 128 * heads + 128 + heads
    assert kda.kda_linear_workspace_bytes(rows, N, HIDDEN) > 0
    x, w = make_linear(rows, N, HIDDEN, seed=300 + rows)
    got = _run(x, w, y_pitch=N + 5, fn="in_proj", heads=heads, workspace="auto")
    assert np.all(got[:, N:] == SENT), "columns beyond N were written"
    got = got[:, :N]
    rng = np.random.default_rng(rows + 7)
    ms, ns = rng.integers(0, rows, 4000), rng.integers(0, N, 4000)
    ms[:2], ns[:2] = rows - 1, N - 1           # the last row and column of the last tile
    _check(x, w, got, ms, ns, label=f"in_proj split rows={rows}")
    again = _run(x, w, fn="in_proj", heads=heads, workspace="auto")
    assert np.array_equal(got, again), "not deterministic"
    # too small a workspace takes the unsplit kernel, as does none at all
    small = _run(x, w, fn="in_proj", heads=heads,
                 workspace=kda.kda_linear_workspace_bytes(rows, N, HIDDEN) - 16)
    none = _run(x, w, fn="in_proj", heads=heads)
    assert np.array_equal(small, none)
    _check(x, w, none, ms, ns, label=f"in_proj unsplit rows={rows}")


@pytest.mark.parametrize("M,N", [(40, 300), (64, 129), (33, 1), (100, 300), (129, 130),
                                 (256, 200)])
def test_split_k_ragged_full(M, N):
    """Every output of a split shape whose N is not a multiple of the 128-wide tile."""
    K = 4096
    x, w = make_linear(M, N, K, seed=M * 31 + N, x_pitch=K + 8)
    got = _run(x, w, y_pitch=N + 3, workspace="auto")
    _check(x, w, got[:, :N], label=f"split M={M} N={N} K={K}")
    assert np.all(got[:, N:] == SENT), "columns beyond N were written"


@pytest.mark.parametrize("rows", [1, 16, 32, 64, 256, 512])
def test_o_proj_full_shape(rows):
    heads = 12
    x, w = make_linear(rows, HIDDEN, 128 * heads, seed=10 + rows)
    got = _run(x, w, fn="o_proj", heads=heads)
    rng = np.random.default_rng(rows + 1)
    ms, ns = rng.integers(0, rows, 3000), rng.integers(0, HIDDEN, 3000)
    _check(x, w, got, ms, ns, label=f"o_proj rows={rows}")


def test_validation():
    import kimi_delta_attention_conv_amd as kda
    x, w = make_linear(4, 16, 64, seed=5)
    xd, wd = x.cuda(), w.cuda()
    y = torch.zeros(4, 16, dtype=torch.bfloat16, device="cuda")
    for args, status in [((xd.data_ptr(), 64, wd.data_ptr(), y.data_ptr(), 16, 4, 16, 60), -2),
                         ((xd.data_ptr(), 60, wd.data_ptr(), y.data_ptr(), 16, 4, 16, 64), -2),
                         ((xd.data_ptr() + 8, 64, wd.data_ptr(), y.data_ptr(), 16, 4, 16, 64), -3),
                         ((0, 64, wd.data_ptr(), y.data_ptr(), 16, 4, 16, 64), -1),
                         ((xd.data_ptr(), 64, wd.data_ptr(), y.data_ptr(), 8, 4, 16, 64), -2)]:
        with pytest.raises(kda.KdaError) as ei:
            kda.kda_linear(*args)
        assert ei.value.status == status
    with pytest.raises(kda.KdaError) as ei:   # a workspace not 16-byte aligned
        kda.kda_linear(xd.data_ptr(), 64, wd.data_ptr(), y.data_ptr(), 16, 4, 16, 64,
                       y.data_ptr() + 4, 64)
    assert ei.value.status == -3
    kda.kda_linear(0, 64, 0, 0, 16, 0, 16, 64)   # M == 0: no-op
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_torch_helper_matches_the_abi_call():
    """kimi_delta_attention_conv_amd.linear (torch tensors, a workspace allocated on
    demand) gives the same bits as kda_linear called directly with the same choice
    of path, and passes workspace=None through to the unsplit kernel."""
    import kimi_delta_attention_conv_amd as kda
    M, N, K = 48, 300, 4096
    x, w = make_linear(M, N, K, seed=77)
    direct_split = _run(x, w, workspace="auto")
    direct_plain = _run(x, w)
    got_split = bf16_np(kda.linear(x.cuda(), w.cuda()).cpu())
    got_plain = bf16_np(kda.linear(x.cuda(), w.cuda(), workspace=None).cpu())
    torch.cuda.synchronize()
    assert np.array_equal(got_split, direct_split)
    assert np.array_equal(got_plain, direct_plain)
    with pytest.raises(ValueError):
        kda.linear(x.cuda(), w.cuda(), workspace="bogus")


def _pipe_class(M, N, K):
    """Whether kda_linear takes the pipelined kernel with prefetching workgroups:
    above 256 rows, K >= 4096 (a multiple of 64), 128 x 128 tiles filling three
    quarters to all but one of the device's compute units."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = -(-M // 128) * -(-N // 128)
    return M > 256 and K >= 4096 and K % 64 == 0 and tiles < cus and 4 * tiles >= 3 * cus


@pytest.mark.parametrize("M,N,K", [(449, 6200, 4096), (500, 6300, 4160), (385, 6144, 4096)])
def test_pipelined_prefetch_shapes(M, N, K):
    """Ragged shapes of the pipelined kernel (an odd K-block count among them):
    every output against the oracle's bar, columns past N untouched, and bit for
    bit the same as the same product computed in two halves of N, each of which
    has too few tiles for that kernel and runs the plain 128 x 128 tile kernel
    with the same summation order."""
    if not _pipe_class(M, N, K):
        pytest.skip("the device's compute-unit count puts this shape outside the pipelined class")
    x, w = make_linear(M, N, K, seed=M + N + K, x_pitch=K + 8)
    got = _run(x, w, y_pitch=N + 3)
    assert np.all(got[:, N:] == SENT), "columns beyond N were written"
    got = got[:, :N]
    rng = np.random.default_rng(M)
    ms, ns = rng.integers(0, M, 6000), rng.integers(0, N, 6000)
    ms[:3], ns[:3] = [M - 1, 0, M - 1], [N - 1, N - 1, 0]
    _check(x, w, got, ms, ns, label=f"pipelined M={M} N={N} K={K}")
    h = N // 2
    assert not _pipe_class(M, h, K) and not _pipe_class(M, N - h, K)
    lo = _run(x, w[:h].contiguous())
    hi = _run(x, w[h:].contiguous())
    assert np.array_equal(got, np.concatenate([lo, hi], axis=1)), "differs from the plain tile kernel"
    again = _run(x, w, y_pitch=N + 3)
    assert np.array_equal(got, again[:, :N]), "not deterministic"


def test_pipelined_prefetch_graph_replays_equal_eager():
    """The pipelined kernel with prefetching workgroups at in_proj's 512-row shape,
    captured in a HIP graph once and replayed with three different inputs (eager work
    between the replays): every replay equals the eager call bit for bit."""
    import kimi_delta_attention_conv_amd as kda
    heads = 12
    M, N, K = 512, 4 * 128 * heads + 128 + heads, HIDDEN
    if not _pipe_class(M, N, K):
        pytest.skip("the device's compute-unit count puts this shape outside the pipelined class")
    _, w = make_linear(1, N, K, seed=901)
    wd = w.cuda()
    gen = torch.Generator().manual_seed(902)
    inputs = [torch.randn(M, K, generator=gen).to(torch.bfloat16) for _ in range(3)]
    x = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")

    def call():
        kda.kda_linear(x.data_ptr(), K, wd.data_ptr(), y.data_ptr(), N, M, N, K,
                       stream=torch.cuda.current_stream().cuda_stream)

    ref = []
    for xi in inputs:
        x.copy_(xi)
        call()
        torch.cuda.synchronize()
        ref.append(y.cpu().view(torch.int16).clone())
    y.zero_()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for k, xi in enumerate(inputs):
        x.copy_(xi)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.cpu().view(torch.int16), ref[k]), f"replay {k}"
    print("[linear] pipelined 512-row in_proj: 3 graph replays equal eager", flush=True)
