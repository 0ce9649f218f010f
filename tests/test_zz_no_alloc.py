"""kda_linear_noalloc (the projection entry point that allocates nothing) through
the C ABI, against kda_linear given a caller's workspace: the same kernels, so
the outputs must agree bit for bit. Two calls in a row share the library's
static scratch buffer, the second with a smaller input, so a result that read
the first call's partial tiles would show; a shape that never splits and a
shape whose split would overflow the buffer (rejected before any work) are
covered too."""
import ctypes

import numpy as np
import pytest
import torch

import kimi_delta_attention_conv_amd as kda
from kda_inputs import HIDDEN, make_linear

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _pair(lib, M, N, K, seed):
    x, w = make_linear(M, N, K, seed=seed)
    xs, ws = x.cuda(), w.cuda()
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = int(lib.kda_linear_workspace_bytes(M, N, K))
    work = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    y_ref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    rc = lib.kda_linear(xs.data_ptr(), K, ws.data_ptr(), y_ref.data_ptr(), N, M, N, K,
                        work.data_ptr(), nbytes, stream)
    assert rc == 0
    rc = lib.kda_linear_noalloc(xs.data_ptr(), K, ws.data_ptr(), y.data_ptr(), N, M, N, K, stream)
    assert rc == 0, kda.kda_status_string(rc)
    torch.cuda.synchronize()
    return nbytes, _bits(y_ref), _bits(y)


def test_noalloc_equals_workspace_path_over_successive_calls():
    lib = kda.load_library()
    cap = int(lib.kda_noalloc_scratch_bytes())
    n_in = 4 * 1536 + 128 + 12
    # in_proj at 256 rows (26.2 MB of partial tiles), then 48 rows (6.4 MB) over
    # the same buffer, then o_proj at 512 rows (never split), then 40 rows again
    for M, N, K, seed in ((256, n_in, HIDDEN, 11), (48, n_in, HIDDEN, 12),
                          (512, HIDDEN, 1536, 13), (40, n_in - 1000, HIDDEN, 14)):
        print(f"[case] noalloc M={M} N={N} K={K}", flush=True)
        nbytes, ref, got = _pair(lib, M, N, K, seed)
        assert nbytes <= cap
        assert (nbytes > 0) == (M <= 256), (M, nbytes)
        assert not np.isnan((ref.astype(np.uint32) << 16).view(np.float32)).any()
        assert np.array_equal(ref, got), (M, N, K, int(np.count_nonzero(ref != got)))


def test_noalloc_rejects_a_split_larger_than_its_buffer():
    lib = kda.load_library()
    cap = int(lib.kda_noalloc_scratch_bytes())
    M, N, K = 256, 40000, 4096
    assert lib.kda_linear_workspace_bytes(M, N, K) > cap
    # buffers of the full shape, so that even a call that ran would stay in bounds
    x = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(N, K, dtype=torch.bfloat16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    rc = lib.kda_linear_noalloc(x.data_ptr(), K, w.data_ptr(), y.data_ptr(), N, M, N, K,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == -8
    assert "scratch" in kda.kda_status_string(rc)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
