"""The state-stream probe (include/kda_probe.h) writes exactly what it declares.

kda_probe_state_stream replays the core kernel's state traffic without its
arithmetic, for the bench's pattern ceiling. Checked here bit for bit on a small
pool: each request's carried tile, scaled by 0.999f once per token in fp32,
lands in every destination slot; skipped requests and every other slot stay
untouched; the decode form scales in place. Every variant (with and without the
barrier between loads and stores, with and without the core's residency) writes
the same."""
import numpy as np
import pytest
import torch

from kimi_delta_attention_conv_amd import probe as kprobe

pytestmark = pytest.mark.gpu

TILE = 128 * 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _expected(pool, table, accepted, tokens, valid):
    """fp32 reference: token t of request r writes c^(t+1) * state[src]."""
    out = pool.copy()
    c = np.float32(0.999)
    for r in range(table.shape[0]):
        if not valid[r]:
            continue
        a = 1 if accepted is None else int(accepted[r])
        tile = pool[table[r, a - 1]].copy()
        for t in range(tokens):
            tile = (tile * c).astype(np.float32)
            out[table[r, t]] = tile
    return out


# (tokens, verify, requests, heads): 15-unit grids take the probe's 16-wave form,
# 32 x 12 = 384 units with two tokens its 8-wave form (on a 256-CU device)
@pytest.mark.parametrize("options", [0, 1, 2, 3])
@pytest.mark.parametrize("tokens,verify,R,H", [(3, True, 5, 3), (8, True, 5, 3), (1, False, 5, 3),
                                               (2, True, 32, 12)])
def test_state_stream_probe_writes_scaled_carried_tiles(tokens, verify, R, H, options):
    print(f"[case] state stream probe tokens={tokens} verify={verify} R={R} H={H} "
          f"options={options}", flush=True)
    lib = kprobe.load_probe_library()
    num_slots, cols = (64, 8 if tokens == 8 else 4) if R * 4 <= 64 else (160, 4)
    g = torch.Generator().manual_seed(900 + tokens)
    pool = torch.randn(num_slots, H, TILE, generator=g).numpy().astype(np.float32)
    perm = torch.randperm(num_slots, generator=g).numpy().astype(np.int32)
    table = perm[:R * cols].reshape(R, cols).copy()
    if not verify:
        table = table[:, :1].copy()
    table[R - 1, 0] = num_slots            # out of range: the last request is skipped
    valid = [True] * (R - 1) + [False]
    accepted = (torch.randint(1, tokens + 1, (R,), generator=g).numpy().astype(np.int32)
                if verify else None)
    dev = "cuda"
    state = torch.from_numpy(pool).to(dev)
    slots = torch.from_numpy(table).to(dev)
    acc = None if accepted is None else torch.from_numpy(accepted).to(dev)
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.kda_probe_state_stream(state.data_ptr(), H * TILE, num_slots, slots.data_ptr(),
                                    table.shape[1], None if acc is None else acc.data_ptr(),
                                    R, tokens, H, options, stream)
    assert rc == 0
    torch.cuda.synchronize()
    want = _expected(pool, table, accepted, tokens, valid)
    got = state.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
