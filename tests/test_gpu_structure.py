"""Structural, bit-exact properties of the HIP path (through the C ABI).

Identity mode (g = 0, beta = 0) shows slot and accepted-count selection bit for
bit; decode equals a one-token verify; verify over L tokens equals L chained
decodes; both conv layouts, strided slots, a padded pitch, per-head norm
weights and no conv bias are handled; invalid requests are skipped and counted;
an empty call is a no-op; host validation rejects bad arguments and leaves the
device untouched."""
import numpy as np
import pytest
import torch

from kda_inputs import make_case, make_config
from oracle_cases import run_oracle
from parity import assert_parity, request_slots

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _identity_projected(case):
    proj = case.projected.clone()
    D = case.D
    proj[:, 4 * D + 128: 4 * D + 128 + case.H] = float("-inf")   # beta = 0
    return proj


@pytest.mark.parametrize("which", ["small", "verify_r64_l8"])
def test_identity_mode_selects_accepted_state_bit_exact(which):
    from gpu_cases import run_gpu
    case = make_case(R=9, L=5, H=2, num_slots=64, seed=400, verify=True) if which == "small" \
        else make_config(3)
    print(f"[case] identity mode {which}", flush=True)
    proj = _identity_projected(case)
    got = run_gpu(case, projected=proj, gate_lower_bound=0.0)
    before = case.state.numpy()
    assert got["errors"] == 0
    for r, (ok, src, dst) in enumerate(request_slots(case)):
        assert ok
        for t, d in enumerate(dst):
            assert np.array_equal(got["state"][d], before[src]), (r, t)


def test_decode_equals_single_token_verify_bit_exact():
    from gpu_cases import run_gpu
    case = make_case(R=20, L=1, H=3, num_slots=40, seed=401, verify=False)
    a = run_gpu(case)
    b = run_gpu(case, accepted=torch.ones(case.R, dtype=torch.int32), decode=False)
    for k in ("out", "conv", "state"):
        assert np.array_equal(a[k], b[k]), k


def test_verify_equals_chained_decodes_bit_exact():
    """The kernel's per-token arithmetic does not depend on L: a verify call and L
    decode calls chained on one slot agree bit for bit."""
    from gpu_cases import GpuCase
    case = make_case(R=4, L=6, H=2, num_slots=32, seed=402, verify=True)
    g = GpuCase(case).run()
    full = g.host()
    g.close()
    reqs = request_slots(case)
    for r, (ok, src, dst) in enumerate(reqs):
        dec = make_case(R=1, L=1, H=2, num_slots=32, seed=402, verify=False)
        dec.conv_weight, dec.conv_bias, dec.f_b = case.conv_weight, case.conv_bias, case.f_b
        dec.A_log, dec.dt_bias, dec.norm_weight = case.A_log, case.dt_bias, case.norm_weight
        state = case.state.clone()
        conv = case.conv_storage.clone()
        tmp = dst[0]
        state[tmp] = state[src]
        conv[tmp] = conv[src]
        dec.state, dec.conv_storage = state, conv
        dec.slots = torch.tensor([tmp], dtype=torch.int32)
        gd = GpuCase(dec)
        try:
            for t in range(case.L):
                row = r * case.L + t
                gd.run(projected=case.projected[row:row + 1])
                h = gd.host()
                assert np.array_equal(h["out"][0], full["out"][row]), (r, t)
                assert np.array_equal(h["state"][tmp], full["state"][dst[t]]), (r, t)
                assert np.array_equal(h["conv"][tmp], full["conv"][dst[t]]), (r, t)
        finally:
            gd.close()


def test_conv_layouts_agree_bit_exact():
    from gpu_cases import run_gpu
    a = make_case(R=6, L=3, H=2, num_slots=32, seed=403, verify=True, conv_dim_first=True)
    b = make_case(R=6, L=3, H=2, num_slots=32, seed=403, verify=True, conv_dim_first=True)
    b.conv_dim_first = False
    b.conv_storage = a.conv_storage.transpose(1, 2).contiguous()
    ra, rb = run_gpu(a), run_gpu(b)
    assert np.array_equal(ra["out"], rb["out"])
    assert np.array_equal(ra["state"], rb["state"])
    assert np.array_equal(ra["conv"], rb["conv"].transpose(0, 2, 1))


def test_strided_block_table_slots_equal_contiguous_copy():
    from gpu_cases import run_gpu
    case = make_case(R=8, L=4, H=2, num_slots=96, seed=404, verify=True, block_table_cols=11)
    assert case.slots.stride(0) == 11
    a = run_gpu(case)
    b = run_gpu(case, slots=case.slots.contiguous())
    for k in ("out", "conv", "state"):
        assert np.array_equal(a[k], b[k]), k


def test_invalid_requests_are_skipped_and_counted():
    from gpu_cases import run_gpu
    case = make_case(R=6, L=3, H=2, num_slots=24, seed=405, verify=True)
    s = case.slots.clone()
    acc = case.accepted.clone()
    s[1, 0] = case.num_slots       # out of range
    s[3, 2] = -1                   # negative
    acc[4] = 0                     # not in 1..L
    acc[5] = case.L + 1
    case.slots, case.accepted = s, acc
    before = case.state.numpy().copy()
    ref = run_oracle(case)
    got = run_gpu(case)
    assert ref["skipped"] == 4
    assert_parity(case, ref, got, before, label="invalid requests")


def test_empty_call_is_a_noop():
    from gpu_cases import GpuCase
    case = make_case(R=2, L=2, H=2, num_slots=8, seed=406, verify=True)
    g = GpuCase(case)
    try:
        before = g.state.clone()
        empty = torch.empty(0, case.pitch, dtype=torch.bfloat16, device="cuda")
        out = torch.empty(0, case.D, dtype=torch.bfloat16, device="cuda")
        slots = torch.empty(0, 2, dtype=torch.int32, device="cuda")
        g.core.verify(empty, out, slots, torch.empty(0, dtype=torch.int32, device="cuda"))
        g.core.decode(empty, out, torch.empty(0, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(before, g.state)
        assert g.core.device_errors() == 0
    finally:
        g.close()


def test_padded_pitch_per_head_norm_and_no_bias():
    from gpu_cases import run_gpu
    case = make_case(R=5, L=2, H=3, num_slots=24, seed=407, verify=True, with_bias=False,
                     pitch=4 * 384 + 128 + 3 + 11)
    nw = torch.rand(case.H, 128, generator=torch.Generator().manual_seed(9)) + 0.5
    before = case.state.numpy().copy()
    ref = run_oracle(case, norm_weight=nw.numpy().reshape(-1), norm_head_stride=128)
    got = run_gpu(case, norm_weight=nw)
    assert_parity(case, ref, got, before, label="padded pitch, per-head norm, no bias")


def test_host_validation_leaves_device_untouched():
    import kimi_delta_attention_conv_amd as kda
    from gpu_cases import GpuCase
    case = make_case(R=2, L=3, H=2, num_slots=8, seed=408, verify=True)
    g = GpuCase(case)
    try:
        before = g.state.clone()
        h = g.core.handle
        p, o = g.projected, g.out
        slots = case.slots.cuda()
        acc = case.accepted.cuda()
        cases = [
            (lambda: kda.kda_verify(h, p.data_ptr(), case.pitch - 2, 2, 3, slots.data_ptr(), 3,
                                    acc.data_ptr(), o.data_ptr()), -2),
            (lambda: kda.kda_verify(h, p.data_ptr(), case.pitch - 1, 2, 3, slots.data_ptr(), 3,
                                    acc.data_ptr(), o.data_ptr()), -2),
            (lambda: kda.kda_verify(h, p.data_ptr(), case.pitch, 2, 9, slots.data_ptr(), 9,
                                    acc.data_ptr(), o.data_ptr()), -4),
            (lambda: kda.kda_verify(h, p.data_ptr(), case.pitch, 2, 3, slots.data_ptr(), 2,
                                    acc.data_ptr(), o.data_ptr()), -2),
            (lambda: kda.kda_verify(h, p.data_ptr(), case.pitch, 2, 3, slots.data_ptr(), 3,
                                    0, o.data_ptr()), -1),
            (lambda: kda.kda_verify(h, p.data_ptr() + 1, case.pitch, 2, 3, slots.data_ptr(), 3,
                                    acc.data_ptr(), o.data_ptr()), -3),
            (lambda: kda.kda_decode(h, p.data_ptr(), case.pitch, -1, slots.data_ptr(),
                                    o.data_ptr()), -2),
            (lambda: kda.kda_decode(h, p.data_ptr(), case.pitch, 2, slots.data_ptr(),
                                    o.data_ptr() + 2), -3),
        ]
        for fn, status in cases:
            with pytest.raises(kda.KdaError) as ei:
                fn()
            assert ei.value.status == status
        # the torch wrapper refuses host tensors and too-narrow rows before any call
        core = g.core
        p2d = p.view(case.S, case.pitch)
        with pytest.raises(TypeError):
            core.verify(p2d.cpu(), o, slots, acc)
        with pytest.raises(TypeError):
            core.verify(p2d, o, slots.cpu(), acc)
        with pytest.raises(TypeError):
            core.verify(p2d, o, slots, acc.cpu())
        with pytest.raises(TypeError):
            core.decode(p2d, o.cpu(), slots.reshape(-1))
        with pytest.raises(ValueError):
            core.verify(p2d[:, :case.pitch - 8], o, slots, acc)
        torch.cuda.synchronize()
        assert torch.equal(before, g.state)
        assert g.core.device_errors() == 0
    finally:
        g.close()


def test_padded_state_slot_stride_and_more_heads():
    """A state pool whose slots carry padding (slot stride > H*128*128) and a head
    count outside the workload set (H = 16, D = 2048)."""
    import kimi_delta_attention_conv_amd as kda
    from gpu_cases import OUT_SENTINEL
    case = make_case(R=3, L=2, H=16, num_slots=9, seed=409, verify=True)
    pad = 4096
    unit = case.H * 128 * 128
    before = case.state.numpy().copy()
    ref = run_oracle(case)
    big = torch.full((case.num_slots, unit + pad), -7.0, dtype=torch.float32)
    big[:, :unit] = case.state.reshape(case.num_slots, unit)
    dev = big.cuda()
    state_view = torch.as_strided(dev, (case.num_slots, case.H, 128, 128),
                                  (unit + pad, 128 * 128, 128, 1))
    conv = case.conv_storage.cuda()
    core = kda.KdaCore(conv_weight=case.conv_weight.cuda(), conv_bias=case.conv_bias.cuda(),
                       f_b=case.f_b.cuda(), A_log=case.A_log.cuda(), dt_bias=case.dt_bias.cuda(),
                       norm_weight=case.norm_weight.cuda(), gate_lower_bound=case.gate_lower_bound,
                       norm_eps=case.norm_eps, l2_eps=case.l2_eps, conv=conv, state=state_view)
    out = torch.full((case.S, case.D), OUT_SENTINEL, dtype=torch.int16).view(torch.bfloat16).cuda()
    core.verify(case.projected.cuda(), out, case.slots.cuda(), case.accepted.cuda())
    torch.cuda.synchronize()
    host = dev.cpu()
    assert torch.all(host[:, unit:] == -7.0), "slot padding was written"
    got = dict(out=out.cpu().view(torch.int16).numpy().view(np.uint16),
               conv=conv.cpu().view(torch.int16).numpy().view(np.uint16),
               state=host[:, :unit].reshape(case.num_slots, case.H, 128, 128).numpy(),
               errors=core.device_errors())
    core.close()
    assert_parity(case, ref, got, before, label="padded slot stride, H=16")


def test_conv_fast_and_generic_store_paths_agree():
    """A dim-first conv pool with a 16-byte aligned base takes the staged 16-byte
    window stores; the same pool one element off alignment takes the per-element
    path. Both must give bit-identical pools, states and outputs."""
    import kimi_delta_attention_conv_amd as kda
    case = make_case(R=5, L=4, H=3, num_slots=24, seed=410, verify=True)
    results = []
    for offset in (0, 1):
        flat = torch.zeros(case.conv_storage.numel() + 8, dtype=torch.bfloat16)
        flat[offset: offset + case.conv_storage.numel()] = case.conv_storage.reshape(-1)
        dflat = flat.cuda()
        conv = torch.as_strided(dflat, case.conv_storage.shape, case.conv_storage.stride(), offset)
        state = case.state.cuda()
        core = kda.KdaCore(conv_weight=case.conv_weight.cuda(), conv_bias=case.conv_bias.cuda(),
                           f_b=case.f_b.cuda(), A_log=case.A_log.cuda(),
                           dt_bias=case.dt_bias.cuda(), norm_weight=case.norm_weight.cuda(),
                           gate_lower_bound=case.gate_lower_bound, norm_eps=case.norm_eps,
                           l2_eps=case.l2_eps, conv=conv, state=state)
        out = torch.zeros(case.S, case.D, dtype=torch.bfloat16, device="cuda")
        core.verify(case.projected.cuda(), out, case.slots.cuda(), case.accepted.cuda())
        torch.cuda.synchronize()
        assert core.device_errors() == 0
        core.close()
        results.append((conv.cpu().view(torch.int16), state.cpu(), out.cpu().view(torch.int16)))
    for a, b in zip(results[0], results[1]):
        assert torch.equal(a, b)


def test_bf16_small_weights_equal_fp32_bit_exact():
    """A_log, dt_bias and the norm weight given as bf16 are converted at prepare time:
    the results equal those from fp32 tensors holding the same values, bit for bit,
    and meet the oracle's bars."""
    import dataclasses
    from gpu_cases import run_gpu
    base = make_case(8, 3, 4, 64, seed=940, verify=True)
    rounded = dataclasses.replace(
        base, A_log=base.A_log.to(torch.bfloat16).float(),
        dt_bias=base.dt_bias.to(torch.bfloat16).float(),
        norm_weight=base.norm_weight.to(torch.bfloat16).float())
    as_bf16 = dataclasses.replace(
        rounded, A_log=rounded.A_log.to(torch.bfloat16), dt_bias=rounded.dt_bias.to(torch.bfloat16),
        norm_weight=rounded.norm_weight.to(torch.bfloat16))
    f32 = run_gpu(rounded)
    b16 = run_gpu(as_bf16)
    for key in ("out", "conv", "state"):
        assert np.array_equal(f32[key], b16[key]), key
    assert_parity(rounded, run_oracle(rounded), b16, rounded.state.numpy(), label="bf16 small weights")


@pytest.mark.parametrize("L", [2, 4])
def test_eight_and_sixteen_wave_units_agree_bit_exact(L):
    """The kernel runs a unit with 16 waves of 8 state rows for one-token calls and
    for grids of at most one unit a compute unit, else with 8 waves of 16 rows; the
    per-row arithmetic is the same in both. Requests are independent, so one verify
    call over 32 requests x 12 heads (384 units: 8 waves on a 256-CU MI355X) and the
    same requests as two calls of 16 (192 units each: 16 waves) must agree bit for
    bit."""
    from gpu_cases import GpuCase
    print(f"[case] wave shapes L={L}", flush=True)
    R = 32
    case = make_case(R=R, L=L, H=12, num_slots=128, seed=430 + L, verify=True)
    whole = GpuCase(case).run().host()
    g = GpuCase(case)
    half = R // 2
    slots = g.case.slots.cuda()
    acc = torch.as_tensor(case.accepted, dtype=torch.int32).cuda()
    for k in range(2):
        rows = slice(k * half * L, (k + 1) * half * L)
        g.core.verify(g.projected[rows], g.out[rows], slots[k * half:(k + 1) * half],
                      acc[k * half:(k + 1) * half])
    torch.cuda.synchronize()
    split = g.host()
    for key in ("out", "conv", "state"):
        assert np.array_equal(whole[key].view(np.uint8), split[key].view(np.uint8)), key
    assert whole["errors"] == split["errors"] == 0


@pytest.mark.parametrize("kind", ["across", "within", "decode"])
def test_distinct_check_skips_colliding_requests(kind):
    """With check_distinct, every request naming a destination slot that another
    (request, token) of the call also names is skipped and counted, exactly as the
    oracle's checked mode defines it; the others are unaffected."""
    import dataclasses

    from gpu_cases import run_gpu
    if kind == "decode":
        base = make_case(R=8, L=1, H=3, num_slots=16, seed=406, verify=False)
        s = base.slots.clone()
        s[5] = s[1]
        involved = {1, 5}
    else:
        base = make_case(R=6, L=3, H=2, num_slots=32, seed=407, verify=True)
        s = base.slots.clone()
        if kind == "across":
            s[3, 1] = s[0, 2]
            involved = {0, 3}
        else:
            s[2, 2] = s[2, 0]
            involved = {2}
    case = dataclasses.replace(base, slots=s)
    print(f"[case] distinct check {kind}", flush=True)
    ref = run_oracle(case, check_distinct=True)
    assert ref["skipped"] == len(involved)
    got = run_gpu(case, check_distinct=True)
    assert_parity(case, ref, got, case.state.numpy(), skip=involved, label=f"distinct_{kind}")


def test_distinct_check_resets_between_calls():
    """The per-slot claims are cleared at the end of every call: a call with a
    collision, then a call without one on the same handle, skips only in the first
    (both checked against the oracle's checked mode, chained)."""
    import dataclasses

    from gpu_cases import GpuCase
    base = make_case(R=6, L=2, H=2, num_slots=24, seed=409, verify=True)
    s1 = base.slots.clone()
    s1[4, 0] = s1[1, 1]
    first = dataclasses.replace(base, slots=s1)
    ref1 = run_oracle(first, check_distinct=True)
    assert ref1["skipped"] == 2
    g = GpuCase(first, check_distinct=True)
    try:
        g.run()
        h1 = g.host()
        assert h1["errors"] == 2
        g.run(slots=base.slots)
        h2 = g.host()
        assert h2["errors"] == 0
    finally:
        g.close()
    conv1 = torch.from_numpy(ref1["conv"].view(np.int16)).view(torch.bfloat16)
    second = dataclasses.replace(base, state=torch.from_numpy(ref1["state"]), conv_storage=conv1)
    ref2 = run_oracle(second, check_distinct=True)
    assert ref2["skipped"] == 0
    # slots untouched by the second call keep the GPU's first-call values
    assert_parity(second, ref2, h2, h1["state"], label="distinct_second_call")


def test_odd_pitch_equals_padded_pitch_bit_exact():
    """An odd pitch (4D + 128 + H for odd H, rows only 2-byte aligned) and a
    projected base that is only 2-byte aligned take 2-byte loads of f_a; the results
    equal those of the same rows padded to an even pitch, bit for bit, and meet the
    oracle's bars."""
    import dataclasses

    from gpu_cases import GpuCase
    case = make_case(R=5, L=3, H=3, num_slots=32, seed=408, verify=True)
    assert case.pitch % 2 == 1
    padded = torch.zeros(case.S, case.pitch + 1, dtype=torch.bfloat16)
    padded[:, :case.pitch] = case.projected
    even = dataclasses.replace(case, projected=padded, pitch=case.pitch + 1)
    results = []
    for c, shift in ((case, 0), (case, 1), (even, 0)):
        buf = torch.zeros(c.S * c.pitch + 1, dtype=torch.bfloat16, device="cuda")
        buf[shift: shift + c.S * c.pitch] = c.projected.reshape(-1).cuda()
        proj = buf[shift: shift + c.S * c.pitch].view(c.S, c.pitch)
        assert proj.data_ptr() % 4 == 2 * shift
        print(f"[case] pitch {c.pitch} base offset {2 * shift} B", flush=True)
        g = GpuCase(c)
        try:
            g.run(projected=proj)
            results.append(g.host())
        finally:
            g.close()
    for k in ("out", "conv", "state"):
        assert np.array_equal(results[0][k], results[1][k]), k
        assert np.array_equal(results[0][k], results[2][k]), k
    ref = run_oracle(case)
    assert_parity(case, ref, results[0], case.state.numpy(), label="odd_pitch")
