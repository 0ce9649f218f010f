"""The core under HIP graph capture: decode and verify launches recorded once and
replayed several times, with new inputs copied into the static buffers between
replays (eager work and synchronisation in between), must equal the same
launches run eagerly, bit for bit, on every replay."""
import numpy as np
import pytest
import torch

from kda_inputs import make_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pools(case):
    conv = case.conv_storage.clone().cuda()
    state = case.state.clone().cuda()
    return conv, state


def _core(case, conv, state):
    import kimi_delta_attention_conv_amd as kda
    view = conv if case.conv_dim_first else conv.transpose(-1, -2)
    return kda.KdaCore(conv_weight=case.conv_weight.cuda(), conv_bias=case.conv_bias.cuda(),
                       f_b=case.f_b.cuda(), A_log=case.A_log.cuda(), dt_bias=case.dt_bias.cuda(),
                       norm_weight=case.norm_weight.cuda(), gate_lower_bound=case.gate_lower_bound,
                       norm_eps=case.norm_eps, l2_eps=case.l2_eps, conv=view, state=state)


@pytest.mark.parametrize("verify", [False, True])
def test_graph_replays_equal_eager(verify):
    case = make_case(R=6, L=3 if verify else 1, H=2, num_slots=32, seed=500 + verify, verify=verify)
    gen = torch.Generator().manual_seed(501)
    inputs = [torch.randn(case.S, case.pitch, generator=gen).to(torch.bfloat16) for _ in range(4)]
    slots = case.slots.cuda()
    acc = case.accepted.cuda() if verify else None

    def step(core, proj, out):
        if verify:
            core.verify(proj, out, slots, acc)
        else:
            core.decode(proj, out, slots)

    # eager reference: four steps on one set of pools
    conv_e, state_e = _pools(case)
    core_e = _core(case, conv_e, state_e)
    proj_e = torch.empty(case.S, case.pitch, dtype=torch.bfloat16, device="cuda")
    out_e = torch.empty(case.S, case.D, dtype=torch.bfloat16, device="cuda")
    ref = []
    for x in inputs:
        proj_e.copy_(x)
        step(core_e, proj_e, out_e)
        torch.cuda.synchronize()
        ref.append((out_e.cpu().clone(), state_e.cpu().clone(), conv_e.cpu().clone()))
    core_e.close()

    # captured once, replayed four times
    conv_g, state_g = _pools(case)
    core_g = _core(case, conv_g, state_g)
    proj_g = torch.zeros(case.S, case.pitch, dtype=torch.bfloat16, device="cuda")
    out_g = torch.empty(case.S, case.D, dtype=torch.bfloat16, device="cuda")
    # capture on a copy of the pools' starting point: the capture itself does not execute
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(core_g, proj_g, out_g)
    torch.cuda.synchronize()
    assert torch.equal(state_g.cpu(), case.state), "capture must not run the kernel"
    for k, x in enumerate(inputs):
        proj_g.copy_(x)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out, st, cv = ref[k]
        assert torch.equal(out_g.cpu().view(torch.int16), out.view(torch.int16)), f"replay {k}: out"
        assert torch.equal(state_g.cpu(), st), f"replay {k}: state"
        assert torch.equal(conv_g.cpu().view(torch.int16), cv.view(torch.int16)), f"replay {k}: conv"
    assert core_g.device_errors() == 0
    core_g.close()
    print(f"[graph] {'verify' if verify else 'decode'}: 4 replays equal eager", flush=True)


def test_layer_graph_replays_equal_eager():
    """in_proj (K split through a workspace: two launches) -> decode -> o_proj, captured
    once and replayed with four different hidden inputs, equals the eager sequence bit
    for bit on every replay (projected rows, core_out, o_proj output, both pools)."""
    import kimi_delta_attention_conv_amd as kda
    from kda_inputs import make_linear
    R, H, hidden = 48, 2, 4096
    case = make_case(R=R, L=1, H=H, num_slots=64, seed=520)
    D, pitch = case.D, case.pitch
    n_in = 4 * D + 128 + H
    ws_bytes = max(kda.kda_linear_workspace_bytes(R, n_in, hidden),
                   kda.kda_linear_workspace_bytes(R, hidden, D))
    assert ws_bytes > 0, "this shape must take the K split"
    w_in = make_linear(1, n_in, hidden, seed=521)[1].cuda()
    w_o = make_linear(1, hidden, D, seed=522)[1].cuda()
    gen = torch.Generator().manual_seed(523)
    inputs = [torch.randn(R, hidden, generator=gen).to(torch.bfloat16) for _ in range(4)]
    slots = case.slots.cuda()

    def buffers():
        conv, state = _pools(case)
        core = _core(case, conv, state)
        x = torch.zeros(R, hidden, dtype=torch.bfloat16, device="cuda")
        proj = torch.zeros(R, pitch, dtype=torch.bfloat16, device="cuda")
        core_out = torch.empty(R, D, dtype=torch.bfloat16, device="cuda")
        y = torch.empty(R, hidden, dtype=torch.bfloat16, device="cuda")
        work = torch.full((ws_bytes // 4,), float("nan"), device="cuda")
        return conv, state, core, x, proj, core_out, y, work

    def step(core, x, proj, core_out, y, work):
        s = torch.cuda.current_stream().cuda_stream
        kda.kda_in_proj(x.data_ptr(), hidden, w_in.data_ptr(), proj.data_ptr(), pitch, R,
                        hidden, H, work.data_ptr(), ws_bytes, stream=s)
        core.decode(proj, core_out, slots)
        kda.kda_o_proj(core_out.data_ptr(), D, w_o.data_ptr(), y.data_ptr(), hidden, R, H,
                       hidden, work.data_ptr(), ws_bytes, stream=s)

    conv_e, state_e, core_e, x_e, proj_e, co_e, y_e, work_e = buffers()
    ref = []
    for x in inputs:
        x_e.copy_(x)
        step(core_e, x_e, proj_e, co_e, y_e, work_e)
        torch.cuda.synchronize()
        ref.append([t.cpu().clone() for t in (proj_e, co_e, y_e, state_e, conv_e)])
    core_e.close()

    conv_g, state_g, core_g, x_g, proj_g, co_g, y_g, work_g = buffers()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(core_g, x_g, proj_g, co_g, y_g, work_g)
    torch.cuda.synchronize()
    assert torch.equal(state_g.cpu(), case.state), "capture must not run the kernels"
    names = ("projected", "core_out", "o_proj out", "state", "conv")
    for k, x in enumerate(inputs):
        x_g.copy_(x)
        work_g.fill_(float("nan"))                # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu() for t in (proj_g, co_g, y_g, state_g, conv_g)]
        for name, g, r in zip(names, got, ref[k]):
            gi = g.view(torch.int16) if g.dtype == torch.bfloat16 else g
            ri = r.view(torch.int16) if r.dtype == torch.bfloat16 else r
            assert torch.equal(gi, ri), f"replay {k}: {name}"
    assert core_g.device_errors() == 0
    core_g.close()
    print("[graph] layer (split in_proj -> decode -> o_proj): 4 replays equal eager", flush=True)
