"""Pins of the CPU oracle to facts outside itself.

Each check takes an `oracle.Oracle` and raises AssertionError when the oracle
disagrees with a closed form, an invariant, a library routine (torch / numpy /
scipy in float64) or brute force. test_oracle_pins.py runs them against the
oracle; test_oracle_mutations.py runs them against copies of the oracle with a
planted mistake and requires that at least one check fails for each copy.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import scipy.special
import torch

import oracle as om
from kda_inputs import make_case
from oracle_cases import bf16_np, run_oracle

PINS = []


def pin(fn):
    PINS.append(fn)
    return fn


def _close(a, b, rtol, atol=0.0, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    if not np.all(err <= lim):
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: max excess at {i}: {a.ravel()[i]!r} vs {b.ravel()[i]!r}")


def _silu(x):
    return torch.nn.functional.silu(torch.as_tensor(x, dtype=torch.float64)).numpy()


# ----------------------------------------------------------------- number formats

@pin
def check_bf16_roundtrip_all_patterns(orc):
    """Every finite bf16 pattern widens exactly and rounds back to itself."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = om.bf16_bits_to_f64(bits)
    finite = np.isfinite(vals)
    assert np.array_equal(orc.f64_to_bf16_bits(vals[finite]), bits[finite])
    for b in (0x0000, 0x3F80, 0xC2F7, 0x0001, 0x7F7F, 0x807F):
        assert orc.bf16_to_f64(b) == vals[b]


@pin
def check_bf16_rounding_matches_torch(orc):
    """fp32 -> bf16 round-to-nearest-even agrees with torch's cast, ties included."""
    rng = np.random.default_rng(11)
    f = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 3,
        (rng.standard_normal(500) * 1e-39).astype(np.float32),  # subnormals
        np.array([1e38, -3.3e38, 3.39e38], dtype=np.float32),
    ])
    # exact ties: a bf16 value plus half an ulp (low 16 bits 0x8000)
    hi = (rng.integers(0x0080, 0x7F00, 400, dtype=np.uint32) << 16) | 0x8000
    f = np.concatenate([f, hi.view(np.float32), -hi.view(np.float32)])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f64_to_bf16_bits(f.astype(np.float64)), ref)


@pin
def check_bf16_rounds_from_double_directly(orc):
    """A double just above a bf16 midpoint rounds up (no double rounding via fp32)."""
    x = 1.00390625 + 2.0 ** -40      # midpoint of 1.0 and 1.0078125, plus a hair
    assert orc.f64_to_bf16_bits(np.array([x]))[0] == 0x3F81
    assert orc.f64_to_bf16_bits(np.array([1.00390625]))[0] == 0x3F80  # tie -> even
    assert orc.f64_to_bf16_bits(np.array([1.01171875]))[0] == 0x3F82  # tie -> even


@pin
def check_sigmoid(orc):
    xs = np.concatenate([np.linspace(-40, 40, 801), [0.0, 1e-8, -700.0, 700.0]])
    got = np.array([orc.sigmoid(x) for x in xs])
    _close(got, scipy.special.expit(xs), 1e-15, 1e-300, "sigmoid vs expit")
    assert orc.sigmoid(0.0) == 0.5
    assert orc.sigmoid(float("inf")) == 1.0 and orc.sigmoid(float("-inf")) == 0.0


# ----------------------------------------------------------------- conv

def _conv_chain(orc, w, b, win0, xs):
    win = win0.copy()
    ys, wins = [], []
    for x in xs:
        y, win = orc.conv_token(w, b, win, x)
        ys.append(y)
        wins.append(win.copy())
    return np.stack(ys, 1), wins


@pin
def check_conv_matches_torch_conv1d(orc):
    """L chained conv tokens == depthwise torch conv1d over [window | x_0..x_L-1] + SiLU."""
    rng = np.random.default_rng(5)
    for W in (4, 3, 2):
        C, L = 7, 6
        w = rng.standard_normal((C, W))
        b = rng.standard_normal(C)
        win0 = rng.standard_normal((C, W - 1))
        xs = rng.standard_normal((L, C))
        ys, wins = _conv_chain(orc, w, b, win0, xs)
        seq = np.concatenate([win0, xs.T], 1)                       # [C, W-1+L]
        ref = torch.nn.functional.conv1d(torch.from_numpy(seq)[None], torch.from_numpy(w)[:, None],
                                         torch.from_numpy(b), groups=C)[0]
        _close(ys, torch.nn.functional.silu(ref).numpy(), 1e-12, 1e-14, f"conv W={W}")
        for t in range(L):
            assert np.array_equal(wins[t], seq[:, t + 1: t + W]), "window after token"


@pin
def check_conv_delta_kernel_is_shift(orc):
    """A one-hot tap j with no bias is a pure shift: y_t = silu(input W-1-j steps back)."""
    rng = np.random.default_rng(6)
    W, C, L = 4, 8, 5
    w = np.zeros((C, W))
    for c in range(C):
        w[c, c % W] = 1.0
    win0 = rng.standard_normal((C, W - 1))
    xs = rng.standard_normal((L, C))
    ys, _ = _conv_chain(orc, w, None, win0, xs)
    seq = np.concatenate([win0, xs.T], 1)
    for c in range(C):
        j = c % W
        exp = seq[c, np.arange(L) + j]          # input (W-1-j) steps before token t
        _close(ys[c], exp * scipy.special.expit(exp), 1e-15, 1e-300, "delta kernel")


# ----------------------------------------------------------------- gate / beta

@pin
def check_gate_projection_and_limits(orc):
    rng = np.random.default_rng(7)
    H = 3
    D = H * 128
    f_b = rng.standard_normal((D, 128)) * 0.09
    f_a = rng.standard_normal(128)
    A_log = rng.uniform(-1, 1, H)
    g1 = f_b @ f_a                                    # numpy float64 matmul
    lb = -5.0
    # dt_bias cancelling the projection: sigmoid(0) = 1/2, so g = lb/2 exactly up to rounding
    _close(orc.gate(f_b, f_a, A_log, -g1, lb), np.full(D, lb / 2), 0, 1e-12, "g at g1+dt=0")
    delta = rng.uniform(-2, 2, D)
    g = orc.gate(f_b, f_a, A_log, -g1 + delta, lb)
    a = np.exp(np.repeat(A_log, 128))                 # one A_log per head of 128
    _close(g / lb, scipy.special.expit(a * delta), 1e-10, 1e-12, "g / lb")
    assert np.all(orc.gate(f_b, f_a, A_log, rng.uniform(-1, 1, D), 0.0) == 0.0)
    g = orc.gate(f_b, f_a, A_log, rng.uniform(-1, 1, D), lb)
    assert np.all((g <= 0.0) & (g >= lb))


# ----------------------------------------------------------------- l2norm

@pin
def check_l2norm(orc):
    rng = np.random.default_rng(8)
    x = rng.standard_normal(128) * 3
    _close(orc.l2norm(x, 0.0), x / np.linalg.norm(x), 1e-14, 0, "l2norm eps=0")
    eps = 1e-6
    for scale in (1.0, 128 ** -0.5):
        y = orc.l2norm(x, eps, scale)
        ss = float(np.dot(x, x))
        _close(np.dot(y, y), scale * scale * ss / (ss + eps), 1e-13, 0, "norm^2")
        cos = np.dot(y, x) / (np.linalg.norm(y) * np.linalg.norm(x))
        _close(cos, 1.0, 1e-14, 0, "direction")
    _close(orc.l2norm(7.5 * x, 0.0), orc.l2norm(x, 0.0), 1e-14, 0, "scale invariance")
    assert np.all(orc.l2norm(np.zeros(128), eps) == 0.0)


# ----------------------------------------------------------------- recurrence

def _rand_unit(rng, n):
    v = rng.standard_normal(n)
    return v / np.linalg.norm(v)


@pin
def check_recur_identity_at_beta0_g0(orc):
    rng = np.random.default_rng(9)
    S = rng.standard_normal((128, 128)) * 0.05
    k, q, v = _rand_unit(rng, 128), rng.standard_normal(128) * 0.1, rng.standard_normal(128)
    S1, o = orc.recur_token(S, np.zeros(128), k, q, v, 0.0)
    assert np.array_equal(S1, S)
    _close(o, S @ q, 1e-12, 1e-15, "o = S q")


@pin
def check_recur_zero_state_closed_form(orc):
    """From a zero state, one token: S = beta v k^T ([v][k] storage), o = beta (k.q) v."""
    rng = np.random.default_rng(10)
    g = -rng.uniform(0, 5, 128)
    k, q, v = _rand_unit(rng, 128), rng.standard_normal(128) * 0.1, rng.standard_normal(128)
    beta = 0.37
    S1, o = orc.recur_token(np.zeros((128, 128)), g, k, q, v, beta)
    _close(S1, beta * np.outer(v, k), 1e-14, 1e-300, "S1")
    _close(o, beta * np.dot(k, q) * v, 1e-12, 1e-300, "o")


@pin
def check_recur_decay_only(orc):
    """beta = 0: S1[j][i] = S0[j][i] exp(g_i) (column-wise over the key channel)."""
    rng = np.random.default_rng(12)
    S = rng.standard_normal((128, 128)) * 0.05
    g = -rng.uniform(0, 5, 128)
    k, q, v = _rand_unit(rng, 128), rng.standard_normal(128), rng.standard_normal(128)
    S1, o = orc.recur_token(S, g, k, q, v, 0.0)
    _close(S1, S * np.exp(g)[None, :], 1e-15, 1e-300, "decayed state")
    _close(o, S1 @ q, 1e-12, 1e-15, "o")


@pin
def check_recur_delta_rule_retrieval(orc):
    """beta = 1, g = 0, unit k: the updated state maps k to v exactly (S1 k = v)."""
    rng = np.random.default_rng(13)
    S = rng.standard_normal((128, 128)) * 0.05
    k, q, v = _rand_unit(rng, 128), rng.standard_normal(128), rng.standard_normal(128)
    S1, _ = orc.recur_token(S, np.zeros(128), k, q, v, 1.0)
    _close(S1 @ k, v, 1e-12, 1e-13, "retrieval")


@pin
def check_recur_dense_matrix_bruteforce(orc):
    """Tiny dims, several tokens: M_t = (I - b k k^T) diag(e^g) M_{t-1} + b k v^T,
    o_t = M_t^T q with M = S^T, by numpy matmuls."""
    rng = np.random.default_rng(14)
    for dk, dv in ((5, 3), (4, 6), (1, 2)):
        S = rng.standard_normal((dv, dk))
        M = S.T.copy()
        for _ in range(4):
            g = -rng.uniform(0, 2, dk)
            k, q, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
            beta = rng.uniform(0, 1)
            M = (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(np.exp(g)) @ M + beta * np.outer(k, v)
            S, o = orc.recur_token(S, g, k, q, v, beta)
            _close(S, M.T, 1e-12, 1e-13, f"state {dk}x{dv}")
            _close(o, M.T @ q, 1e-12, 1e-13, f"o {dk}x{dv}")


# ----------------------------------------------------------------- gated RMSNorm

@pin
def check_gated_rmsnorm(orc):
    rng = np.random.default_rng(15)
    o = rng.standard_normal(128) * 0.3
    gate = rng.standard_normal(128)
    w = rng.uniform(0.5, 1.5, 128)
    eps = 1e-6
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (128,), torch.from_numpy(w), eps)
    _close(orc.gated_rmsnorm(o, gate, w, eps), ref.numpy() * scipy.special.expit(gate), 1e-12,
           1e-15, "vs torch rms_norm")
    y = orc.gated_rmsnorm(o, np.full(128, np.inf), np.ones(128), eps)
    m = float(np.mean(o * o))
    _close(np.mean(y * y), m / (m + eps), 1e-13, 0, "output mean square")
    _close(orc.gated_rmsnorm(4.0 * o, gate, w, 0.0), orc.gated_rmsnorm(o, gate, w, 0.0), 1e-14,
           1e-300, "scale invariance")


# ----------------------------------------------------------------- whole call

def _small_verify(seed=21, **kw):
    return make_case(R=3, L=3, H=2, num_slots=16, seed=seed, verify=True, **kw)


def _src_dst(case):
    s = case.slots.numpy()
    acc = case.accepted.numpy() if case.accepted is not None else np.ones(case.R, np.int32)
    if s.ndim == 1:
        s = s[:, None]
    return [int(s[r, acc[r] - 1]) for r in range(case.R)], [list(map(int, s[r])) for r in range(case.R)]


@pin
def check_call_identity_mode_selects_accepted_state(orc):
    """lb = 0 (g = 0) and beta_raw = -inf (beta = 0): every written state equals the
    accepted source state bit for bit, so the selection slots[r][accepted[r]-1] shows."""
    case = _small_verify(22)
    D = case.D
    proj = case.projected.clone()
    proj[:, 4 * D + 128: 4 * D + 128 + case.H] = float("-inf")
    res = run_oracle(case, orc, projected=proj, gate_lower_bound=0.0)
    before = case.state.numpy()
    src, dst = _src_dst(case)
    assert res["skipped"] == 0
    for r in range(case.R):
        for t in range(case.L):
            assert np.array_equal(res["state"][dst[r][t]], before[src[r]]), (r, t)


@pin
def check_call_decay_closed_form(orc):
    """beta_raw = -inf (beta = 0) and dt_bias = -(f_b f_a) by numpy for a shared f_a
    row: the gate's sigmoid sees 0, so g = lb/2 on every channel and every written
    state is the source state times e^(lb/2) once per token (fp32 after each)."""
    case = _small_verify(30)
    D, H = case.D, case.H
    proj = case.projected.clone()
    proj[:, 4 * D + 128: 4 * D + 128 + H] = float("-inf")
    proj[:, 4 * D: 4 * D + 128] = proj[0, 4 * D: 4 * D + 128]      # one f_a for all rows
    f_a = om.bf16_bits_to_f64(bf16_np(proj[0, 4 * D: 4 * D + 128]))
    f_b = om.bf16_bits_to_f64(bf16_np(case.f_b))
    dt = (-(f_b @ f_a)).astype(np.float32)
    res = run_oracle(case, orc, projected=proj, dt_bias=dt)
    # dt is fp32-rounded, so the sigmoid sees |g1 + dt| <= ~1e-7 rather than 0
    decay = np.exp(case.gate_lower_bound / 2)
    src, dst = _src_dst(case)
    before = case.state.numpy().astype(np.float64)
    for r in range(case.R):
        s = before[src[r]]
        for t in range(case.L):
            s = s * decay
            _close(res["state"][dst[r][t]], s, 1e-5, 1e-30, f"decayed state {r},{t}")


@pin
def check_call_conv_window_closed_form(orc):
    """conv[dst[t]] holds the last W-1 inputs of [window(src) | x_0 .. x_t], exactly."""
    for dim_first in (True, False):
        case = _small_verify(23, conv_dim_first=dim_first)
        res = run_oracle(case, orc)
        before = bf16_np(case.conv_view())                 # [slots, 3D, W-1]
        after = res["conv"] if dim_first else res["conv"].transpose(0, 2, 1)
        proj = bf16_np(case.projected)
        src, dst = _src_dst(case)
        C = 3 * case.D
        for r in range(case.R):
            seq = np.concatenate([before[src[r]], proj[r * case.L:(r + 1) * case.L, :C].T], 1)
            for t in range(case.L):
                assert np.array_equal(after[dst[r][t]], seq[:, t + 1: t + case.W]), (r, t)


@pin
def check_call_verify_equals_chained_decodes(orc):
    """verify over L tokens == L decode calls chained on one slot, bit for bit
    (core_out rows and every per-token state and conv window), in the fused and
    in the bf16 hand-off mode."""
    for hand in (False, True):
        case = _small_verify(24)
        res = run_oracle(case, orc, handoff_bf16=hand)
        src, dst = _src_dst(case)
        D = case.D
        for r in range(case.R):
            conv = bf16_np(case.conv_storage).copy()
            state = case.state.numpy().copy()
            tmp = dst[r][0]  # chain in place on one slot, seeded with the source
            conv[tmp] = conv[src[r]]
            state[tmp] = state[src[r]]
            for t in range(case.L):
                row = r * case.L + t
                out = np.zeros((1, D), np.uint16)
                orc.run(heads=case.H, width=case.W, requests=1, tokens=1,
                        projected=bf16_np(case.projected[row:row + 1]), pitch=case.pitch,
                        slots=np.array([tmp], np.int32), slots_row_stride=1, accepted=None,
                        num_slots=case.num_slots, conv=conv.reshape(-1),
                        conv_strides=case.conv_strides(), state=state.reshape(-1),
                        state_slot_stride=case.H * 128 * 128,
                        conv_weight=bf16_np(case.conv_weight),
                        conv_bias=bf16_np(case.conv_bias), f_b=bf16_np(case.f_b),
                        A_log=case.A_log.numpy(), dt_bias=case.dt_bias.numpy(),
                        norm_weight=case.norm_weight.numpy(), norm_head_stride=0,
                        gate_lower_bound=case.gate_lower_bound, norm_eps=case.norm_eps,
                        l2_eps=case.l2_eps, core_out=out, handoff_bf16=hand)
                assert np.array_equal(out[0], res["out"][row]), (hand, r, t)
                assert np.array_equal(state[tmp], res["state"][dst[r][t]]), (hand, r, t)
                assert np.array_equal(conv[tmp], res["conv"][dst[r][t]]), (hand, r, t)


@pin
def check_call_decode_equals_verify_single_token(orc):
    dec = make_case(R=4, L=1, H=2, num_slots=8, seed=25, verify=False)
    a = run_oracle(dec, orc)
    b = run_oracle(dec, orc, accepted=np.ones(4, np.int32))
    for key in ("out", "conv", "state"):
        assert np.array_equal(a[key], b[key]), key


@pin
def check_call_zero_state_closed_form(orc):
    """Zero carried state, one token: the written state is beta v k^T and, because
    o = beta (k.q) v = c v is a multiple of v, core_out = c v / sqrt(c^2 mean(v^2) +
    eps) * w * sigmoid(gate). q, k, v come from torch conv1d + SiLU."""
    case = make_case(R=2, L=1, H=2, num_slots=4, seed=26, verify=False)
    zero = torch.zeros_like(case.state)
    res = run_oracle(case, orc, state=zero)
    D, W = case.D, case.W
    conv0 = bf16_np(case.conv_view())
    w = om.bf16_bits_to_f64(bf16_np(case.conv_weight))             # [3D, 1, W]
    b = om.bf16_bits_to_f64(bf16_np(case.conv_bias))
    for r in range(case.R):
        slot = int(case.slots[r])
        x = om.bf16_bits_to_f64(bf16_np(case.projected[r]))
        seq = np.concatenate([om.bf16_bits_to_f64(conv0[slot]), x[:3 * D, None]], 1)
        y = torch.nn.functional.silu(torch.nn.functional.conv1d(
            torch.from_numpy(seq)[None], torch.from_numpy(w), torch.from_numpy(b),
            groups=3 * D))[0, :, 0].numpy()
        for h in range(case.H):
            q, k, v = (y[s * D + 128 * h: s * D + 128 * (h + 1)] for s in range(3))
            kh = k / np.sqrt(np.dot(k, k) + case.l2_eps)
            qh = q / np.sqrt(np.dot(q, q) + case.l2_eps) * 128 ** -0.5
            beta = scipy.special.expit(x[4 * D + 128 + h])
            _close(res["state"][slot, h], np.float32(beta * np.outer(v, kh)), 2e-7, 1e-30,
                   "state")
            gate = x[3 * D + 128 * h: 3 * D + 128 * (h + 1)]
            c = beta * np.dot(kh, qh)                 # o = c v
            exp = c * v / np.sqrt(c * c * np.mean(v * v) + case.norm_eps) \
                * case.norm_weight.numpy() * scipy.special.expit(gate)
            _close(res["out_f64"][r, 128 * h: 128 * (h + 1)], exp, 1e-9, 1e-12, "core_out")


@pin
def check_call_skips_invalid_requests(orc):
    """Out-of-range slots or accepted counts skip the request: no reads, no writes,
    its out rows untouched; the other requests are as if run alone."""
    case = _small_verify(27)
    s = case.slots.clone()
    acc = case.accepted.clone()
    s[1, 2] = case.num_slots          # out of range
    acc[2] = 0                        # not in 1..L
    bad = make_case(R=3, L=3, H=2, num_slots=16, seed=27, verify=True)
    bad.slots, bad.accepted = s, acc
    res = run_oracle(bad, orc)
    assert res["skipped"] == 2
    D, L = case.D, case.L
    assert np.all(res["out"][L:] == 0)
    alone = dataclasses.replace(case, R=1, projected=case.projected[:L].clone(),
                                slots=s[:1].clone(), accepted=acc[:1].clone())
    ref = run_oracle(alone, orc)
    assert np.array_equal(res["out"][:L], ref["out"])
    assert np.array_equal(res["state"], ref["state"])
    assert np.array_equal(res["conv"], ref["conv"])
    written = set(int(x) for x in s[0])
    before = case.state.numpy()
    for slot in range(case.num_slots):
        if slot not in written:
            assert np.array_equal(res["state"][slot], before[slot]), slot


@pin
def check_call_duplicate_destinations(orc):
    """A slot named twice as a destination in one call -- by two requests, or by two
    tokens of one request -- makes the call undefined: the oracle rejects it and
    writes nothing. With check_distinct every request involved is skipped and
    counted, and the others are as if run alone."""
    base = make_case(R=4, L=3, H=2, num_slots=24, seed=34, verify=True)
    for kind in ("across", "within"):
        s = base.slots.clone()
        if kind == "across":
            s[2, 1] = s[0, 2]          # requests 0 and 2 share a destination
            involved = {0, 2}
        else:
            s[1, 2] = s[1, 0]          # request 1 names one slot for tokens 0 and 2
            involved = {1}
        case = dataclasses.replace(base, slots=s)
        conv = bf16_np(case.conv_storage)
        state = case.state.numpy().copy()
        out = np.zeros((case.S, case.D), np.uint16)
        try:
            run_oracle(case, orc)
        except ValueError:
            pass
        else:
            raise AssertionError(f"duplicate destinations ({kind}) accepted")
        # nothing written on rejection: run in place on explicit arrays
        kw = dict(heads=case.H, width=case.W, requests=case.R, tokens=case.L,
                  projected=bf16_np(case.projected), pitch=case.pitch,
                  slots=s.contiguous().numpy(), slots_row_stride=case.L,
                  accepted=case.accepted.numpy(), num_slots=case.num_slots,
                  conv=conv.reshape(-1), conv_strides=case.conv_strides(),
                  state=state.reshape(-1), state_slot_stride=case.H * 128 * 128,
                  conv_weight=bf16_np(case.conv_weight), conv_bias=bf16_np(case.conv_bias),
                  f_b=bf16_np(case.f_b), A_log=case.A_log.numpy(),
                  dt_bias=case.dt_bias.numpy(), norm_weight=case.norm_weight.numpy(),
                  norm_head_stride=0, gate_lower_bound=case.gate_lower_bound,
                  norm_eps=case.norm_eps, l2_eps=case.l2_eps, core_out=out)
        try:
            orc.run(**kw)
        except ValueError:
            pass
        assert np.array_equal(conv, bf16_np(case.conv_storage)) and \
            np.array_equal(state, case.state.numpy()) and not out.any(), kind
        res = run_oracle(case, orc, check_distinct=True)
        assert res["skipped"] == len(involved), (kind, res["skipped"])
        keep = [r for r in range(case.R) if r not in involved]
        for r in involved:
            assert not res["out"][r * case.L:(r + 1) * case.L].any(), (kind, r)
        alone = dataclasses.replace(
            case, R=len(keep),
            projected=torch.cat([case.projected[r * case.L:(r + 1) * case.L] for r in keep]),
            slots=s[keep].clone(), accepted=case.accepted[keep].clone())
        ref = run_oracle(alone, orc)
        for i, r in enumerate(keep):
            assert np.array_equal(res["out"][r * case.L:(r + 1) * case.L],
                                  ref["out"][i * case.L:(i + 1) * case.L]), (kind, r)
        assert np.array_equal(res["state"], ref["state"]), kind
        assert np.array_equal(res["conv"], ref["conv"]), kind


@pin
def check_call_layout_and_option_equivalences(orc):
    """Both conv layouts, no bias vs zero bias, and a per-head norm weight equal to
    the shared one give identical results."""
    a = _small_verify(28, conv_dim_first=True)
    b = _small_verify(28, conv_dim_first=True)
    b.conv_dim_first = False
    b.conv_storage = a.conv_storage.transpose(1, 2).contiguous()
    ra, rb = run_oracle(a, orc), run_oracle(b, orc)
    assert np.array_equal(ra["out"], rb["out"]) and np.array_equal(ra["state"], rb["state"])
    assert np.array_equal(ra["conv"], rb["conv"].transpose(0, 2, 1))
    nb = _small_verify(28, with_bias=False)
    zb = _small_verify(28)
    zb.conv_bias = torch.zeros_like(zb.conv_bias)
    rn, rz = run_oracle(nb, orc), run_oracle(zb, orc)
    assert np.array_equal(rn["out"], rz["out"]) and np.array_equal(rn["state"], rz["state"])
    tiled = np.tile(a.norm_weight.numpy(), a.H)
    rt = run_oracle(a, orc, norm_weight=tiled, norm_head_stride=128)
    assert np.array_equal(ra["out"], rt["out"])


@pin
def check_call_state_stays_bounded(orc):
    """With beta in [0, 1], unit-norm k and e^g <= 1, I - beta k k^T has eigenvalues in
    [0, 1]: repeated decode steps at the decay extremes keep the state bounded."""
    case = make_case(R=2, L=1, H=2, num_slots=4, seed=29, verify=False, beta_std=2.0,
                     a_log_range=(-3.0, 2.0))
    state = case.state.clone()
    conv = case.conv_storage.clone()
    vmax = 0.0
    for step in range(12):
        res = run_oracle(case, orc, state=state, conv_storage=conv)
        state = torch.from_numpy(res["state"])
        conv = torch.from_numpy(res["conv"]).view(torch.int16).view(torch.bfloat16)
        vmax = max(vmax, float(np.abs(res["state"]).max()))
        assert np.all(np.isfinite(res["out_f64"]))
    assert vmax < 50.0, vmax


# ----------------------------------------------------------------- projections

def _bf16_bits(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pin
def check_linear_against_numpy_and_closed_forms(orc):
    """y = x W^T: numpy float64 matmul on the widened inputs; an identity block
    copies columns exactly; one-hot rows of x pick columns of W exactly; the
    entry-wise form equals the full one; x rows may be padded (pitch > K)."""
    rng = np.random.default_rng(31)
    M, N, K, pitch = 5, 9, 48, 56
    x = _bf16_bits(rng, (M, pitch))
    w = _bf16_bits(rng, (N, K), 0.2)
    y, y64 = orc.linear(x, w, x_pitch=pitch)
    ref = om.bf16_bits_to_f64(x[:, :K]) @ om.bf16_bits_to_f64(w).T
    _close(y64, ref, 1e-12, 1e-14, "linear vs numpy")
    assert np.array_equal(y, orc.f64_to_bf16_bits(y64)), "bf16 output is the RNE of the sum"
    eye = np.zeros((N, K), np.uint16)
    eye[np.arange(N), np.arange(N)] = 0x3F80                  # 1.0 in bf16
    y_eye, _ = orc.linear(x, eye, x_pitch=pitch)
    assert np.array_equal(y_eye, x[:, :N])
    onehot = np.zeros((K, K), np.uint16)
    onehot[np.arange(K), np.arange(K)] = 0x3F80
    y_oh, _ = orc.linear(onehot, w)
    assert np.array_equal(y_oh, w.T)
    ms, ns = rng.integers(0, M, 20), rng.integers(0, N, 20)
    _close(orc.linear_entries(x, w, ms, ns, x_pitch=pitch), y64[ms, ns], 0, 0, "entries")


# ----------------------------------------------------------------- bf16 hand-off mode

def _bf16_rne(x):
    """Round float64 values to bf16 (8 significant bits, ties to even), in numpy."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(np.abs(x))
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.copysign(np.round(np.abs(x) / q) * q, x)


def _near_ties(x, m):
    return int(np.count_nonzero(_bf16_rne(x - m) != _bf16_rne(x + m)))


def _conv_outputs(case, conv_slot, x):
    """SiLU(conv) of one token via torch conv1d, and the near-tie magnitude per channel:
    |SiLU'(pre)| (|bias| + sum |w * input|) + (1 + |pre|) |SiLU(pre)|."""
    D = case.D
    conv0 = om.bf16_bits_to_f64(bf16_np(case.conv_view()))[conv_slot]
    w = om.bf16_bits_to_f64(bf16_np(case.conv_weight))                   # [3D, 1, W]
    b = om.bf16_bits_to_f64(bf16_np(case.conv_bias))
    seq = np.concatenate([conv0, x[:3 * D, None]], 1)                   # [3D, W]
    y = torch.nn.functional.silu(torch.nn.functional.conv1d(
        torch.from_numpy(seq)[None], torch.from_numpy(w), torch.from_numpy(b),
        groups=3 * D))[0, :, 0].numpy()
    mag = np.abs(b) + np.abs(w[:, 0, :] * seq).sum(1)
    pre = torch.nn.functional.conv1d(torch.from_numpy(seq)[None], torch.from_numpy(w),
                                     torch.from_numpy(b), groups=3 * D)[0, :, 0].numpy()
    sg = scipy.special.expit(pre)
    slope = sg * (1.0 + pre * (1.0 - sg))
    return y, np.abs(slope) * mag + (1.0 + np.abs(pre)) * np.abs(y)


@pin
def check_handoff_zero_state_closed_form(orc):
    """Hand-off mode, zero carried state, one token: q, k, v are the bf16-rounded
    SiLU(conv) outputs, the written state is beta v_r k_r^T (normalised k_r), o =
    beta (k.q) v_r is rounded to bf16 before the gated RMSNorm; and the near-tie
    counts of conv out, o and core_out equal brute-force counts over the same values."""
    case = make_case(R=2, L=1, H=2, num_slots=4, seed=26, verify=False)
    mu = 2.0 ** -10
    ties = np.zeros((case.R, case.H, 4), np.int32)
    res = run_oracle(case, orc, state=torch.zeros_like(case.state), handoff_bf16=True,
                     ties=ties, tie_margins=(mu, 0.0, mu, mu))
    D = case.D
    for r in range(case.R):
        slot = int(case.slots[r])
        x = om.bf16_bits_to_f64(bf16_np(case.projected[r]))
        y, mag = _conv_outputs(case, slot, x)
        yr = _bf16_rne(y)
        for h in range(case.H):
            seg = [slice(s * D + 128 * h, s * D + 128 * (h + 1)) for s in range(3)]
            conv_ties = sum(_near_ties(y[sl], mu * mag[sl]) for sl in seg)
            q, k, v = (yr[sl] for sl in seg)
            kh = k / np.sqrt(np.dot(k, k) + case.l2_eps)
            qh = q / np.sqrt(np.dot(q, q) + case.l2_eps) * 128 ** -0.5
            beta = scipy.special.expit(x[4 * D + 128 + h])
            _close(res["state"][slot, h], np.float32(beta * np.outer(v, kh)), 2e-7, 1e-30,
                   "hand-off state")
            o = beta * np.dot(kh, qh) * v
            o_ties = _near_ties(o, mu * abs(beta) * np.abs(v) * np.abs(kh * qh).sum())
            orr = _bf16_rne(o)
            gate = x[3 * D + 128 * h: 3 * D + 128 * (h + 1)]
            exp = orr / np.sqrt(np.mean(orr * orr) + case.norm_eps) \
                * case.norm_weight.numpy() * scipy.special.expit(gate)
            _close(res["out_f64"][r, 128 * h: 128 * (h + 1)], exp, 1e-9, 1e-12, "hand-off core_out")
            y_ties = _near_ties(exp, mu * np.abs(exp))
            assert tuple(ties[r, h]) == (conv_ties, 0, o_ties, y_ties), (r, h, ties[r, h],
                                                                          (conv_ties, o_ties, y_ties))
    assert ties[:, :, 0].sum() > 0 and ties[:, :, 2].sum() > 0 and ties[:, :, 3].sum() > 0


@pin
def check_handoff_g1_rounding_closed_form(orc):
    """Hand-off mode with beta = 0: the written state is the carried state decayed by
    e^g per key column, g = lb sigmoid(e^A_log (bf16(f_b f_a) + dt_bias)), with g1
    from numpy in float64 and rounded to bf16; the fused mode decays by the unrounded
    g1 instead."""
    case = make_case(R=2, L=1, H=2, num_slots=4, seed=31, verify=False)
    D = case.D
    proj = case.projected.clone()
    proj[:, 4 * D + 128: 4 * D + 128 + case.H] = float("-inf")
    f_b = om.bf16_bits_to_f64(bf16_np(case.f_b))
    before = case.state.numpy().astype(np.float64)
    for hand in (True, False):
        res = run_oracle(case, orc, projected=proj, handoff_bf16=hand)
        for r in range(case.R):
            slot = int(case.slots[r])
            f_a = om.bf16_bits_to_f64(bf16_np(proj[r, 4 * D: 4 * D + 128]))
            g1 = f_b @ f_a
            if hand:
                g1 = _bf16_rne(g1)
            a = np.repeat(np.exp(case.A_log.numpy().astype(np.float64)), 128)
            g = case.gate_lower_bound * scipy.special.expit(a * (g1 + case.dt_bias.numpy()))
            exp = before[slot] * np.exp(g).reshape(case.H, 1, 128)
            _close(res["state"][slot], exp, 2e-7, 1e-30, f"decay, hand-off={hand}")


@pin
def check_handoff_g1_tie_certificate(orc):
    """g1 near ties: with coarse gate operands every fp32 sum is exact, so no g1
    value is a near tie even at a margin factor of 1 (while conv outputs are); with
    ordinary operands the count equals a brute-force count at factor 2^-10."""
    case = make_case(R=2, L=1, H=2, num_slots=4, seed=32, verify=False, coarse_gate=True)
    ties = np.zeros((case.R, case.H, 4), np.int32)
    run_oracle(case, orc, handoff_bf16=True, ties=ties, tie_margins=(1.0, 1.0, 0.0, 0.0))
    assert ties[:, :, 1].sum() == 0 and ties[:, :, 0].sum() > 0, ties

    case = make_case(R=2, L=1, H=2, num_slots=4, seed=33, verify=False)
    mu = 2.0 ** -10
    ties = np.zeros((case.R, case.H, 4), np.int32)
    run_oracle(case, orc, handoff_bf16=True, ties=ties, tie_margins=(0.0, mu, 0.0, 0.0))
    f_b = om.bf16_bits_to_f64(bf16_np(case.f_b))
    D = case.D
    for r in range(case.R):
        f_a = om.bf16_bits_to_f64(bf16_np(case.projected[r, 4 * D: 4 * D + 128]))
        g1 = f_b @ f_a
        mag = np.abs(f_b * f_a[None, :]).sum(1)
        for h in range(case.H):
            sl = slice(128 * h, 128 * (h + 1))
            assert ties[r, h, 1] == _near_ties(g1[sl], mu * mag[sl]), (r, h)
    assert ties[:, :, 1].sum() > 0


@pin
def check_handoff_ties_replay_matches_run(orc):
    """The near-tie counter replays the call on its own copies: its core_out values
    must be the run's. Over a three-token verify, the core_out near ties it counts
    per (request, head) equal a brute-force count over the run's unrounded core_out
    at the same margin (2^-12 relative: about one value in eight counts), so a
    replay that drifted from the run by more than a small fraction of that margin
    in any step or token would disagree (an fp32-level drift, ~1e-8, would not)."""
    case = _small_verify(35)
    mu = 2.0 ** -12
    ties = np.zeros((case.R, case.H, 4), np.int32)
    res = run_oracle(case, orc, handoff_bf16=True, ties=ties, tie_margins=(0.0, 0.0, 0.0, mu))
    y = res["out_f64"]
    total = 0
    for r in range(case.R):
        rows = y[r * case.L:(r + 1) * case.L]
        for h in range(case.H):
            v = rows[:, 128 * h: 128 * (h + 1)]
            n = _near_ties(v, mu * np.abs(v))
            assert ties[r, h, 3] == n, (r, h, ties[r, h, 3], n)
            total += n
    assert total > 0.05 * y.size, total
