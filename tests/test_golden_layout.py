"""The oracle against the operand layout the prepared page prints
(tests/golden/prepared_operands.json): which columns of the packed projection
row feed which part of the method, and the q scale. Perturbing one column
inside a segment must change exactly the outputs that segment feeds, and
columns past the last segment (row padding) must change nothing."""
import ast
import json
import os

import numpy as np
import torch

import oracle as om
from kda_inputs import make_case
from oracle_cases import run_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prepared_operands.json")


def _arith(expr, env):
    """Value of an arithmetic expression over numbers and the names in env
    (+, -, *, ** only; anything else is rejected)."""
    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return n.value
        if isinstance(n, ast.Name) and n.id in env:
            return env[n.id]
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, ast.USub):
            return -ev(n.operand)
        if isinstance(n, ast.BinOp):
            ops = {ast.Add: lambda a, b: a + b, ast.Sub: lambda a, b: a - b,
                   ast.Mult: lambda a, b: a * b, ast.Pow: lambda a, b: a ** b}
            if type(n.op) in ops:
                return ops[type(n.op)](ev(n.left), ev(n.right))
        raise ValueError(f"unsupported expression: {expr!r}")
    return ev(ast.parse(expr, mode="eval"))


def _layout(H):
    g = json.load(open(GOLDEN))
    env = {"d": 128 * H, "h": H}
    return {k: (_arith(v["start"], env), _arith(v["width"], env))
            for k, v in g["projected_columns"].items()}, g


def _changed(a, b):
    return not np.array_equal(a, b)


def test_q_scale_is_the_printed_scalar():
    _, g = _layout(1)
    assert om.HEAD_DIM == g["head_dim"] == 128
    import inspect
    default = inspect.signature(om.Oracle.run).parameters["q_scale"].default
    assert default == _arith(g["q_scale"], {})


def test_segments_partition_the_row_and_feed_what_the_page_says():
    H = 2
    seg, _ = _layout(H)
    D = 128 * H
    order = sorted(seg.values())
    assert order[0][0] == 0
    for (s0, w0), (s1, _) in zip(order, order[1:]):
        assert s0 + w0 == s1, "segments must tile the row without gaps"
    end = order[-1][0] + order[-1][1]
    case = make_case(R=1, L=1, H=H, num_slots=2, seed=960, verify=False, pitch=end + 6)
    slot = int(case.slots[0])
    base = run_oracle(case)

    def perturbed(col):
        proj = case.projected.clone()
        proj[0, col] = proj[0, col].float() + 0.75
        return run_oracle(case, projected=proj)

    def heads(res):
        st = res["state"][slot]
        out = res["out"][0].reshape(H, 128)
        return [(st[h], out[h]) for h in range(H)]

    b = heads(base)
    # v of head 1 (third block of qkv): head 1's state and output only
    r = heads(perturbed(seg["qkv"][0] + 2 * D + 128 + 5))
    assert not _changed(r[0][0], b[0][0]) and not _changed(r[0][1], b[0][1])
    assert _changed(r[1][0], b[1][0]) and _changed(r[1][1], b[1][1])
    # output gate of head 1: head 1's core_out only, no state anywhere
    r = heads(perturbed(seg["gate"][0] + 128 + 7))
    assert not _changed(r[0][0], b[0][0]) and not _changed(r[1][0], b[1][0])
    assert not _changed(r[0][1], b[0][1]) and _changed(r[1][1], b[1][1])
    # f_a: the decay gate of every channel of every head
    r = heads(perturbed(seg["f_a"][0] + 3))
    assert _changed(r[0][0], b[0][0]) and _changed(r[1][0], b[1][0])
    # beta_raw of head 0: head 0 only
    r = heads(perturbed(seg["beta_raw"][0] + 0))
    assert _changed(r[0][0], b[0][0]) and not _changed(r[1][0], b[1][0])
    assert not _changed(r[1][1], b[1][1])
    # row padding past the last segment: nothing
    for col in range(end, end + 6):
        r = perturbed(col)
        assert not _changed(r["state"], base["state"]) and not _changed(r["out"], base["out"])
