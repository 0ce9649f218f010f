"""A static check of the driver scripts that needs no GPU: inside each function of
bench.py, __graft_entry__.py and the binding, a local name is not read on a line
before the first line that assigns it (the GPU-only code paths of these files
never run in the CPU suite, so an UnboundLocalError there would otherwise show up
only on the GPU)."""
import ast
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = ["bench.py", "__graft_entry__.py", os.path.join("kimi_delta_attention_conv_amd", "__init__.py")]


def _first_lines(fn):
    """First line each name is stored / loaded in fn's own scope (nested functions,
    lambdas and comprehensions excluded; arguments count as stored at the def)."""
    stores, loads = {}, {}
    for a in fn.args.args + fn.args.kwonlyargs + fn.args.posonlyargs:
        stores[a.arg] = fn.lineno
    for a in (fn.args.vararg, fn.args.kwarg):
        if a is not None:
            stores[a.arg] = fn.lineno
    declared = set()

    def visit(node):
        for child in ast.iter_child_nodes(node):
            if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef, ast.Lambda, ast.ClassDef,
                                  ast.ListComp, ast.SetComp, ast.DictComp, ast.GeneratorExp)):
                if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
                    stores.setdefault(child.name, child.lineno)
                continue
            if isinstance(child, (ast.Global, ast.Nonlocal)):
                declared.update(child.names)
            if isinstance(child, ast.Name):
                table = stores if isinstance(child.ctx, (ast.Store, ast.Del)) else loads
                table[child.id] = min(table.get(child.id, child.lineno), child.lineno)
            if isinstance(child, (ast.Import, ast.ImportFrom)):
                for alias in child.names:
                    name = (alias.asname or alias.name).split(".")[0]
                    stores[name] = min(stores.get(name, child.lineno), child.lineno)
            if isinstance(child, ast.ExceptHandler) and child.name:
                stores[child.name] = min(stores.get(child.name, child.lineno), child.lineno)
            visit(child)

    visit(fn)
    return stores, loads, declared


@pytest.mark.parametrize("rel", FILES)
def test_no_local_read_before_assignment(rel):
    tree = ast.parse(open(os.path.join(ROOT, rel)).read())
    problems = []
    for node in ast.walk(tree):
        if not isinstance(node, (ast.FunctionDef, ast.AsyncFunctionDef)):
            continue
        stores, loads, declared = _first_lines(node)
        for name, line in loads.items():
            if name in stores and name not in declared and line < stores[name]:
                problems.append(f"{rel}:{line} {node.name}(): '{name}' read before its "
                                f"assignment on line {stores[name]}")
    assert not problems, "\n".join(problems)
