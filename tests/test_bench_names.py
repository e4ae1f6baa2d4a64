"""Every name a function of bench.py reads is bound in that function (a parameter, an
assignment, a loop or comprehension variable, an import, a nested function or lambda
argument), at module level or among the builtins.  The non-default bench paths run only
on a GPU; this catches a name left undefined in one of them on the CPU."""
import ast
import builtins
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bound(node):
    names = set()
    for n in ast.walk(node):
        if isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.Lambda)):
            a = n.args
            for arg in a.posonlyargs + a.args + a.kwonlyargs:
                names.add(arg.arg)
            for arg in (a.vararg, a.kwarg):
                if arg is not None:
                    names.add(arg.arg)
            if not isinstance(n, ast.Lambda):
                names.add(n.name)
        elif isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
            names.add(n.id)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            for al in n.names:
                names.add((al.asname or al.name).split(".")[0])
        elif isinstance(n, ast.ExceptHandler) and n.name:
            names.add(n.name)
        elif isinstance(n, ast.ClassDef):
            names.add(n.name)
    return names


def test_bench_functions_read_only_bound_names():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    module_names = set(dir(builtins))
    for node in tree.body:
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            module_names.add(node.name)
        else:
            module_names |= _bound(node)
    missing = []
    for node in tree.body:
        if not isinstance(node, ast.FunctionDef):
            continue
        local = _bound(node)
        for n in ast.walk(node):
            if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load):
                if n.id not in local and n.id not in module_names:
                    missing.append(f"{node.name}: {n.id} (line {n.lineno})")
    assert not missing, "names read but never bound: " + ", ".join(missing)
