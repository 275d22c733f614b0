"""CPU check of bench.py without a GPU: the module parses, and no top-level function reads a name
that neither it (parameters, assignments, nested definitions, imports) nor the module nor Python's
builtins define.  The GPU legs of the bench only run on the device; this catches a misplaced or
misspelt name before then."""
import ast
import builtins
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _module_names(tree):
    names = set()
    for node in tree.body:
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            names.add(node.name)
        elif isinstance(node, ast.Assign):
            for t in node.targets:
                for n in ast.walk(t):
                    if isinstance(n, ast.Name):
                        names.add(n.id)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            for a in node.names:
                names.add((a.asname or a.name).split(".")[0])
    return names


def _function_names(fn):
    defined, used = set(), set()
    for node in ast.walk(fn):
        if isinstance(node, ast.Name):
            (defined if isinstance(node.ctx, (ast.Store, ast.Del)) else used).add(node.id)
        elif isinstance(node, ast.arg):
            defined.add(node.arg)
        elif isinstance(node, ast.FunctionDef):
            defined.add(node.name)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            for a in node.names:
                defined.add((a.asname or a.name).split(".")[0])
        elif isinstance(node, ast.ExceptHandler) and node.name:
            defined.add(node.name)
    return defined, used


def test_bench_functions_read_only_defined_names():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    module = _module_names(tree) | set(dir(builtins))
    missing = {}
    for fn in tree.body:
        if isinstance(fn, ast.FunctionDef):
            defined, used = _function_names(fn)
            undefined = sorted(used - defined - module)
            if undefined:
                missing[fn.name] = undefined
    assert not missing, missing
