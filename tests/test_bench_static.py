"""bench.py runs on the GPU only, so its functions are checked statically here:
every name a function reads is assigned in it, a module-level name or a builtin."""
import ast
import builtins
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _undefined_names(path):
    tree = ast.parse(open(path).read())
    module = set(dir(builtins))
    for node in tree.body:
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            module.add(node.name)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            module.update((a.asname or a.name).split(".")[0] for a in node.names)
        elif isinstance(node, (ast.Assign, ast.AnnAssign)):
            for t in node.targets if isinstance(node, ast.Assign) else [node.target]:
                module.update(x.id for x in ast.walk(t) if isinstance(x, ast.Name))
    problems = {}
    for fn in (n for n in tree.body if isinstance(n, ast.FunctionDef)):
        bound = set()
        for x in ast.walk(fn):
            if isinstance(x, ast.arg):
                bound.add(x.arg)
            elif isinstance(x, ast.Name) and isinstance(x.ctx, (ast.Store, ast.Del)):
                bound.add(x.id)
            elif isinstance(x, ast.FunctionDef):
                bound.add(x.name)
            elif isinstance(x, (ast.Import, ast.ImportFrom)):
                bound.update((a.asname or a.name).split(".")[0] for a in x.names)
            elif isinstance(x, ast.ExceptHandler) and x.name:
                bound.add(x.name)
        used = {x.id for x in ast.walk(fn) if isinstance(x, ast.Name) and isinstance(x.ctx, ast.Load)}
        missing = used - bound - module
        if missing:
            problems[fn.name] = sorted(missing)
    return problems


def test_bench_has_no_undefined_names():
    assert _undefined_names(os.path.join(ROOT, "bench.py")) == {}
