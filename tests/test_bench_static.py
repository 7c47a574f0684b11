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


def test_tile_probe_ids_read_no_tile_twice():
    """The tile-read probe's block ids: in range, whole rounds of head groups, and within each
    head group (item t reads group t mod heads / team) every block at most once -- so a launch
    reads each of its (block, head) tiles once and the caches cannot serve a repeat."""
    import numpy as np
    import bench

    rng = np.random.default_rng(0)
    for n_blocks, heads, team, n in ((1000, 8, 1, 6000), (1000, 8, 4, 1999), (300, 8, 2, 5000), (64, 6, 2, 100)):
        ids = bench.tile_probe_ids(rng, n_blocks, heads, team, n)
        groups = heads // team
        assert ids.dtype == np.int32 and ids.size % groups == 0
        assert ids.size == min(n // groups, n_blocks) * groups
        assert ids.min() >= 0 and ids.max() < n_blocks
        for g in range(groups):
            mine = ids[g::groups]
            assert np.unique(mine).size == mine.size, (n_blocks, heads, team, g)
        tiles = ids.astype(np.int64) * heads + (np.arange(ids.size) % groups) * team   # first head of each item
        assert np.unique(tiles).size == tiles.size
