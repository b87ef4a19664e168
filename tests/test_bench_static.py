"""bench.py has side workloads (prefill, key graph, host tier, per-layer
budgets) that only run on a GPU. A name left undefined in one of them
would only show there, so every module-level script is checked here for
loads of names that nothing binds (a static check; nothing is executed)."""

import ast
import builtins
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def unbound_names(path):
    tree = ast.parse(open(path).read(), path)
    bound = set(dir(builtins)) | {"__file__"}
    for n in ast.walk(tree):
        if isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            bound.add(n.name)
        elif isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
            bound.add(n.id)
        elif isinstance(n, ast.arg):
            bound.add(n.arg)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            for a in n.names:
                bound.add((a.asname or a.name).split(".")[0])
        elif isinstance(n, ast.ExceptHandler) and n.name:
            bound.add(n.name)
    return sorted({(n.id, n.lineno) for n in ast.walk(tree)
                   if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load) and n.id not in bound})


@pytest.mark.parametrize("rel", ["bench.py", "__graft_entry__.py",
                                 "top_sparse_attention_gqa_amd/_lib.py",
                                 "top_sparse_attention_gqa_amd/build.py",
                                 "synth/gen.py", "synth/configs.py", "oracle/ra_oracle.py"])
def test_no_unbound_names(rel):
    assert unbound_names(os.path.join(ROOT, rel)) == []


def test_more_than_one_gpu_is_refused_with_a_message():
    # one GPU per box: --gpus N > 1 (or a launcher's WORLD_SIZE > 1) exits
    # with status 2 and says why, before touching any device
    import subprocess
    import sys
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "8"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                           capture_output=True, text=True, timeout=120,
                           env=dict(os.environ, **env))
        assert r.returncode == 2, (args, r.returncode, r.stderr[-500:])
        assert "one GPU" in r.stderr
