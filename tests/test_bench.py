"""bench.py's host-side contract (no GPU needed): more than one GPU is
refused with a one-line JSON message and a non-zero exit, before anything
touches a device; and every name that bench.py's and __graft_entry__.py's
functions read is bound somewhere in scope (their GPU paths cannot run here,
so a misnamed variable would otherwise surface only on the GPU)."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    msg = json.loads(lines[0])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _names_bound(fn):
    """Every name a function (with its nested functions and lambdas) binds."""
    import ast
    names = set()
    for n in ast.walk(fn):
        if isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
            names.add(n.id)
        elif isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            names.add(n.name)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            names.update((a.asname or a.name).split(".")[0] for a in n.names)
        elif isinstance(n, ast.ExceptHandler) and n.name:
            names.add(n.name)
        elif isinstance(n, ast.arg):
            names.add(n.arg)
    return names


def _unbound_loads(path):
    """Names a function reads that neither it, its enclosing scopes, the module
    nor the builtins bind: the NameErrors that only a run on a GPU would show."""
    import ast
    import builtins
    tree = ast.parse(open(path).read())
    module = set(dir(builtins)) | {"__file__", "__name__"}
    for st in tree.body:
        if isinstance(st, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            module.add(st.name)
            continue
        for n in ast.walk(st):
            if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Store):
                module.add(n.id)
            elif isinstance(n, (ast.Import, ast.ImportFrom)):
                module.update((a.asname or a.name).split(".")[0] for a in n.names)
    bad = []
    for st in tree.body:
        if isinstance(st, (ast.FunctionDef, ast.AsyncFunctionDef)):
            ok = module | _names_bound(st)
            bad += [f"{st.name}: {n.id} (line {n.lineno})" for n in ast.walk(st)
                    if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load) and n.id not in ok]
    return bad


def test_bench_and_entry_names_resolve():
    for f in ("bench.py", "__graft_entry__.py"):
        assert _unbound_loads(os.path.join(ROOT, f)) == [], f


def test_cpu_baseline_leg_runs_on_host():
    """bench.py's cpu_baseline leg (the natively built scalar oracle, dense and
    sparse, one thread and all threads) on the tiny workload, host only."""
    sys.path.insert(0, ROOT)
    import bench
    from workloads import make_tiny
    r = bench.cpu_baseline(make_tiny(), 0.05)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["cores"] >= 1
    assert r["value"] > 0 and r["dense_tokens_per_s"] > 0
    assert r["one_thread"]["sparse_tokens_per_s"] > 0 and r["one_thread"]["dense_tokens_per_s"] > 0
    assert "-march=native" in r["build"] and "-ffp-contract=off" in r["build"]
    import oracle
    assert oracle.max_threads() >= 1  # the portable library is back in use
