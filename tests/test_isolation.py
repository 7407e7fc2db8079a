"""Static checks of the oracle's isolation: the product package never imports
it, bench.py imports it only in its CPU-baseline leg and __graft_entry__ only
in smoke(); the oracle never imports the HIP package.  Also the bench's
refusal to run on more than one GPU (no GPU needed)."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(path):
    """(module name, enclosing function name or None) of every import."""
    tree = ast.parse(open(path).read(), path)
    out = []

    def visit(node, fn):
        for ch in ast.iter_child_nodes(node):
            f = ch.name if isinstance(ch, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(ch, ast.Import):
                out.extend((a.name, fn) for a in ch.names)
            elif isinstance(ch, ast.ImportFrom) and ch.module:
                out.append((ch.module, fn))
            visit(ch, f)
    visit(tree, None)
    return out


def _is_oracle(mod):
    return mod == "oracle" or mod.startswith("oracle.")


def test_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "cache_guided_sparse_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                for mod, _ in _imports(os.path.join(dirpath, f)):
                    assert not _is_oracle(mod), f"{f} imports {mod}"


def test_bench_and_entry_import_the_oracle_only_where_allowed():
    for f, allowed in (("bench.py", {"cpu_baseline"}), ("__graft_entry__.py", {"smoke"})):
        for mod, fn in _imports(os.path.join(ROOT, f)):
            if _is_oracle(mod):
                assert fn in allowed, f"{f}: oracle imported in {fn}"


def test_oracle_never_imports_the_hip_package():
    od = os.path.join(ROOT, "oracle")
    for f in os.listdir(od):
        if f.endswith(".py"):
            for mod, _ in _imports(os.path.join(od, f)):
                assert not mod.startswith("cache_guided_sparse_amd"), f"oracle/{f} imports {mod}"
                assert mod.split(".")[0] not in ("torch", "ctypes"), f"oracle/{f} imports {mod}"


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
