"""CPU checks of the package's contracts: the binding has no fallback path,
bench.py refuses more than one GPU, and the oracle stays out of the product
path."""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bf16_attention_forward_amd")


def test_missing_library_raises_instead_of_falling_back(tmp_path):
    from bf16_attention_forward_amd import binding
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.load_library(str(tmp_path / "libattn_fwd.so"))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_product_code_never_imports_the_oracle():
    """Only tests, smoke() and bench.py's CPU baseline may use the oracle: no
    module of the package imports it."""
    for name in os.listdir(PKG):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            else:
                continue
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)


def test_bench_uses_the_oracle_only_for_the_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    users = set()
    for fn in [n for n in ast.walk(tree) if isinstance(n, ast.FunctionDef)]:
        for node in ast.walk(fn):
            if isinstance(node, (ast.Import, ast.ImportFrom)):
                mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                if any(m == "oracle" or m.startswith("oracle.") for m in mods):
                    users.add(fn.name)
    assert users == {"cpu_baseline"}, users
