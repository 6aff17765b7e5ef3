"""The oracle and the HIP path share nothing: the package (Python binding and HIP/C++ sources)
never names the oracle, the oracle never names the package or its sources, and outside the tests
only the benchmark's CPU-baseline function and the build/smoke entry points import the oracle."""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _files(d, exts):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        if "__pycache__" in dp:
            continue
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(dp, f)


def test_package_never_names_the_oracle():
    for p in _files("rvq_quantized_moe_amd", (".py", ".hip", ".hpp", ".cpp", ".h")):
        text = open(p, encoding="utf-8").read()
        assert not re.search(r"\boracle\b|rvq_oracle|orc_", text), p


def test_oracle_never_uses_the_package():
    for p in _files("oracle", (".py",)):
        tree = ast.parse(open(p, encoding="utf-8").read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                assert all(a.name.split(".")[0] != "rvq_quantized_moe_amd" for a in node.names), p
            if isinstance(node, ast.ImportFrom):
                assert (node.module or "").split(".")[0] != "rvq_quantized_moe_amd", p
        text = open(p, encoding="utf-8").read()
        assert "librvq.so" not in text and "csrc" not in text and "include/rvq.h" not in text, p
    for p in _files("oracle", (".c", ".h")):
        text = open(p, encoding="utf-8").read()
        assert not re.search(r"#include\s+\"", text), p   # system headers only, nothing shared


def _oracle_imports(path):
    """(enclosing function name or None) for every import of the oracle in a Python file."""
    tree = ast.parse(open(path, encoding="utf-8").read())
    found = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            name = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(child, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in child.names):
                found.append(fn)
            if isinstance(child, ast.ImportFrom) and (child.module or "").split(".")[0] == "oracle":
                found.append(fn)
            visit(child, name)
    visit(tree, None)
    return found


def test_only_the_cpu_baseline_and_entry_points_import_the_oracle():
    assert set(_oracle_imports(os.path.join(ROOT, "bench.py"))) <= {"cpu_baseline"}
    assert set(_oracle_imports(os.path.join(ROOT, "__graft_entry__.py"))) <= {"build", "smoke"}
    for p in _files("rvq_quantized_moe_amd", (".py",)):
        assert _oracle_imports(p) == [], p
