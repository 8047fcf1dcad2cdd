"""The oracle and the product path share no code and do not import each other."""

import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _py_files(d):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        for f in fs:
            if f.endswith(".py"):
                yield os.path.join(dp, f)


def _imports(path):
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom) and node.module:
            yield node.module


def test_oracle_does_not_import_product():
    for f in _py_files("oracle"):
        for m in _imports(f):
            assert not m.startswith("gemm_chain_amd"), f"{f} imports {m}"


def test_product_does_not_import_oracle():
    for f in _py_files("gemm_chain_amd"):
        for m in _imports(f):
            assert not m.startswith("oracle"), f"{f} imports {m}"
    csrc = os.path.join(ROOT, "gemm_chain_amd", "csrc")
    if os.path.isdir(csrc):
        for dp, _, fs in os.walk(csrc):
            for fn in fs:
                text = open(os.path.join(dp, fn), errors="ignore").read()
                assert "oracle/" not in text and "oracle." not in text, fn
