"""The oracle and the HIP path share nothing, and the product path has no fallback (CPU).

- No source of the package (the binding, the HIP kernels, the C ABI) or of the public header
  names the oracle, and no source of the oracle names the package, its kernels or its header.
- The seeded input generators import neither side.
- bench.py imports the oracle only inside its CPU-baseline functions, and the package never.
- With the library missing, the binding raises instead of computing anything.
"""
import ast
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "scaled_dot_product_11_amd")
SOURCE_EXT = (".py", ".hip", ".cpp", ".h", ".c")


def _sources(*dirs):
    for d in dirs:
        for base, _, files in os.walk(d):
            if "__pycache__" in base:
                continue
            for f in files:
                if f.endswith(SOURCE_EXT):
                    path = os.path.join(base, f)
                    with open(path, encoding="utf-8") as fh:
                        yield path, fh.read()


def test_product_sources_never_name_the_oracle():
    found = [p for p, text in _sources(PKG, os.path.join(ROOT, "include"))
             if re.search(r"oracle", text, re.IGNORECASE)]
    assert not found, f"product sources naming the oracle: {found}"


def test_oracle_sources_never_name_the_product():
    pattern = re.compile(r"scaled_dot_product_11_amd|sdpa\.h|sdpa_internal|csrc|libsdpa")
    found = [p for p, text in _sources(os.path.join(ROOT, "oracle")) if pattern.search(text)]
    assert not found, f"oracle sources naming the product: {found}"


def test_input_generators_import_neither_side():
    path = os.path.join(ROOT, "workloads", "__init__.py")
    tree = ast.parse(open(path, encoding="utf-8").read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    assert not names & {"oracle", "scaled_dot_product_11_amd"}, names


def test_bench_imports_the_oracle_only_in_its_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read())
    for node in tree.body:  # module level: no oracle import
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module]
            assert "oracle" not in mods, "bench.py imports the oracle at module level"
    users = []
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, ast.Import) and any(a.name == "oracle" for a in node.names):
                    users.append(fn.name)
    assert users and all(u.startswith("cpu_baseline") for u in users), users


def test_binding_raises_without_the_library(monkeypatch):
    """Every entry point of the binding reaches the library through load_library, which
    raises when the library is missing (CPU tensors are refused before that, by a test of
    their own)."""
    import scaled_dot_product_11_amd._binding as B
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libsdpa_gfx950.so"))
    with pytest.raises(ImportError):
        B.load_library()
    src = open(os.path.join(PKG, "_binding.py"), encoding="utf-8").read()
    assert "ctypes.CDLL(" in src and src.count("ctypes.CDLL(") == 1, "one library load only"
