"""Structural guards, no GPU needed.

* The binding raises at import when the native library is missing: there is
  no fallback path.
* The product package never imports the oracle, the oracle never imports the
  product, and the shared input generators import neither.
"""
import ast
import importlib.util
import os
import shutil

import pytest

from tests.conftest import ROOT

PKG = os.path.join(ROOT, "mla_chunked_context_amd")


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def _py_files(folder):
    for dirpath, _, files in os.walk(folder):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(dirpath, f)


def test_missing_library_raises_at_import(tmp_path):
    pkg = tmp_path / "mla_pkg_without_lib"
    pkg.mkdir()
    shutil.copy(os.path.join(PKG, "__init__.py"), pkg / "__init__.py")
    spec = importlib.util.spec_from_file_location("mla_pkg_without_lib", pkg / "__init__.py",
                                                  submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="missing"):
        spec.loader.exec_module(mod)


def test_product_does_not_import_the_oracle():
    for f in _py_files(PKG):
        assert "oracle" not in _imports(f), f


def test_oracle_does_not_import_the_product():
    for f in _py_files(os.path.join(ROOT, "oracle")):
        assert "mla_chunked_context_amd" not in _imports(f), f


def test_shared_inputs_import_neither_side():
    for f in _py_files(os.path.join(ROOT, "workloads")):
        names = _imports(f)
        assert "oracle" not in names and "mla_chunked_context_amd" not in names, f


def test_native_sources_do_not_reference_the_oracle():
    for dirpath, _, files in os.walk(os.path.join(PKG, "csrc")):
        for fn in files:
            text = open(os.path.join(dirpath, fn), errors="replace").read()
            assert "oracle" not in text.lower(), fn
