"""The product path has no fallback and does not touch the oracle: the binding raises when
its library is missing, no package source imports the oracle, and libgtms.so neither defines
nor needs an oracle symbol."""
from __future__ import annotations

import ast
import os
import subprocess

import pytest

import variable_length_causal_amd as g

PKG = os.path.dirname(os.path.abspath(g.__file__))


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(g, "LIB_PATH", str(tmp_path / "libgtms.so"))
    monkeypatch.setattr(g, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        g.lib()
    with pytest.raises(RuntimeError):
        g.version()


def test_package_sources_do_not_import_the_oracle():
    for root, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(root, f)).read())
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                assert not any(n.split(".")[0] == "oracle" for n in names), (f, names)


def test_library_has_no_oracle_symbols():
    lib = os.path.join(PKG, "libgtms.so")
    if not os.path.exists(lib):
        pytest.skip("libgtms.so is not built")
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "gtms_oracle" not in out
    needed = subprocess.run(["readelf", "-d", lib], capture_output=True, text=True,
                            check=True).stdout
    assert "oracle" not in needed
