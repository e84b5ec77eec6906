"""The product path has no fallback and never touches the oracle: the binding
raises when the HIP library is missing, and no file of the package imports
the oracle or the test helpers."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp8_block_scaled_sigmoid_amd")


def test_binding_raises_without_the_library(monkeypatch, tmp_path):
    import fp8_block_scaled_sigmoid_amd as moe
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing" / "libmoe_fp8.so"))
    with pytest.raises(RuntimeError, match="not built"):
        moe.lib()
    with pytest.raises(RuntimeError, match="not built"):
        moe.moe_permute_workspace_bytes(8, 16, 2)


def test_package_never_imports_the_oracle():
    pat = re.compile(r"^\s*(from|import)\s+(oracle|tests|helpers)\b", re.M)
    seen = 0
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), errors="replace").read()
                assert not pat.search(text), f"{f} imports test infrastructure"
                assert "importlib" not in text, f"{f} imports modules by name"
                seen += 1
    assert seen >= 10
    # the HIP sources include nothing from the oracle
    for f in os.listdir(os.path.join(PKG, "csrc")):
        text = open(os.path.join(PKG, "csrc", f), errors="replace").read()
        assert not re.search(r'#include\s+["<][^">]*oracle', text), f
