"""CPU: the product path has no fallback.

Without the built HIP library every entry point must raise instead of
computing anything another way, and the package never reaches the CPU oracle
(which only the tests, the smoke check and the benchmark's CPU baseline use).
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_fails_loudly(monkeypatch):
    from sparse_attention_token_amd import hisa

    monkeypatch.setattr(hisa, "_lib", None)
    monkeypatch.setattr(hisa, "_LIB_PATH", os.path.join(ROOT, "no-such-dir", "libhisa.so"))
    with pytest.raises(RuntimeError, match="not built"):
        hisa.lib()
    with pytest.raises(RuntimeError, match="not built"):
        hisa.hisa_abi_version()
    with pytest.raises(RuntimeError, match="not built"):
        hisa.hisa_index_workspace(1, 1, 4, 64, 1024, 64, 4, 64)


def test_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "sparse_attention_token_amd")
    for name in sorted(os.listdir(pkg)):
        if name.endswith(".py"):
            text = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), name
            assert "libhisa_oracle" not in text, name
