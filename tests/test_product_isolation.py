"""The product path stands alone: it never loads the oracle, and without its native library it fails
with an error instead of computing anything another way (no GPU needed)."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "compressed_kv_cache_03_amd")


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_package_sources_never_import_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith(".py"):
                assert "oracle" not in _imports(os.path.join(dirpath, f)), f


def test_native_sources_never_include_the_oracle():
    csrc = os.path.join(PKG, "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f)).read()
        assert "csa2_oracle" not in text and "oracle/" not in text, f


def test_importing_the_package_loads_no_oracle_module():
    code = ("import sys; sys.path.insert(0, %r); import compressed_kv_cache_03_amd as c; c.lib(); "
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().endswith("[]")


def test_missing_library_fails_loudly():
    code = ("import sys; sys.path.insert(0, %r); import compressed_kv_cache_03_amd as c; "
            "c.LIB_PATH = '/nonexistent/libcsa2.so'; c.version()") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "is not built" in r.stderr
