"""The product path stands on its own: it fails loudly without libpma.so, it
never reaches the oracle (no import in the package, no link in the library),
and the oracle's C library links nothing of libpma.  CPU only."""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "packed_masked_attention_amd")


def _imports(path):
    tree = ast.parse(open(path).read(), path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            yield from (a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith(".py"):
                for mod in _imports(os.path.join(dirpath, f)):
                    assert not mod.split(".")[0] == "oracle", f"{f} imports {mod}"


def test_oracle_never_imports_the_package():
    for dirpath, _, files in os.walk(os.path.join(ROOT, "oracle")):
        for f in files:
            if f.endswith(".py"):
                for mod in _imports(os.path.join(dirpath, f)):
                    assert "packed_masked_attention_amd" not in mod, f"{f} imports {mod}"


def _needed(so):
    """DT_NEEDED entries of an ELF shared library, read with readelf."""
    out = subprocess.run(["readelf", "-d", so], capture_output=True, text=True, check=True).stdout
    return [ln.split("[", 1)[1].rstrip("]") for ln in out.splitlines() if "(NEEDED)" in ln]


@pytest.mark.parametrize("so,other", [
    ("packed_masked_attention_amd/libpma.so", "oracle"),
    ("oracle/liboracle.so", "pma"),
])
def test_libraries_do_not_link_each_other(so, other):
    path = os.path.join(ROOT, so)
    if not os.path.exists(path):
        pytest.skip(f"{so} not built")
    needed = _needed(path)
    assert not any(other in n for n in needed), needed


def test_missing_library_fails_loudly(tmp_path):
    """With libpma.so absent the binding raises on its first call instead of
    falling back to anything else."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from packed_masked_attention_amd import binding as B\n"
        "B.LIB_PATH = %r\n"
        "B._lib = None\n"
        "try:\n"
        "    B.lib()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(1)\n" % (ROOT, str(tmp_path / "libpma.so")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "is missing" in r.stdout
