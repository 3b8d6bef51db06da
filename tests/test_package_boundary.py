"""The Python package is a thin binding over libsta: importing it loads the
HIP library and nothing of the oracle, and without the library it refuses
to import (there is no CPU fallback)."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sliding_tile_attention_amd")


def _run(code, cwd):
    return subprocess.run([sys.executable, "-c", code], cwd=cwd, capture_output=True, text=True, timeout=300)


def test_import_loads_libsta_and_not_the_oracle():
    r = _run("import sys, sliding_tile_attention_amd as sta\n"
             "print(sta.LIB_PATH)\n"
             "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.') or 'tests' in m))\n"
             "maps = open('/proc/self/maps').read()\n"
             "print('libsta.so' in maps, 'liboracle' in maps)", ROOT)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    assert lines[0] == os.path.join(PKG, "libsta.so")
    assert lines[1] == "[]"
    assert lines[2] == "True False"


def test_import_without_the_library_raises(tmp_path):
    dst = tmp_path / "sliding_tile_attention_amd"
    dst.mkdir()
    shutil.copy(os.path.join(PKG, "__init__.py"), dst / "__init__.py")
    r = _run("import sliding_tile_attention_amd", str(tmp_path))
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr
