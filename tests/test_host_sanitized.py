"""libsta's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The host-side sources (argument checks, index sizing, the workspace pool)
are compiled with both sanitizers on the host pass only (device code as in
the library), linked with the other objects of the in-tree build into a
scratch shared library, and driven by tests/host_asan_check.c: status
strings, index sizing over a sweep of geometries, and malformed calls of
every entry point, which must be refused before anything is launched.  No
GPU is used.
"""
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sliding_tile_attention_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_ONLY = ["api.hip", "workspace.hip"]
# each sanitizer flag goes to the host compilation only
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build_module():
    spec = importlib.util.spec_from_file_location("_sta_build", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="needs hipcc")
def test_host_code_under_sanitizers(tmp_path):
    b = _build_module()
    others = [os.path.join(b.OBJ, s.replace(".hip", ".o")) for s in b.SOURCES if s not in HOST_ONLY]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        pytest.skip("library objects not built: %s" % ", ".join(missing))
    host_flags = [x for f in SANITIZE for x in ("-Xarch_host", f)]
    flags = [f if f != "-O3" else "-O1" for f in b.FLAGS] + ["-g"] + host_flags
    objs = []
    for src in HOST_ONLY:
        o = str(tmp_path / src.replace(".hip", ".o"))
        _run([b.HIPCC] + flags + ["-c", os.path.join(b.CSRC, src), "-o", o])
        objs.append(o)
    lib = str(tmp_path / "libsta_sanitized.so")
    _run([b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + objs + others)
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    drv_o, exe = str(tmp_path / "drv.o"), str(tmp_path / "host_asan_check")
    _run([clang, "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
          "-c", os.path.join(ROOT, "tests", "host_asan_check.c"), "-o", drv_o])
    _run([clang + "++", "-fsanitize=address,undefined", drv_o, "-o", exe, "-L" + str(tmp_path),
          "-l:libsta_sanitized.so", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + str(tmp_path) + ":" + os.path.join(ROCM, "lib")])
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host sanitized ok" in r.stdout
