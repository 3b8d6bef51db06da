"""Builds libsta.so (all HIP sources, gfx950) in place, next to this file.

    python sliding_tile_attention_amd/build.py [--force]

Run as a script (not as a module of the package): importing the package
loads libsta.so, which is what this builds.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsta.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "workspace.hip", "reorder.hip", "index.hip", "attn_f32.hip", "fwd_bf16.hip", "fwd_fp8.hip",
           "bwd_bf16.hip", "shifts.hip", "schedule.hip"]
HEADERS = ["common.h", "mfma.h", "tiles.h"]
# Per-source extra compiler flags (none at present).
EXTRA = {}
# Compile-time variants of the kernels for measurements, e.g.
#   STA_DEFINES="-DSTA_FWD_QG=2" python sliding_tile_attention_amd/build.py --force
# (the forward with two row groups per wave); empty for the library as shipped.
DEFINES = os.environ.get("STA_DEFINES", "").split()

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # keep the compiler from emitting packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _newest(paths):
    return max(os.path.getmtime(p) for p in paths)


def _compile(src, force):
    s = os.path.join(CSRC, src)
    o = os.path.join(OBJ, src.replace(".hip", ".o"))
    deps = [s] + [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(ROOT, "include", "libsta.h")]
    if not force and not DEFINES and os.path.exists(o) and os.path.getmtime(o) >= _newest(deps):
        return o
    cmd = [HIPCC] + FLAGS + DEFINES + EXTRA.get(src, []) + ["-c", s, "-o", o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return o


PROBE_SRC = "probes.hip"             # measurement probes of bench.py, a library of their own
PROBE_LIB = os.path.join(HERE, "libsta_probe.so")


def build_probe(force=True):
    """The measurement probes that bench.py runs (not part of libsta)."""
    src = os.path.join(CSRC, PROBE_SRC)
    if not force and os.path.exists(PROBE_LIB) and os.path.getmtime(PROBE_LIB) >= os.path.getmtime(src):
        return PROBE_LIB
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (PROBE_SRC, " ".join(cmd), r.stderr))
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(force=True, jobs=None):
    """Compile every HIP source and link libsta.so.  force=True recompiles
    everything (the default: a build step must really build)."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    build_probe(force)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))
