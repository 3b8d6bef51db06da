"""Builds tests/c_abi_check.c, a plain C program that drives libsta through
its C ABI and checks it against the CPU oracle, into tests/_build/."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_check.c")
EXE = os.path.join(ROOT, "tests", "_build", "c_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    tmp = EXE + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
                           "-I" + os.path.join(ROOT, "include"), SRC, "-o", tmp,
                           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                           "-L" + os.path.join(ROOT, "sliding_tile_attention_amd"), "-l:libsta.so",
                           "-L" + os.path.join(ROOT, "oracle"), "-l:liboracle.so", "-lm"])
    os.replace(tmp, EXE)
    return EXE


def library_path():
    """LD_LIBRARY_PATH that finds libsta.so, the oracle and the HIP runtime."""
    parts = [os.path.join(ROOT, "sliding_tile_attention_amd"), os.path.join(ROOT, "oracle"), os.path.join(ROCM, "lib")]
    old = os.environ.get("LD_LIBRARY_PATH")
    return ":".join(parts + ([old] if old else []))
