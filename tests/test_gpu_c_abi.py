"""The boundary from plain C: tests/c_abi_check.c allocates device memory
with hipMalloc and runs sta_tile_reorder, sta_index_dims, sta_build_index,
sta_fwd and sta_bwd (fp32 and bf16, shifted windows) with no Python or torch
in the process, checking every output against the CPU oracle."""
import os
import subprocess

import pytest

from tests import c_abi_build
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_c_program_through_the_boundary():
    if not os.path.exists(c_abi_build.EXE):
        c_abi_build.build()
    say("C ABI program")
    env = dict(os.environ, LD_LIBRARY_PATH=c_abi_build.library_path())
    r = subprocess.run([c_abi_build.EXE], capture_output=True, text=True, timeout=180, env=env)
    print(r.stdout, r.stderr)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr
