"""Planted mistakes in the quantized-attention oracle must be caught by its
pins (CPU only).  Each case copies oracle/quant.py, makes one plausible
mistake in the copy, imports it as a module of its own and runs every check
of tests/test_oracle_quant.py against it: at least one must fail.  The real
module is never changed."""
import importlib.util
import os

import pytest

from tests import test_oracle_quant as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "quant.py")

MUTANTS = {
    # step 6: where P is rounded
    "p-shift-sign-flipped": ("x = np.exp2(s - M + P_SHIFT)", "x = np.exp2(s - M - P_SHIFT)"),
    "floor-for-ceil-of-row-max": ("    M = float(np.ceil(s.max()))", "    M = float(np.floor(s.max()))"),
    "p-rescale-dropped": ("return e4m3(x) * 2.0 ** -P_SHIFT, M, x", "return e4m3(x), M, x"),
    "p-unrounded": ("return e4m3(x) * 2.0 ** -P_SHIFT, M, x", "return x * 2.0 ** -P_SHIFT, M, x"),
    # step 7: the smoothing's LSE correction
    "lse-correction-sign": ("lse[n_] = lse0 + scale * float(", "lse[n_] = lse0 - scale * float("),
    "lse-correction-dropped": ("lse[n_] = lse0 + scale * float(", "lse[n_] = lse0 + 0 * scale * float("),
    # steps 1-4: the scale groups and the smoothing
    "k-scaled-per-tile": ("blk = tid * ((L + KEY_BLOCK - 1) // KEY_BLOCK) + rank // KEY_BLOCK", "blk = tid"),
    "k-blocks-of-32": ("blk = tid * ((L + KEY_BLOCK - 1) // KEY_BLOCK) + rank // KEY_BLOCK",
                       "blk = tid * ((L + 31) // 32) + rank // 32"),
    "v-scaled-per-row": ("amax_v = np.abs(v).max(axis=2, keepdims=True)",
                         "amax_v = np.abs(v).max(axis=3, keepdims=True)"),
    "q-scaled-per-column": ("qc, sq = int8_codes(q, np.abs(q).max(axis=3, keepdims=True))",
                            "qc, sq = int8_codes(q, np.abs(q).max(axis=2, keepdims=True))"),
    "smoothing-dropped": ("ks = (k - m).astype(np.float32)", "ks = k.astype(np.float32)"),
    "v-codes-unrounded": ("vc = e4m3((v * inv_v).astype(np.float32))", "vc = (v * inv_v).astype(np.float64)"),
    "int8-truncated": ("np.clip(np.rint((x * inv).astype(np.float32)), -127, 127)",
                       "np.clip(np.trunc((x * inv).astype(np.float32)), -127, 127)"),
    # the flip bound
    "bound-ignores-subnormals": ("step = np.where(x < 2.0 ** -5, 2.0 ** -8, step)", "step = step"),
    "bound-margin-too-small": ("rel = 2.0 * (np.log(2.0)", "rel = 2.0 ** -30 * (np.log(2.0)"),
}


def _load_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must occur exactly once: %r" % old
    path = tmp_path / ("quant_%s.py" % name.replace("-", "_"))
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("quant_mutant_" + name.replace("-", "_"), str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _failures(mod):
    failed = []
    for name, check in pins.all_checks():
        try:
            check(mod)
        except Exception:            # a failed assertion, or a crash of the altered copy
            failed.append(name)
    return failed


def test_unaltered_copy_passes(tmp_path):
    mod = _load_variant(tmp_path, "none", "import numpy as np", "import numpy as np")
    assert _failures(mod) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    mod = _load_variant(tmp_path, name, old, new)
    failed = _failures(mod)
    assert failed, "mutant %s passes every pin" % name
