"""Planted mistakes in the window-shift producer's oracle must be caught by
its pins (CPU only).  Each case copies oracle/shift.py, makes one plausible
mistake in the copy, imports it as a module of its own and runs every check
of tests/test_oracle_shift.py against it: at least one must fail.  The real
module is never changed."""
import importlib.util
import os

import pytest

from tests import test_oracle_shift as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "shift.py")

MUTANTS = {
    "shift-sign-flipped": ("off = np.tile(np.asarray(o, np.int32), (T, 1))",
                           "off = np.tile(-np.asarray(o, np.int32), (T, 1))"),
    "mass-not-weighted-by-length": ("e = lens[None, None, None, :] * np.exp(z)", "e = np.exp(z)"),
    "means-are-sums": ("return sums / lens[None, None, :, None], lens", "return sums, lens"),
    "ties-to-largest-shift": ("order = np.lexsort((np.arange(len(cands)), l1))",
                              "order = np.lexsort((np.arange(len(cands)), -l1))"),
    "ties-to-last-in-raster-order": ("order = np.lexsort((np.arange(len(cands)), l1))",
                                     "order = np.lexsort((-np.arange(len(cands)), l1))"),
    "pooling-averages-logits": ("        qm, km = qm.mean(axis=0, keepdims=True), km.mean(axis=0, keepdims=True)\n"
                                "    z = scale * np.einsum(\"bhqd,bhkd->bhqk\", qm, km)",
                                "        z = (scale * np.einsum(\"bhqd,bhkd->bhqk\", qm, km)).mean(axis=0, keepdims=True)\n"
                                "    else:\n"
                                "        z = scale * np.einsum(\"bhqd,bhkd->bhqk\", qm, km)"),
    "scale-dropped": ("z = scale * np.einsum(\"bhqd,bhkd->bhqk\", qm, km)",
                      "z = np.einsum(\"bhqd,bhkd->bhqk\", qm, km)"),
    "logits-q-against-q": ("z = scale * np.einsum(\"bhqd,bhkd->bhqk\", qm, km)",
                           "z = scale * np.einsum(\"bhqd,bhkd->bhqk\", qm, qm)"),
    "window-of-unshifted-tile": ("lists = window_lists(grid, tile, window, o, border)",
                                 "lists = window_lists(grid, tile, window, 0 * o, border)"),
    "border-rule-ignored": ("kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, [window], off, border=border)",
                            "kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, [window], off)"),
}


def _load_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must occur exactly once: %r" % old
    path = tmp_path / ("shift_%s.py" % name.replace("-", "_"))
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("shift_mutant_" + name.replace("-", "_"), str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _failures(mod):
    failed = []
    for name, check in pins.all_checks():
        try:
            check(mod)
        except AssertionError:
            failed.append(name)
    return failed


def test_unaltered_copy_passes(tmp_path):
    mod = _load_variant(tmp_path, "none", "import itertools", "import itertools")
    assert _failures(mod) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    mod = _load_variant(tmp_path, name, old, new)
    failed = _failures(mod)
    assert failed, "mutant %s passes every pin" % name
