"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies sta_oracle.c, makes one plausible mistake in the copy (a
wrong index, a dropped term, a flipped sign, a transposed operand, a wrong
border rule), builds it in a temporary directory and runs the pin suite
against it in a child process.  The unaltered source must pass; every
altered copy must fail at least one pin.  The real oracle is never changed.

Not listed: dropping the cap c = min(w, n).  With c = w > n the clamped
start becomes n - w < 0 and the window still covers exactly the whole axis,
so that change alters no output (an equivalent mutant).
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sta_oracle.c")

MUTANTS = {
    "window-start-rounds-up": ("int start = qc[d] + o - win[d] / 2;",
                               "int start = qc[d] + o - (win[d] + 1) / 2;"),
    "no-high-border-clamp": ("if (start > n[d] - cnt) start = n[d] - cnt;", ""),
    "no-low-border-clamp": ("if (start < 0) start = 0;", ""),
    "offset-sign-flipped": ("int o = off ? off[d] : 0;", "int o = off ? -off[d] : 0;"),
    "window-end-off-by-one": ("kc[d] >= s[d] + c[d]", "kc[d] > s[d] + c[d]"),
    "tile-coords-transposed": ("tc[1] = (id / n[2]) % n[1];", "tc[1] = (id / n[1]) % n[2];"),
    "token-coords-transposed": ("int h = (int)((r / grid[2]) % grid[1]);",
                                "int h = (int)((r / grid[1]) % grid[2]);"),
    "perm-in-tile-order-transposed": (
        "for (int h = b * tile[1]; h < (b + 1) * tile[1] && h < grid[1]; ++h)\n"
        "                        for (int w = c * tile[2]; w < (c + 1) * tile[2] && w < grid[2]; ++w)",
        "for (int w = c * tile[2]; w < (c + 1) * tile[2] && w < grid[2]; ++w)\n"
        "                        for (int h = b * tile[1]; h < (b + 1) * tile[1] && h < grid[1]; ++h)"),
    "lse-drops-max": ("return mx + log(sum);", "return log(sum);"),
    "score-drops-scale": ("ss[m] = p->scale * dot(", "ss[m] = dot("),
    "score-uses-v": ("dot(qi, row_of(p, p->k, b, h, j), p->D)", "dot(qi, row_of(p, p->v, b, h, j), p->D)"),
    "ds-sign": ("double dsij = pij * (dpij - dl);", "double dsij = pij * (dpij + dl);"),
    "dk-drops-scale": ("dk[r * D + d] = scale * ak[d];", "dk[r * D + d] = ak[d];"),
    "dv-uses-ds": ("av[d] += pij * (double)doi[d];", "av[d] += dsij * (double)doi[d];"),
    "dq-uses-v": ("const float *kj = row_of(&p, p.k, b, h, js[a]);",
                  "const float *kj = row_of(&p, p.v, b, h, js[a]);"),
    "delta-drops-p": ("dl += exp(ss[a] - L) * dot(", "dl += dot("),
    "truncate-window-end-off-by-one": ("int hi = lo + win[d] - 1;", "int hi = lo + win[d];"),
    "truncate-centre-not-clamped-high": ("if (centre > n[d] - 1) centre = n[d] - 1;", ""),
    "truncate-centre-not-clamped-low": ("if (centre < 0) centre = 0;", ""),
    "head-offsets-ignore-head-stride": ("((flags & ORACLE_HEAD_OFFS) ? h * T : 0)",
                                        "((flags & ORACLE_HEAD_OFFS) ? h : 0)"),
    "text-keys-hidden-from-video": ("if (i >= p->Nv || j >= p->Nv)\n        return 1;",
                                    "if (i >= p->Nv)\n        return 1;\n    if (j >= p->Nv)\n        return 0;"),
    "perm-cut-tiles-keep-padding-slots": ("= pos++;", "= ((int64_t)(a * n[1] + b) * n[2] + c) * tile[0] * tile[1] * tile[2] + "
                                          "((int64_t)(t % tile[0]) * tile[1] + h % tile[1]) * tile[2] + w % tile[2];"),
    "ragged-tiles-counted-by-floor": ("n[d] = (grid[d] + tile[d] - 1) / tile[d];",
                                      "n[d] = grid[d] / tile[d] + (grid[d] < tile[d]);"),
    "text-queries-see-text-only": ("if (i >= p->Nv || j >= p->Nv)\n        return 1;",
                                   "if (j >= p->Nv)\n        return 1;\n    if (i >= p->Nv)\n        return 0;"),
}


def _build_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must occur exactly once: %r" % old
    path = tmp_path / ("sta_oracle_%s.c" % name)
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("liboracle_%s.so" % name))
    oracle.build(force=True, src=str(path), lib=lib)
    return lib


def _pins_hold(lib):
    r = subprocess.run([sys.executable, "-m", "tests.pin_runner", lib], cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    return r.returncode == 0, r.stdout + r.stderr


def test_unaltered_oracle_passes_pins(tmp_path):
    ok, out = _pins_hold(oracle.build())
    assert ok, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    ok, out = _pins_hold(_build_variant(tmp_path, name, old, new))
    assert not ok, "mutant %s survived every pin:\n%s" % (name, out)
