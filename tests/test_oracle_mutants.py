"""Plant plausible mistakes in a copy of the CPU oracle and check that the
pins (hand-derived examples, validation rules, data invariants, brute force)
catch every one of them (no GPU; the mistakes live only in temporary copies
of the oracle source, built with gcc)."""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "tie_break_slot_descending": (
        "return (x->slot > y->slot) - (x->slot < y->slot);",
        "return (x->slot < y->slot) - (x->slot > y->slot);"),
    "evict_most_recent": (
        "return (x->last_use > y->last_use) - (x->last_use < y->last_use);",
        "return (x->last_use < y->last_use) - (x->last_use > y->last_use);"),
    "hit_not_stamped": (
        "      out[i] = s;\n      st->last_use[s] = t;\n",
        "      out[i] = s;\n"),
    "miss_not_stamped": (
        "    st->slot2pos[s] = p;\n    st->last_use[s] = t;\n",
        "    st->slot2pos[s] = p;\n"),
    "window_off_by_one": (
        "(int64_t)p >= ctx - R", "(int64_t)p > ctx - R"),
    "ring_slot_without_offset": (
        "out[i] = C + (p % R);", "out[i] = (p % R);"),
    "old_position_not_unmapped": (
        "      st->pos2slot[q] = -1;\n", ""),
    "clock_not_advanced": (
        "const int32_t t = ++st->t[0];", "const int32_t t = st->t[0] + 1;"),
    "victims_paired_in_reverse": (
        "int32_t s = order[j].slot;", "int32_t s = order[n_miss - 1 - j].slot;"),
    "range_check_off_by_one": (
        "(p >= 0 && (int64_t)p >= ctx)", "(p >= 0 && (int64_t)p > ctx)"),
    "wrong_row_copied": (
        "copy_row(st, s, p);\n    out[i] = s;", "copy_row(st, s, q >= 0 ? q : p);\n    out[i] = s;"),
    "bytes_counted_per_selection": (
        "(int64_t)n_miss * st->row_bytes;", "(int64_t)k * st->row_bytes;"),
    "duplicates_accepted": (
        "if (sorted[i] == sorted[i - 1]) status |= HSO_STATUS_SEL_DUP;",
        "if (0) status |= HSO_STATUS_SEL_DUP;"),
    "append_skips_ring_slot": (
        "    memcpy(st->slots + (st->C + ctx % st->R) * st->row_bytes, row, (size_t)st->row_bytes);\n",
        "    ;\n"),
}

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
from oracle.oracle import load
from tests import pins
lib = load({lib!r})
try:
    pins.check_validation(lib)
    pins.check_golden("lru_hand_example.txt", lib)
    pins.check_golden("resident_window_example.txt", lib)
    pins.check_data_invariants(lib)
    pins.check_bruteforce_random(lib, n_traces=150)
except AssertionError as e:
    print("caught:", str(e)[:200])
    sys.exit(3)
sys.exit(0)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = obuild.build(str(path), str(tmp_path / "libmutant.so"))
    proc = subprocess.run([sys.executable, "-c", RUNNER.format(root=ROOT, lib=lib)],
                          capture_output=True, text=True, timeout=300)
    assert proc.returncode == 3, (
        f"mistake {name} not caught (exit {proc.returncode}): {proc.stdout} {proc.stderr[-500:]}")


def test_unmutated_oracle_passes_the_same_runner(tmp_path):
    proc = subprocess.run([sys.executable, "-c", RUNNER.format(root=ROOT, lib=obuild.LIB)],
                          capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stdout + proc.stderr[-500:]
