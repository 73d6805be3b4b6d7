"""The oracle's pins must catch plausible mistakes.

Each case copies oracle.c, plants one mistake (on the CPU, in a temporary
build), and runs the pin suite against that build in a subprocess: the suite
has to fail.  This is what makes the pins a check on the oracle rather than a
restatement of it.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "score_without_scale": ("group += scale * dot;", "group += dot;"),
    "tie_to_higher_index": ("return (a->j > b->j) - (a->j < b->j);",
                            "return (a->j < b->j) - (a->j > b->j);"),
    "centroid_divides_by_page_size": ("(float)(sum / v);", "(float)(sum / P);"),
    "centroid_reads_unused_slots": ("for (int t = 0; t < v; ++t)\n                    sum +=",
                                    "for (int t = 0; t < P; ++t)\n                    sum +="),
    "lse_without_log": ("(float)(m + log(Z));", "(float)(m + Z);"),
    "v_read_token_major": ("return (((size_t)page * Hkv + g) * D + d) * P + t;",
                           "return (((size_t)page * Hkv + g) * P + t) * D + d;"),
    "head_to_group_interleaved": ("g = h / r;", "g = h % Hkv;"),
    "indices_in_rank_order": ("qsort(keep, (size_t)kb, sizeof(int), int_cmp);", ""),
    "partial_block_one_token_short": ("return v < P ? v : P;", "return v < P ? (v > 1 ? v - 1 : v) : P;"),
    "group_score_is_max_head": ("group += scale * dot;", "group = fmax(group, scale * dot * r);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w",
                           "-o", str(so), str(mutant), "-lm"])
    env = dict(os.environ, BTK_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"pins did not catch mutant {name}:\n{res.stdout[-2000:]}"
