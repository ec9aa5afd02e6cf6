"""The oracle's pins catch planted mistakes (no GPU).

Each case plants one plausible slip in a copy of oracle/ksa_oracle.c, builds
that copy with the same compiler flags into a temporary directory, and runs
the pin suite against it in a child process (KSA_ORACLE_LIB selects the
build).  The pins must fail for every mutant; the unmodified source must pass
(checked by test_oracle_pins.py itself).
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "ksa_oracle.c")

# (name, text in the oracle, planted replacement)
MUTANTS = [
    ("mean_over_block_size", "double mean = sum / (double)n;", "double mean = sum / (double)s->Bs;"),
    ("truncating_summary_rounding", "ldexp(rint(ldexp(x, -q)), q)", "ldexp(trunc(ldexp(x, -q)), q)"),
    ("wrong_kv_head_of_query", "const int64_t g = h / G;\n  const double sc",
     "const int64_t g = h % s->Hkv;\n  const double sc"),
    ("wrong_heads_in_group_score", "int64_t h = g * G + hh;", "int64_t h = g + hh * s->Hkv;"),
    ("ties_to_highest_index", "return (x->idx > y->idx) - (x->idx < y->idx);",
     "return (x->idx < y->idx) - (x->idx > y->idx);"),
    ("lse_without_max", "lse[b * s->Hq + h] = m + log(z);", "lse[b * s->Hq + h] = log(z);"),
    ("votes_over_whole_context", "const int64_t C = T - W, Kv = N - W;\n#pragma omp parallel for schedule(static)\n  for (int64_t b = 0; b < B; ++b) {\n    orc_rank* a = (orc_rank*)malloc((size_t)C * sizeof(orc_rank));\n    for (int64_t h",
     "const int64_t C = T, Kv = N - W;\n#pragma omp parallel for schedule(static)\n  for (int64_t b = 0; b < B; ++b) {\n    orc_rank* a = (orc_rank*)malloc((size_t)C * sizeof(orc_rank));\n    for (int64_t h"),
    ("window_off_by_one", "row[Kv + i] = (int32_t)(C + i);", "row[Kv + i] = (int32_t)(C + i - 1);"),
    ("partial_block_reads_past_T", "t < (j + 1) * s->Bs && t < s->T; ++t", "t < (j + 1) * s->Bs; ++t"),
    ("scale_one_over_D", "1.0 / sqrt((double)s->D)", "1.0 / (double)s->D"),
    ("selection_not_ascending", "qsort(out + r * keff, (size_t)keff, sizeof(int32_t), orc_cmp_i32);", ";"),
    ("fewest_votes_first", "a[t].val = (double)votes[b * T + t];", "a[t].val = -(double)votes[b * T + t];"),
    ("softmax_weights_unnormalised", "out[(b * s->Hq + h) * s->D + d] = acc / z;",
     "out[(b * s->Hq + h) * s->D + d] = acc;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished from the oracle: %s" % name
    mutated = src.replace(old, new, 1)
    msrc = tmp_path / "ksa_oracle_mutant.c"
    msrc.write_text(mutated)
    mlib = str(tmp_path / "libksa_oracle_mutant.so")
    oracle.build(force=True, src=str(msrc), out=mlib)
    env = dict(os.environ, KSA_ORACLE_LIB=mlib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
