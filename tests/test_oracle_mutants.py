"""Mutation check of the oracle pins: each plausible mistake below is planted
in a private copy of the oracle, compiled on the CPU, and the pin suite must
fail against it.  The real oracle is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lsa_oracle.c")

MUTANTS = {
    "eligible_off_by_one": ("int64_t e = t / bs - window / bs + 1;",
                            "int64_t e = t / bs - window / bs;"),
    "tie_break_highest_index": ("return (a->c > b->c) - (a->c < b->c);",
                                "return (a->c < b->c) - (a->c > b->c);"),
    "mean_wrong_divisor": ("(float)(s / (double)bs)", "(float)(s / (double)(bs - 1))"),
    "window_starts_late": ("lo[nr] = ncand * bs;", "lo[nr] = ncand * bs + 1;"),
    "gqa_interleaved_groups": ("const int64_t kvh = b * Hkv + h / rep;",
                               "const int64_t kvh = b * Hkv + h % Hkv;"),
    "scale_dropped_in_exp": ("exp(l * scale - m)", "exp(l - m)"),
    "score_reversed_operand": ("s += qd[d] * (double)summ[c * D + d];",
                               "s += qd[d] * (double)summ[c * D + (D - 1 - d)];"),
    "keeps_one_block_too_few": ("const int64_t keep = ncand < k ? ncand : k;",
                                "const int64_t keep = ncand < k ? ncand : k - 1;"),
    "window_excludes_query": ("hi[nr] = t + 1;", "hi[nr] = t;"),
    "consensus_first_head_only": ("for (int64_t hh = 0; hh < rep; ++hh) {",
                                  "for (int64_t hh = 0; hh < 1; ++hh) {"),
    "consensus_interleaved_groups": ("const int64_t qr = ((b * Hq + g * rep + hh) * per + p) * D;",
                                     "const int64_t qr = ((b * Hq + g + hh * Hkv) * per + p) * D;"),
    "consensus_scores_last_head": ("s += sh;", "s = sh;"),
    "cumulant_sample_covariance": ("S[d * D + e] = a / (double)bs;",
                                   "S[d * D + e] = a / (double)(bs - 1);"),
    "cumulant_missing_half": ("buf[c].s = first + 0.5 * beta * quad;",
                              "buf[c].s = first + beta * quad;"),
    "cumulant_second_moment": ("m[d] = a / (double)bs;", "m[d] = 0.0 * a;"),
    "tree_tail_dropped": ("for (int64_t c = S * F; c < E; ++c) {",
                          "for (int64_t c = S * F; c < S * F; ++c) {"),
    "tree_node_strided": ("cbuf[nc].c = kept[j] * F + x;", "cbuf[nc].c = kept[j] + x * nn;"),
    "tree_node_mean_divisor": ("nu[gs * D + d] = (float)(a / (double)F);",
                               "nu[gs * D + d] = (float)(a / (double)(F - 1));"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           str(mut), "-o", str(so), "-lm"])
    env = dict(os.environ, LSA_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
