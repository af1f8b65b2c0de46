"""Plant mistakes in copies of the oracle's source and check the pins catch each one.

Each mutant is a one-line textual change to oracle/oracle.c (a wrong tie-break, a
dropped term, a wrong sign, a transposed operand, an off-by-one in the iteration
count, ...), compiled with gcc into a temporary library and run through every pin
in a child process.  The real oracle must pass every pin (test_oracle_pins.py);
each mutant must fail at least one.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "tie_break_highest_index": ("if (s > best) {", "if (s >= best) {"),
    "dropped_first_component": ("for (int c = 0; c < d; ++c)", "for (int c = 1; c < d; ++c)"),
    "argmin_instead_of_argmax": ("s += (double)a[c] * (double)b[c];", "s -= (double)a[c] * (double)b[c];"),
    "top2_not_shifted": ("second = best;\n            best = s;", "best = s;"),
    "mutual_check_dropped": ("if (nn21[j] != i) continue;", "if (0) continue;"),
    "mutual_pair_transposed": ("pairs[2 * m + 1] = j;", "pairs[2 * m + 1] = (int32_t)i;"),
    "one_iteration_short": ("for (int32_t t = 0; t < T; ++t) {", "for (int32_t t = 0; t + 1 < T; ++t) {"),
    "collect_without_reciprocity": ("if (u2 == u) {", "if (u2 == u || t == 0) {"),
    "restart_from_seed": ("cur[c] = u2;", "cur[c] = u;"),
    "backward_search_transposed": ("orc_nn_parallel(B, todo, nt, A, n1, d,", "orc_nn_parallel(A, todo, nt, B, n2, d,"),
    "seed_grid_column_major": ("cur[c] = (int32_t)(y * W1 + x);", "cur[c] = (int32_t)(x * H1 + y);"),
    "clean_flag_ignores_backward": ("if (!(mg12[u] > eps) || !(mg21[v] > eps)) clean[c] = 0;",
                                    "if (!(mg12[u] > eps)) clean[c] = 0;"),
    "fresh_counts_every_live_pixel": ("if (!ever1[u]) ++first_visits;", "++first_visits;"),
    "fresh_forgets_earlier_iterations": ("if (alive[c]) { seen1[cur[c]] = 0; ever1[cur[c]] = 1; }",
                                         "if (alive[c]) { seen1[cur[c]] = 0; }"),
    "seed_end_records_partner": ("if (seed_u) seed_u[c] = u;", "if (seed_u) seed_u[c] = v;"),
    "seed_clean_always_set": ("for (int64_t c = 0; c < ns; ++c) seed_clean[c] = clean[c];",
                              "for (int64_t c = 0; c < ns; ++c) seed_clean[c] = 1;"),
    # pointmap metric
    "point_metric_ignored": ("if (metric == ORC_NEG_SQ_L2) {", "if (0) {"),
    "point_farthest_instead_of_nearest": ("return -acc;", "return acc;"),
    "point_dropped_first_coordinate": ("for (int k = 0; k < d; ++k) {", "for (int k = 1; k < d; ++k) {"),
    "point_abs_difference": ("acc += diff * diff;", "acc += fabs(diff);"),
    "point_backward_search_inner_product": ("orc_nn_parallel(B, todo, nt, A, n1, d, metric,",
                                            "orc_nn_parallel(B, todo, nt, A, n1, d, ORC_INNER,"),
    "point_margin_absolute": ("return (top1 - top2) / -top2;", "return top1 - top2;"),
    # matching loss
    "nce_shift_dropped": ("sum += exp(orc_similarity(q, j->B + k * (int64_t)j->d, j->d) / j->tau - m);",
                          "sum += exp(orc_similarity(q, j->B + k * (int64_t)j->d, j->d) / j->tau);"),
    "nce_positive_from_query_index": ("j->B + (int64_t)j->gt[2 * t + 1] * j->d", "j->B + (int64_t)j->gt[2 * t] * j->d"),
    "nce_temperature_ignored": ("const double z = orc_similarity(q, j->B + k * (int64_t)j->d, j->d) / j->tau;",
                                "const double z = orc_similarity(q, j->B + k * (int64_t)j->d, j->d);"),
    "nce_sign_flipped": ("j->terms[t] = m + log(sum) - pos;", "j->terms[t] = pos - m - log(sum);"),
    # matching-loss gradient
    "grad_positive_term_dropped": ("for (int e = 0; e < d; ++e) g[e] -= (double)bj[e];", ""),
    "grad_rows_without_temperature": ("row[e] += g[t * (int64_t)d + e] / tau;", "row[e] += g[t * (int64_t)d + e];"),
    "grad_cols_match_on_query_index": ("if (j->gt[2 * t + 1] == k)", "if (j->gt[2 * t] == k)"),
    "grad_cols_softmax_unnormalised": ("const double pk = exp(orc_similarity(a, bk, d) / j->tau - j->lse[t]);",
                                       "const double pk = exp(orc_similarity(a, bk, d) / j->tau);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique/found"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                           "-pthread", str(src), "-o", str(lib), "-lm"])
    out = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "pins.py"), str(lib)],
                         capture_output=True, text=True, timeout=300)
    if out.returncode != 0:
        return  # the broken build crashed the pin run: caught
    failed = json.loads(out.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} passed every pin"
