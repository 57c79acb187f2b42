"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant below is a plausible slip in the oracle's source (a flipped
comparison, a dropped term, a wrong index or sign, a transposed operand).
The test writes the mutated source to a temporary directory, compiles it
with g++, and runs the fast pin battery (tests/oracle_battery.py) against it
in a separate process.  Every mutant must make the battery fail; the
unmodified source must pass it.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")
BATTERY = os.path.join(ROOT, "tests", "oracle_battery.py")

MUTANTS = {
    "accept_test_transposed": ("bool accept = u * p < q;", "bool accept = u * q < p;"),
    "residual_sign": ("std::max(0.0, tq[n].pi[v] - dp[n].pi[v])",
                      "std::max(0.0, dp[n].pi[v] - tq[n].pi[v])"),
    "bonus_wrong_position": ("w[v] = tq[Kb].pi[v];", "w[v] = tq[0].pi[v];"),
    "temperature_dropped": ("std::exp((x[v] - M) / tau)", "std::exp((x[v] - M))"),
    "temperature_inverted": ("std::exp((x[v] - M) / tau)", "std::exp((x[v] - M) * tau)"),
    "topk_off_by_one": ("sorted[top_k - 1]", "sorted[top_k > 1 ? top_k - 2 : 0]"),
    "topk_ties_dropped": ("keep[v] = (x[v] >= kth);", "keep[v] = (x[v] > kth);"),
    "topp_excludes_crossing_group": ("bool kept = (i == 0) || (before < top_p);",
                                     "bool kept = (i == 0) || (before + group_mass < top_p);"),
    "cdf_unscaled_target": ("double target = u * S;", "double target = u;"),
    "philox_multiplier": ("const uint32_t kMulA = 0xD2511F53u;", "const uint32_t kMulA = 0xD2511F51u;"),
    "uniform_shift": ("(draw_word(seed, g, t, purpose) >> 8)", "(draw_word(seed, g, t, purpose) >> 9)"),
    "counter_words_swapped": ("uint32_t ctr[4] = {(uint32_t)g, t, purpose, (uint32_t)(g >> 32)};",
                              "uint32_t ctr[4] = {(uint32_t)g, purpose, t, (uint32_t)(g >> 32)};"),
    "greedy_highest_index": ("while (x[gidx] != M) ++gidx;",
                             "gidx = V - 1; while (x[gidx] != M) --gidx;"),
    "draft_row_stride": ("size_t base = ((size_t)b * KM + t) * Vs;",
                         "size_t base = ((size_t)b * KM + (t + 1) % (KM > 0 ? KM : 1)) * Vs;"),
    "no_stop_at_first_rejection": ("if (!accept) { n = t; break; }", "if (!accept) { n = t; }"),
    "emitted_prefix_reversed": ("for (int t = 0; t < n; ++t) toks[t] = d[t];",
                                "for (int t = 0; t < n; ++t) toks[t] = d[n - 1 - t];"),
    "resample_reuses_accept_uniform": (
        "u = draw_uniform(a->seed, g, (uint32_t)n, ORACLE_PURPOSE_RESAMPLE);",
        "u = draw_uniform(a->seed, g, (uint32_t)n, ORACLE_PURPOSE_ACCEPT);"),
    "empty_row_undetected": ("if (x[v] != -kInf) any_not_neg_inf = true;", "any_not_neg_inf = true;"),
    "diag_swapped": ("a->diag[((size_t)b * KM + t) * 2 + 0] = q;",
                     "a->diag[((size_t)b * KM + t) * 2 + 0] = p;"),
    # the boundary flags that excuse a row from exact comparison.  (Dropping
    # the accept flag's guard q/p < 1 + 1e-6 is not a mutant: u < 1, so
    # |u - q/p| < 1e-6 already implies it.)
    "window_times_10": ("const double kWindow = 1e-6;", "const double kWindow = 1e-5;"),
    "window_over_10": ("const double kWindow = 1e-6;", "const double kWindow = 1e-7;"),
    "accept_flag_inverted": ("std::fabs(u - ratio) < kWindow", "std::fabs(u - ratio) > kWindow"),
    "accept_flag_one_sided": ("std::fabs(u - ratio) < kWindow", "u - ratio < kWindow"),
    "cdf_flag_low_side_dropped": ("if ((ilo && u - lo < kWindow) || (ihi && hi - u < kWindow))",
                                  "if (ihi && hi - u < kWindow)"),
    "cdf_flag_high_side_dropped": ("if ((ilo && u - lo < kWindow) || (ihi && hi - u < kWindow))",
                                   "if (ilo && u - lo < kWindow)"),
    "cdf_flag_sides_swapped": ("if ((ilo && u - lo < kWindow) || (ihi && hi - u < kWindow))",
                               "if ((ilo && hi - u < kWindow) || (ihi && u - lo < kWindow))"),
    "cdf_low_end_counts": ("*interior_lo = any_before;", "*interior_lo = true;"),
    "cdf_high_end_counts": ("*interior_hi = any_after;", "*interior_hi = true;"),
    "topp_draft_flag_dropped": ("if (dp[t].topp_margin < kWindow) flags |= ORACLE_FL_TOPP;",
                                "if (false) flags |= ORACLE_FL_TOPP;"),
    "topp_margin_signed": ("margin = std::min(margin, std::fabs(before - top_p));",
                           "margin = std::min(margin, top_p - before);"),
    "accept_position_index": ("double q = tq[t].pi[d[t]], p = dp[t].pi[d[t]];",
                              "double q = tq[t + 1].pi[d[t]], p = dp[t].pi[d[t]];"),
}


def _run_battery(lib_path):
    r = subprocess.run([sys.executable, BATTERY, lib_path], capture_output=True, text=True,
                       timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-400:]


def _build(src_text, d):
    src = os.path.join(d, "oracle.cpp")
    with open(src, "w") as f:
        f.write(src_text)
    # the header is the oracle's own; copy it next to the mutant
    with open(os.path.join(ROOT, "oracle", "oracle.h")) as f:
        hdr = f.read()
    with open(os.path.join(d, "oracle.h"), "w") as f:
        f.write(hdr)
    return oracle.compile_oracle(src, os.path.join(d, "liboracle_mut.so"))


def test_unmodified_oracle_passes_battery():
    with tempfile.TemporaryDirectory() as d:
        lib = _build(open(SRC).read(), d)
        rc, out = _run_battery(lib)
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        lib = _build(text.replace(old, new), d)
        rc, out = _run_battery(lib)
    assert rc != 0, f"mutant {name} survived the pins: {out}"
