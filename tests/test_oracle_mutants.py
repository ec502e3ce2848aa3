"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the
pins catch every one of them.

Each mutant is the oracle's C source with one textual substitution, built
with gcc into a temporary directory.  A mutant that passes every pin would
mean the pins leave that part of the oracle unchecked.
"""
import os

import pytest

import oracle as oracle_pkg
from oracle import build as oracle_build
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle_pkg.__file__), "attn_oracle.c")

MUTANTS = {
    "drop_scale": ("e[j] = scale * dot;", "e[j] = dot;"),
    "head_map_modulo": ("const int64_t g = h / G;", "const int64_t g = h % Hkv;"),
    "no_max_subtraction": ("e[j] = exp(e[j] - m);", "e[j] = exp(e[j]); m = 0.0;"),
    "lse_log2": ("*lse = m + log(sum);", "*lse = m + log2(sum);"),
    "lse_without_max": ("*lse = m + log(sum);", "*lse = log(sum);"),
    "transposed_k": ("dot += qrow[d] * kj[d];", "dot += qrow[d] * K[(d * nvis + j) % (nvis * D)];"),
    "unnormalised_weights": ("const double p = e[j] / sum;", "const double p = e[j];"),
    "last_key_dropped": ("for (int64_t j = 0; j < nvis; ++j) {\n    const double* kj",
                         "for (int64_t j = 0; j < nvis - (nvis > 1); ++j) {\n    const double* kj"),
    "value_row_index": ("const double* vj = V + j * D;",
                        "const double* vj = V + ((j + 1) % nvis) * D;"),
    "f16_exponent_bias": ("expo - 25", "expo - 24"),
    "f16_subnormal_scale": ("(double)frac, -24", "(double)frac, -25"),
    "bf16_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "score_sign": ("e[j] = scale * dot;", "e[j] = -scale * dot;"),
    "query_row_offset": ("qrow[d] = widen(q16[flat * D + d], dtype);",
                         "qrow[d] = widen(q16[((flat + 1) % (B * Hq * Lq)) * D + d], dtype);"),
    # causal masking and key slices
    "causal_off_by_one": ("const int64_t n = i + (lk_total - Lq) - key_begin + 1;",
                          "const int64_t n = i + (lk_total - Lq) - key_begin;"),
    "causal_top_left": ("const int64_t n = i + (lk_total - Lq) - key_begin + 1;",
                        "const int64_t n = i - key_begin + 1;"),
    "causal_ignored": ("if (!causal) return Lk;", "return Lk;"),
    "causal_slice_local": ("const int64_t n = i + (lk_total - Lq) - key_begin + 1;",
                           "const int64_t n = i + (Lk - Lq) + 1;"),
    "empty_row_lse_zero": ("    *lse = -INFINITY;\n    return;", "    *lse = 0.0;\n    return;"),
    "empty_keys_refused": ("Lq < 0 || Lk < 0 || D <= 0) return -2;",
                           "Lq < 0 || Lk <= 0 || D <= 0) return -2;"),
    "empty_rows_refused": ("if (B < 0 || Hq < 0 ||", "if (B <= 0 || Hq <= 0 ||"),
    # merge
    "merge_no_max": ("sum += exp(lse_parts[g * nrows + r] - top);",
                     "sum += exp(lse_parts[g * nrows + r]); top = 0.0;"),
    "merge_weight_unnormalised": ("const double w = exp(lse_parts[g * nrows + r] - lse);",
                                  "const double w = exp(lse_parts[g * nrows + r] - top);"),
    "merge_lse_log2": ("const double lse = top + log(sum);", "const double lse = top + log2(sum);"),
    "merge_plain_average": ("const double w = exp(lse_parts[g * nrows + r] - lse);",
                            "const double w = 1.0 / nparts;"),
    "merge_part_stride": ("const double* og = o_parts + (g * nrows + r) * D;",
                          "const double* og = o_parts + (r * nparts + g) * D;"),
}


def _build_mutant(tmp_path, name):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) >= 1, "mutation site for %s not found" % name
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(text.replace(before, after, 1))
    out = str(tmp_path / ("libmutant_%s.so" % name))
    oracle_build.build(src=str(src), out=out, quiet=True)
    return oracle_pkg.Oracle(out)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    orc = _build_mutant(tmp_path, name)
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "mutant %s passes every pin" % name
