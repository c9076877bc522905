"""Planted mistakes in the oracle must fail its pins.

Each case copies oracle.c, applies one plausible mistake (a dropped term, a
wrong sign, index or operand), builds it with gcc and runs the pin suite
against that build in a subprocess. The suite must fail for every mutant.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "relu_dropped": ("const double r = d > 0.0 ? d : 0.0;", "const double r = d;"),
    "relu_wrong_side": ("const double r = d > 0.0 ? d : 0.0;", "const double r = d < 0.0 ? -d : 0.0;"),
    "query_scale_wrong_block": ("oracle_ue8m0_value(q_scale_head[b])", "oracle_ue8m0_value(q_scale_head[3 - b])"),
    "key_scale_missing": ("* oracle_ue8m0_value(k_scale_vec[b])", ""),
    "last_head_dropped": ("for (int h = 0; h < ORACLE_H; ++h)", "for (int h = 0; h < ORACLE_H - 1; ++h)"),
    "weights_transposed": ("acc += (double)w_row[h] * r;", "acc += (double)w_row[ORACLE_H - 1 - h] * r;"),
    "scale_bias": ("ldexp(1.0, (e & 255) - 127)", "ldexp(1.0, (e & 255) - 128)"),
    "e2m1_table_typo": ("0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,", "0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 4.0, 6.0,"),
    "key_element_shifted": ("E2M1_VALUE[element_code(k_vec, i)]", "E2M1_VALUE[element_code(k_vec, i ^ 1)]"),
    "tie_break_reversed": ("    return ia < ib;\n}", "    return ia > ib;\n}"),
    "nan_ranks_high": ("if (na != nb) return nb;", "if (na != nb) return na;"),
    "signed_zero_reversed": ("return signbit(sb) ? 1 : 0;", "return signbit(sa) ? 1 : 0;"),
    "short_row_relative": ("out_raw[i] = (int32_t)(start + i);", "out_raw[i] = (int32_t)i;"),
    "short_row_padding": ("for (int64_t i = 0; i < K; ++i) out_raw[i] = -1;", "for (int64_t i = 0; i < K; ++i) out_raw[i] = 0;"),
    "slot_offset_wrong": ("* ORACLE_PAGE + raw % ORACLE_PAGE;", "* ORACLE_PAGE + raw / ORACLE_PAGE;"),
    "window_end_off_by_one": ("end > ORACLE_PAGE * P_log) return -1;", "end >= ORACLE_PAGE * P_log) return -1;"),
    "last_page_unchecked": ("p <= (end - 1) / ORACLE_PAGE; ++p)\n            if", "p < (end - 1) / ORACLE_PAGE; ++p)\n            if"),
    "selection_not_sorted": ("    qsort(out_raw, (size_t)K, sizeof(int32_t), cmp_i32);\n", ""),
    # MXFP4 quantiser
    "quant_ties_away_from_zero": ("if (dm < db || (dm == db && (m & 1) == 0)) best = m;", "if (dm <= db) best = m;"),
    "quant_emax_3": ("int byte = (e2 - 1) - 2 + 127;", "int byte = (e2 - 1) - 3 + 127;"),
    "quant_exponent_rounded_up": ("int byte = (e2 - 1) - 2 + 127;", "int byte = e2 - 2 + 127;"),
    "quant_negative_zero_lost": ("const int neg = signbit(v) ? 1 : 0;", "const int neg = v < 0.0 ? 1 : 0;"),
    "quant_nibbles_swapped": ("codes[16 * b + j] = (uint8_t)(lo | (hi << 4));", "codes[16 * b + j] = (uint8_t)(hi | (lo << 4));"),
    "quant_infinity_not_flagged": ("if (!isfinite(x[i])) return 0xFF;", "if (isnan(x[i])) return 0xFF;"),
    "quant_scale_not_clamped": ("if (byte < 0) byte = 0;", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/not found"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(mut), "-o", str(so),
                    "-lm"], check=True)
    env = dict(os.environ, MQA_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_quant_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
