"""Every plausible slip in the oracle must fail at least one pin.

Each case copies ``oracle/attn_oracle.c``, plants one mistake by text
replacement (a dropped term, a wrong sign, a wrong index, a transposed operand,
an off-by-one mask, a wrong log base), compiles the copy into a temporary
directory and runs the pin suite on it.  The real oracle is never modified.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "dot_wrong_index": ("dot += q_i[d] * k_j[d];", "dot += q_i[d] * k_j[0];"),
    "dropped_scale": ("p[j] = scale * dot;", "p[j] = dot;"),
    "min_not_max": ("if (p[j] > m)", "if (p[j] < m)"),
    "no_max_subtraction": ("p[j] = exp(p[j] - m);", "p[j] = exp(p[j]);"),
    "exp_sign_flip": ("p[j] = exp(p[j] - m);", "p[j] = exp(m - p[j]);"),
    "pv_wrong_index": ("acc[d] += p[j] * v_j[d];", "acc[d] += p[j] * v_j[0];"),
    "no_normalisation": ("o_i[d] = acc[d] / l;", "o_i[d] = acc[d];"),
    "lse_base2": ("*lse_i = m + log(l);", "*lse_i = m + log2(l);"),
    "lse_drops_max": ("*lse_i = m + log(l);", "*lse_i = log(l);"),
    "causal_off_by_one": ("int64_t a = 0, b = causal && i < Sk - 1 ? i : Sk - 1;",
                          "int64_t a = 0, b = causal && i < Sk - 1 ? (i > 0 ? i - 1 : 0) : Sk - 1;"),
    "causal_wrong_triangle": ("int64_t a = 0, b = causal && i < Sk - 1 ? i : Sk - 1;",
                              "int64_t a = causal && i < Sk - 1 ? i : 0, b = Sk - 1;"),
    "k_transposed": ("const double *k_j = k_bh + j * D;", "const double *k_j = k_bh + j;"),
    "v_transposed": ("const double *v_j = v_bh + j * D;", "const double *v_j = v_bh + j;"),
    "k_head_offset_dropped": ("k + (kvh * Sk + lo) * D", "k + lo * D"),
    "v_head_offset_dropped": ("v + (kvh * Sk + lo) * D", "v + lo * D"),
    "acc_init_one": ("acc[d] = 0.0;", "acc[d] = 1.0;"),
    "l_init_one": ("double l = 0.0;", "double l = 1.0;"),
    "q_row_offset": ("q + flat * D", "q + bh * Sq * D"),
    # backward
    "bwd_drops_row_term": ("const double ds = w[j] * (g[j] - row);", "const double ds = w[j] * g[j];"),
    "bwd_ds_without_p": ("const double ds = w[j] * (g[j] - row);", "const double ds = g[j] - row;"),
    "bwd_row_term_sign": ("const double ds = w[j] * (g[j] - row);", "const double ds = w[j] * (g[j] + row);"),
    "bwd_dq_no_scale": ("dq_i[d] += scale * ds * kr[d];", "dq_i[d] += ds * kr[d];"),
    "bwd_dq_uses_v": ("dq_i[d] += scale * ds * kr[d];", "dq_i[d] += scale * ds * v_h[(lo + j) * D + d];"),
    "bwd_dk_uses_k": ("dk_j[d] += scale * ds * q_i[d];", "dk_j[d] += scale * ds * kr[d];"),
    "bwd_dv_uses_ds": ("dv_j[d] += w[j] * do_i[d];", "dv_j[d] += ds * do_i[d];"),
    "bwd_dv_wrong_index": ("dv_j[d] += w[j] * do_i[d];", "dv_j[d] += w[j] * do_i[0];"),
    "bwd_dp_wrong_row": ("const double *vr = v_bh + j * D;", "const double *vr = v_bh;"),
    "bwd_unnormalised_p": ("w[j] /= total;", "w[j] /= 1.0;"),
    "bwd_causal_sees_all": ("key_range(i, Sk, causal, wl, wr, &lo, &hi);\n            const int64_t n_keys = hi - lo + 1;\n            const double *q_i = q_g",
                            "key_range(i, Sk, 0, wl, wr, &lo, &hi);\n            const int64_t n_keys = hi - lo + 1;\n            const double *q_i = q_g"),
    "bwd_rows_p_not_normalised": ("const double p = exp(scale * acc - top[x]) / sum[x];",
                                  "const double p = exp(scale * acc - top[x]);"),
    "bwd_rows_key_range": ("if (t < lo || t > hi)", "if (t < lo)"),
    "bwd_rows_ignores_left_window": ("if (t < lo || t > hi)", "if (t > hi)"),
    # grouped heads and windows
    "kv_head_interleaved": ("return bh / (H / Hkv);", "return bh % Hkv;"),
    "window_left_off_by_one": ("if (wl >= 0 && i - wl > a)\n        a = i - wl;",
                               "if (wl >= 0 && i - wl + 1 > a)\n        a = i - wl + 1;"),
    "window_right_ignored": ("if (wr >= 0 && i + wr < b)\n        b = i + wr;", ""),
    "window_sides_swapped": ("if (wl >= 0 && i - wl > a)", "if (wr >= 0 && i - wr > a)"),
    "bwd_group_not_summed": ("for (int64_t hq = 0; hq < G; ++hq) {\n        for (int64_t i = 0; i < Sq; ++i) {",
                             "for (int64_t hq = G - 1; hq < G; ++hq) {\n        for (int64_t i = 0; i < Sq; ++i) {"),
    # queries and keys of different length
    "empty_row_lse_zero": ("*lse_i = -INFINITY;", "*lse_i = 0.0;"),
    "empty_row_o_one": ("o_i[d] = 0.0;\n        *lse_i = -INFINITY;", "o_i[d] = 1.0;\n        *lse_i = -INFINITY;"),
    "causal_clip_to_first_key": ("? i : Sk - 1;", "? i : 0;"),
    "rows_query_index_mod_sk": ("const int64_t bh = flat / Sq;\n            const int64_t i = flat % Sq;",
                                "const int64_t bh = flat / Sq;\n            const int64_t i = flat % Sk;"),
    "bwd_rows_query_index_mod_sk": ("const int64_t bh = qrows[r] / Sq, t = qrows[r] % Sq;",
                                    "const int64_t bh = qrows[r] / Sq, t = qrows[r] % Sk;"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE, encoding="utf-8") as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert old in source, f"mutation site for {name!r} no longer exists in the oracle source"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(old, new), encoding="utf-8")
    lib = oracle.build(str(src), str(tmp_path / f"lib{name}.so"))
    mutant = oracle.Oracle(lib)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, FloatingPointError) as e:
            failures.append(pin.__name__)
    assert failures, f"mutant {name!r} passed every pin"


def test_unmutated_copy_passes(source, tmp_path):
    src = tmp_path / "same.c"
    src.write_text(source, encoding="utf-8")
    same = oracle.Oracle(oracle.build(str(src), str(tmp_path / "libsame.so")))
    for pin in oracle_pins.ALL_PINS:
        pin(same)
