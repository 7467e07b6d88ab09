"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/oracle.c (on the CPU, in a
temporary directory), builds it, runs every pin against it and expects at
least one pin to fail. The real oracle passes all of them (test_oracle_pins.py).
"""
import os

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement); every occurrence of the text is replaced
MUTANTS = [
    ("relu_dropped", "if (dot < 0) dot = 0;", ""),
    ("relu_wrong_side", "if (dot < 0) dot = 0;", "if (dot > 0) dot = 0;"),
    ("weight_of_head0", "acc += (int64_t)w[h] * dot;", "acc += (int64_t)w[0] * dot;"),
    ("key_row_shift", "(int64_t)kI[s * d_I + j]", "(int64_t)kI[(s > 0 ? s - 1 : 0) * d_I + j]"),
    ("query_head_fixed", "(int64_t)qI[h * d_I + j]", "(int64_t)qI[j]"),
    ("smallest_first", "return a->score > b->score ? -1 : 1;",
     "return a->score < b->score ? -1 : 1;"),
    ("tie_higher_index", "    return (a->pos > b->pos) - (a->pos < b->pos);\n}\n\nstatic int orc_cmp_pos",
     "    return (a->pos < b->pos) - (a->pos > b->pos);\n}\n\nstatic int orc_cmp_pos"),
    ("output_in_rank_order", "qsort(pr, (size_t)m, sizeof(orc_pair), orc_cmp_pos);", ""),
    ("causal_excludes_self", "orc_topk_row(S, p + 1, K, ir, sr);", "orc_topk_row(S, p, K, ir, sr);"),
    ("causal_scores_exclude_self", "rc |= orc_score_row(H_I, d_I, qI, kI, wr, p + 1, S + r * (int64_t)Tk);",
     "rc |= orc_score_row(H_I, d_I, qI, kI, wr, p, S + r * (int64_t)Tk);"),
    ("no_softmax_scale", "logit[t] = scale * dot;", "logit[t] = dot;"),
    ("gqa_modulo", "int g = h / G;", "int g = h % Hkv;"),
    ("keys_as_values", "o[j] += e * ld(v, ", "o[j] += e * ld(k, "),
    ("no_normalisation", "o[j] /= Z;", ""),
    ("gate_sign", "exp(-G)", "exp(G)"),
    ("gate_dropped", "return s * o + ", "return o + "),
    ("mix_weight_swapped", "(1.0 - s) * orc_bf16(mix[j])", "s * orc_bf16(mix[j])"),
    ("mix_of_head0", "mix ? mix + (size_t)h * d : NULL", "mix"),
    ("empty_row_not_mixed", "            if (lse) lse[h] = -INFINITY;\n        } else {",
     "            if (lse) lse[h] = -INFINITY;\n            continue;\n        } else {"),
    ("invalid_row_not_mixed", "mix ? mix + qrow * Hq * d : NULL, j)", "NULL, j)"),
    ("layer_drops_mix", "NULL, mix ? mix + qrow * Hq * d : NULL, scale,\n                     orow",
     "NULL, NULL, scale,\n                     orow"),
    ("lse_without_max", "lse[h] = m + log(Z);", "lse[h] = log(Z);"),
    ("padding_read_as_position0", "if (s < 0 || s >= kv_len)", "if (s < 0) s = 0; if (s >= kv_len)"),
    ("append_off_by_one", "int64_t dst = old + t;", "int64_t dst = old + t + 1;"),
    ("append_ignores_count", "for (int64_t t = 0; t < n; ++t) {", "for (int64_t t = 0; t < Tn; ++t) {"),
    ("append_length_not_advanced", "kv_len_out[b] = (int32_t)(old + n < Tk ? old + n : Tk);",
     "kv_len_out[b] = (int32_t)old;"),
    ("append_offset_is_new_length", "q_offset_out[b] = (int32_t)old;",
     "q_offset_out[b] = (int32_t)(old + n);"),
    ("append_no_capacity_clamp", "(int32_t)(old + n < Tk ? old + n : Tk)", "(int32_t)(old + n)"),
    ("block_score_min", "if (S[s] > m) m = S[s];", "if (m == INT32_MIN || S[s] < m) m = S[s];"),
    ("block_expand_not_causal", "(s >= 0 && s < n) ? (int32_t)s : -1;", "(s >= 0) ? (int32_t)s : -1;"),
    ("block_index_unscaled", "(int64_t)bi[kk] * block + t", "(int64_t)bi[kk] + t"),
    ("layer_ignores_blocks", "if (bl > 1)\n                orc_block_topk_row",
     "if (0)\n                orc_block_topk_row"),
    ("sets_share_group0_heads", "const int8_t *qI = q_idx + (((int64_t)b * Tq + i) * H_I + (int64_t)gs * Hg) * d_I;",
     "const int8_t *qI = q_idx + ((int64_t)b * Tq + i) * H_I * d_I;"),
    ("sets_share_group0_weights", "wr + gs * Hg, p + 1, S);", "wr, p + 1, S);"),
    ("heads_read_set0", "const int32_t *ih = idx + (int64_t)(h / hps) * K;",
     "const int32_t *ih = idx;"),
    ("sets_by_kv_head", "const int32_t *ih = idx + (int64_t)(h / hps) * K;",
     "const int32_t *ih = idx + (int64_t)(g * sets / Hkv < sets ? g * sets / Hkv : 0) * K;"),
    ("sets_by_head_modulo", "const int32_t *ih = idx + (int64_t)(h / hps) * K;",
     "const int32_t *ih = idx + (int64_t)(h % sets) * K;"),
    ("bwd_no_delta", "double dl = P[t] * (dP[t] - delta);", "double dl = P[t] * dP[t];"),
    ("bwd_heads_read_set0", "const int32_t *ir = idx + (row * ns + h / hps) * K;",
     "const int32_t *ir = idx + row * ns * K;"),
    ("bwd_gate_derivative", "gy * (o[j] - x) * sg * (1.0 - sg)", "gy * (o[j] - x) * sg * (1.0 + sg)"),
    ("bwd_dk_unscaled", "dkr[j] += scale * dl * orc_bf16(q[hb + j]);", "dkr[j] += dl * orc_bf16(q[hb + j]);"),
    ("bwd_dv_ungated", "dvr[j] += P[t] * dO[j];", "dvr[j] += P[t] * orc_bf16(dy[hb + j]);"),
    ("bwd_dq_from_values", "dq[hb + j] += scale * dl * orc_bf16(kb[", "dq[hb + j] += scale * dl * orc_bf16(vb["),
    ("history_clamped_to_allocation", "kv_len[b] <= Tk ? kv_len[b] : 0", "kv_len[b] < Tk ? kv_len[b] : Tk"),
    ("ibwd_relu_mask_dropped", "                    if (d <= 0) continue;\n", ""),
    ("ibwd_no_tau", "double g = tau * (pt * Tsum - Tr[t]);", "double g = (pt * Tsum - Tr[t]);"),
    ("ibwd_sets_heads_of_group0", "const int8_t *qI = q_idx + (row * H_I + (int64_t)gs * Hs) * d_I;",
     "const int8_t *qI = q_idx + row * H_I * d_I;"),
    ("ibwd_sets_weights_of_group0", "(int64_t)i * w_stride_q + gs * Hs;", "(int64_t)i * w_stride_q;"),
    ("ibwd_sets_rows_of_set0", "int64_t srow = ((int64_t)b * ns + gs) * Tq + i;",
     "int64_t srow = (int64_t)b * ns * Tq + i;"),
    ("ibwd_sign", "double g = tau * (pt * Tsum - Tr[t]);", "double g = tau * (Tr[t] - pt * Tsum);"),
    ("ibwd_teacher_mass_ignored", "double g = tau * (pt * Tsum - Tr[t]);", "double g = tau * (pt - Tr[t]);"),
    ("ibwd_dk_without_weight", "dkr[j] += g * (double)wr[h] * (double)qI[h * d_I + j];",
     "dkr[j] += g * (double)qI[h * d_I + j];"),
    ("ibwd_dw_without_relu", "dwr[h] += g * (double)(d > 0 ? d : 0);", "dwr[h] += g * (double)d;"),
    ("ibwd_entries_past_p", "if (s < 0 || s > p) { z[t] = -INFINITY; continue; }",
     "if (s < 0) { z[t] = -INFINITY; continue; }"),
    ("overflow_unchecked", "if (acc > INT32_MAX) { acc = INT32_MAX; rc = ORC_OVERFLOW; }", ""),
]


def test_mutant_table_applies():
    text = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert text.count(old) >= 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(text.replace(old, new))
    lib = oracle.compile_source(str(src), str(tmp_path / f"liboracle_{name}.so"))
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except Exception:          # a failing assertion, or a crash of the mutant's output
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name!r}"
