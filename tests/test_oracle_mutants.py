"""The pins catch plausible mistakes in the oracle (CPU only).

Each case plants one slip into a copy of oracle/attn_oracle.c (a dropped term, a
wrong sign or index, a transposed operand, an off-by-one mask), builds it into a
temporary library, and runs the whole pin battery on it: at least one pin must
fail.  Every planted slip keeps all memory accesses in bounds.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

# (name, text in attn_oracle.c, replacement); each text must occur exactly once.
MUTANTS = [
    ("mask_drops_diagonal", "for (int64_t j = i + 1; j < N; ++j)\n            s[j] = -INFINITY;",
     "for (int64_t j = i; j < N; ++j)\n            s[j] = -INFINITY;"),
    ("mask_upper_triangle", "for (int64_t j = i + 1; j < N; ++j)\n            s[j] = -INFINITY;",
     "for (int64_t j = 0; j < i; ++j)\n            s[j] = -INFINITY;"),
    ("scale_dropped", "s[j] = dot * scale;\n    }\n    /* step 3", "s[j] = dot;\n    }\n    /* step 3"),
    ("scale_divides", "s[j] = dot * scale;\n    }\n    /* step 3", "s[j] = dot / scale;\n    }\n    /* step 3"),
    ("key_row_index", "const double *k_j = k + j * d;", "const double *k_j = k + j;"),
    ("query_used_as_key", "dot += q_i[c] * k_j[c];", "dot += q_i[c] * q_i[c] * k_j[c];"),
    ("dot_drops_last_term", "for (int64_t c = 0; c < d; ++c)\n            dot += q_i[c] * k_j[c];",
     "for (int64_t c = 0; c + 1 < d; ++c)\n            dot += q_i[c] * k_j[c];"),
    ("exp_sign_flipped", "s[j] = exp(s[j] - m); /* s now", "s[j] = exp(m - s[j]); /* s now"),
    ("max_not_subtracted_in_lse", "*lse_i = m + log(l);", "*lse_i = log(l);"),
    ("lse_log2", "*lse_i = m + log(l);", "*lse_i = m + log2(l);"),
    ("not_normalised", "const double p = s[j] / l;", "const double p = s[j];"),
    ("value_row_index", "const double *v_j = v + j * d;", "const double *v_j = v + (N - 1 - j) * d;"),
    ("value_transposed", "o_i[c] += p * v_j[c];", "o_i[c] += p * v[(c % N) * d + (j % d)];"),
    ("max_is_min", "if (s[j] > m)\n            m = s[j];\n\n    for", "if (s[j] < m || m == -INFINITY)\n            m = s[j];\n\n    for"),
    ("sum_skips_first_key", "for (int64_t j = 0; j < N; ++j) {\n        s[j] = exp(s[j] - m);",
     "for (int64_t j = 0; j < N; ++j) {\n        s[j] = exp(s[j] - m) * (j > 0);"),
    ("dense_mask_off_by_one", "if (causal && j > i) s[j] = -INFINITY;", "if (causal && j >= i + 2) s[j] = -INFINITY;"),
    ("dense_not_normalised", "for (int64_t j = 0; j < N; ++j) p[j] /= l;", "for (int64_t j = 0; j < N; ++j) p[j] /= (l + 1e-3);"),
    ("rows_head_offset", "attention_row(q + i * d, k, v, N, d, scale, causal, i, s,",
     "attention_row(q + i * d, k, v, N, d, scale, causal, 0, s,"),
    ("batched_head_offset", "const int64_t base = head * N * d;", "const int64_t base = (head / 2) * N * d;"),
    # backward
    ("bwd_dk_scale_dropped", "dkh[j * d + c] += scale * ds * q_i[c];", "dkh[j * d + c] += ds * q_i[c];"),
    ("bwd_dq_scale_dropped", "dq_i[c] += scale * ds * kh[j * d + c];", "dq_i[c] += ds * kh[j * d + c];"),
    ("bwd_row_term_dropped", "const double ds = P[j] * (dP[j] - D);", "const double ds = P[j] * dP[j];"),
    ("bwd_row_term_unweighted", "D += P[j] * dot;", "D += dot;"),
    ("bwd_dk_uses_key", "dkh[j * d + c] += scale * ds * q_i[c];", "dkh[j * d + c] += scale * ds * kh[j * d + c];"),
    ("bwd_dv_uses_ds", "dvh[j * d + c] += P[j] * do_i[c];", "dvh[j * d + c] += ds * do_i[c];"),
    ("bwd_dp_uses_key", "for (int64_t c = 0; c < d; ++c) dot += do_i[c] * vh[j * d + c];",
     "for (int64_t c = 0; c < d; ++c) dot += do_i[c] * kh[j * d + c];"),
    ("bwd_mask_drops_diagonal", "const int64_t nvis = causal ? i + 1 : N;", "const int64_t nvis = causal ? i : N;"),
    ("bwd_not_normalised", "for (int64_t j = 0; j < nvis; ++j) P[j] /= l;", "for (int64_t j = 0; j < nvis; ++j) P[j] /= (l + 0.5);"),
    ("masked_top_left_causal", "if (causal && j > i + (Nk - Nq))", "if (causal && j > i)"),
    ("masked_bias_subtracted", "s[j] += bias_i[j];", "s[j] -= bias_i[j];"),
    ("masked_bias_ignored", "s[j] += bias_i[j];", "s[j] += 0.0 * bias_i[j];"),
    ("masked_no_safe_softmax", "lse[r] = -INFINITY;\n                continue;", "lse[r] = -INFINITY;"),
    ("masked_strides_swapped", "bias + b * sb + h * sh + i * Nk", "bias + h * sb + b * sh + i * Nk"),
    ("masked_wrong_value_row", "o_i[c] += w * vh[j * d + c];", "o_i[c] += w * vh[c];"),
    ("masked_not_normalised", "const double w = s[j] / l;", "const double w = s[j];"),
    ("masked_diagonal_hidden", "if (causal && j > i + (Nk - Nq))", "if (causal && j >= i + (Nk - Nq))"),
    ("lin_not_causal", "for (int64_t t = 0; t <= j; ++t) {   /* causal: keys t <= j */",
     "for (int64_t t = 0; t < N; ++t) {   /* causal: keys t <= j */"),
    ("lin_strictly_causal", "for (int64_t t = 0; t <= j; ++t) {   /* causal: keys t <= j */",
     "for (int64_t t = 0; t < j + (j == 0); ++t) {   /* causal: keys t <= j */"),
    ("lin_elu_without_one", "return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x : exp(x) - 1.0;"),
    ("lin_eps_dropped", "const double z = 1.0 / (den + eps);", "const double z = 1.0 / den;"),
    ("lin_value_row_of_query", "const double *vt = v + (h * N + t) * M;", "const double *vt = v + (h * N + j) * M;"),
    ("lin_denominator_unmapped", "for (int64_t e = 0; e < E; ++e) den += qj[e] * ksum[e];",
     "for (int64_t e = 0; e < E; ++e) den += q[r * E + e] * ksum[e];"),
    ("lin_feature_map_on_q_only", "fk[x] = feature_map ? elu_plus_one(k[x]) : k[x];", "fk[x] = k[x];"),
    ("bwd_scores_unscaled", "P[j] = dot * scale;\n                    if (P[j] > m) m = P[j];",
     "P[j] = dot;\n                    if (P[j] > m) m = P[j];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = os.path.join(tmp_path, f"mutant_{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(src=path, out=os.path.join(tmp_path, f"libmutant_{name}.so"), werror=False)
    orc = oracle.OracleLib(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, RuntimeError, ValueError) as e:
            caught.append(f"{pin.__name__}: {str(e)[:80]}")
    assert caught, f"no pin caught mutant {name}"
