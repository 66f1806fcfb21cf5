"""Plant plausible mistakes in copies of the oracle source (on the CPU) and
require that the pin suite catches each one.  This measures the pins'
power: a pin suite that a dropped term, a wrong sign or index, or a
transposed operand could pass would not be a pin."""
import os
import subprocess
import tempfile

import pytest

import oracle_pins
from oracle import oracle as O

MUTANTS = [
    ("relu_dropped", "if (dot > 0.0)\n                    acc +=", "if (1)\n                    acc +="),
    ("relu_after_weight", "if (dot > 0.0)\n                    acc +=", "if ((double)w[h] * dot > 0.0)\n                    acc +="),
    ("key_index_shifted", "idx_value(k[d], idx_f16);", "idx_value(k[(d + 1) % d_idx], idx_f16);"),
    ("head_stride_wrong", "idx_value(qi[h * d_idx + d], idx_f16)", "idx_value(qi[h + d], idx_f16)"),
    ("rows_off_by_one", "const int64_t rows = q_nvis[q] / kpool;", "const int64_t rows = (q_nvis[q] - 1) / kpool;"),
    ("seq_ignored_in_scores", "const int64_t seq = q_seq ? q_seq[q] : q;", "const int64_t seq = 0;"),
    ("ties_to_higher_index", "return (a->r > b->r) - (a->r < b->r);", "return (a->r < b->r) - (a->r > b->r);"),
    ("ascending_sort_dropped", "qsort(pick, (size_t)keep, sizeof *pick, by_index);", ";"),
    ("tail_dropped", "for (int64_t t = rows * kpool; t < n_vis; t++)", "for (int64_t t = rows * kpool; t < rows * kpool; t++)"),
    # ("rows < keep" would be an equivalent mutant: keeping keep of keep rows is dense)
    ("dense_one_past_budget", "if (rows <= keep) {", "if (rows <= keep + 1) {"),
    ("keep_one_short", "for (int64_t i = 0; i < keep; i++)\n                pick[i] = all[i].r;",
     "for (int64_t i = 0; i < keep; i++)\n                pick[i] = all[i + (i == keep - 1)].r;"),
    ("scale_dropped", "z[i] = (double)scale * dot;", "z[i] = dot;"),
    ("rope_dropped", "for (int32_t d = 0; d < D; d++)\n                    dot += bf16_value(qh[d])",
     "for (int32_t d = 0; d < d_latent; d++)\n                    dot += bf16_value(qh[d])"),
    ("v_from_rope_side", "o[j] += p * bf16_value(c[j]);", "o[j] += p * bf16_value(c[j + d_rope]);"),
    ("not_normalised", "dst[j] = (float)(o[j] / l);", "dst[j] = (float)o[j];"),
    ("lse_without_max", "(float)(m + log(l));", "(float)log(l);"),
    ("query_head_transposed", "q + ((int64_t)qq * n_heads + h) * D;", "q + ((int64_t)h * n_q + qq) * D;"),
    ("seq_ignored_in_attend", "const int64_t seq = q_seq ? q_seq[qq] : qq;", "const int64_t seq = 0;"),
    ("pool_expand_wrong", "dst[count++] = (int32_t)(pick[i] * kpool + j);", "dst[count++] = (int32_t)(pick[i] + j);"),
    ("pool_no_position_embedding", "+ (double)pos_emb[j * d_idx + d];", "+ 0.0;"),
    ("pool_position_slot_reversed", "(double)pos_emb[j * d_idx + d];", "(double)pos_emb[(3 - j) * d_idx + d];"),
    ("pool_one_logit_per_slot", "a[j] = bf16_value(c[j][d_idx + d]) + (double)pos_emb[j * d_idx + d];",
     "a[j] = bf16_value(c[j][d_idx]) + (double)pos_emb[j * d_idx];"),
    ("pool_gate_as_value", "num += e * bf16_value(c[j][d]);", "num += e * bf16_value(c[j][d_idx + d]);"),
    ("pool_not_normalised", "out[d] = bf16_from_double(num / den);", "out[d] = bf16_from_double(num / 4.0);"),
    ("pool_complete_on_slot_0", "if (slot == 3) {", "if (slot == 0) {"),
    ("pool_index_off", "t / 4) * d_idx);", "(t / 4 + (t >= 8))) * d_idx);"),
    ("pool_round_truncates", "const double r = rint(ldexp(m, 8));", "const double r = trunc(ldexp(m, 8));"),
    ("absorb_weight_transposed", "bf16_value(W[(int64_t)k * d_latent + n]);", "bf16_value(W[(int64_t)n * d_nope + k]);"),
    ("absorb_last_term_dropped", "for (int32_t k = 0; k < d_nope; k++)\n                    acc += bf16_value(qn[k])",
     "for (int32_t k = 0; k < d_nope - 1; k++)\n                    acc += bf16_value(qn[k])"),
    ("absorb_rope_dropped", "dst[d_latent + r] = q_rope[((int64_t)m * n_heads + h) * d_rope + r];", "dst[d_latent + r] = 0;"),
    ("absorb_wrong_head_weight", "const uint16_t *W = w_uk + (int64_t)h * d_nope * d_latent;", "const uint16_t *W = w_uk;"),
    ("project_weight_transposed", "bf16_value(W[(int64_t)i * d_latent + j]);", "bf16_value(W[(int64_t)j * d_v + i]);"),
    ("project_wrong_head_weight", "const uint16_t *W = w_uv + (int64_t)h * d_v * d_latent;", "const uint16_t *W = w_uv;"),
    ("project_half_the_latent", "for (int32_t j = 0; j < d_latent; j++)\n                    acc += (double)oh[j]",
     "for (int32_t j = 0; j < d_latent / 2; j++)\n                    acc += (double)oh[j]"),
    ("f16_keys_read_as_bf16", "idx_value(k[d], idx_f16);", "idx_value(k[d], 0);"),
    ("f16_decode_bias", "else v = ldexp((double)(1024 + f), e - 25);", "else v = ldexp((double)(1024 + f), e - 24);"),
    ("prep_rotation_unscaled", "y[i] = acc * norm;", "y[i] = acc;"),
    ("prep_hadamard_sign_pattern", "__builtin_popcount((unsigned)(i & j))", "__builtin_popcount((unsigned)(i | j))"),
    ("prep_rope_on_head", "const int32_t o = d_idx - d_rope;", "const int32_t o = 0;"),
    ("prep_rope_neox_pairs", "const double a = x[o + 2 * j], b = x[o + 2 * j + 1];",
     "const double a = x[o + j], b = x[o + j + d_rope / 2];"),
    ("prep_rope_not_a_rotation", "r[o + 2 * j] = a * cos(t) - b * sin(t);", "r[o + 2 * j] = a * cos(t) + b * sin(t);"),
    ("prep_rope_clockwise", "r[o + 2 * j] = a * cos(t) - b * sin(t);\n        r[o + 2 * j + 1] = a * sin(t) + b * cos(t);",
     "r[o + 2 * j] = a * cos(t) + b * sin(t);\n        r[o + 2 * j + 1] = -a * sin(t) + b * cos(t);"),
    ("prep_rope_frequency_exponent", "pow(base, -2.0 * j / d_rope)", "pow(base, -2.0 * j / (d_rope - 2))"),
    ("prep_query_position_off", "pos = (int64_t)q_nvis[v / n_idx_heads] - 1;", "pos = (int64_t)q_nvis[v / n_idx_heads];"),
    ("prep_key_row_transposed", "dst = k_cache + (seq * key_seq_stride + pos) * d_idx;",
     "dst = k_cache + (pos * n_seq + seq) * d_idx;"),
    ("prep_f16_truncates", "double r = rint(ldexp(m, 11));", "double r = trunc(ldexp(m, 11));"),
    ("prep_f16_subnormal_scale", "return sign | (uint16_t)rint(ldexp(a, 24));", "return sign | (uint16_t)rint(ldexp(a, 25));"),
]


def _build_mutant(src: str, name: str, old: str, new: str, tmp: str) -> str:
    assert old in src, f"mutant {name}: pattern not found"
    path_c = os.path.join(tmp, f"{name}.c")
    path_so = os.path.join(tmp, f"lib{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-o", path_so, path_c, "-lm"])
    return path_so


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(O.SRC).read()
    with tempfile.TemporaryDirectory() as tmp:
        L = O.load(_build_mutant(src, name, old, new, tmp))
        failed = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(L)
            except AssertionError:
                failed.append(pin.__name__)
            except Exception as e:   # a crash or a refused call also counts
                failed.append(f"{pin.__name__}: {type(e).__name__}")
        assert failed, f"mutant {name} passed every pin"
