"""Plants one mistake at a time in a copy of the oracle's source, on the CPU,
and checks that at least one pin catches it. This shows the pins would catch
a dropped term, a wrong sign, index or operand in the oracle itself."""
import os

import pytest

import oracle
import oracle_pins as pins

# (name, text in msa_oracle.c, replacement)
MUTANTS = [
    ("diagonal_key_dropped",
     "j <= p && j < (blk + 1) * S; ++j) keys[n++] = j;\n        const uint16_t *k_grp",
     "j < p && j < (blk + 1) * S; ++j) keys[n++] = j;\n        const uint16_t *k_grp"),
    ("backward_diagonal_key_dropped",
     "j <= p && j < (blk + 1) * S; ++j) keys[n++] = j;\n        if (n == 0) continue;",
     "j < p && j < (blk + 1) * S; ++j) keys[n++] = j;\n        if (n == 0) continue;"),
    ("pool_starts_at_zero", "double m = s[lo];", "double m = 0.0;"),
    ("pool_sums", "if (s[j] > m) m = s[j];", "m += s[j];"),
    ("ties_to_higher_block", "return (x->block > y->block) - (x->block < y->block);",
     "return (x->block < y->block) - (x->block > y->block);"),
    ("ascending_scores", "if (x->score > y->score) return -1;\n    if (x->score < y->score) return 1;",
     "if (x->score > y->score) return 1;\n    if (x->score < y->score) return -1;"),
    ("no_softmax_scale", "z[a] = tau * acc;", "z[a] = acc;"),
    ("lse_without_max", "*lse_head = m + log(l);", "*lse_head = log(l);"),
    ("unnormalised_weights", "double w = exp(z[a] - m) / l;", "double w = exp(z[a] - m);"),
    ("interleaved_heads", "int h = g * R + r;", "int h = r * G + g;"),
    ("wrong_group_index_query", "index_elem(cfg, q_idx_row, (int64_t)g * dI + c)",
     "index_elem(cfg, q_idx_row, (int64_t)((g + 1) % G) * dI + c)"),
    ("e4m3_bias_8", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("zero_padding", "sel[g * K + k] = -1;", "sel[g * K + k] = 0;"),
    ("bf16_shift", "v.u = (uint32_t)bits << 16;", "v.u = (uint32_t)bits << 15;"),
    ("ignores_q_start", "int64_t p = (int64_t)w->q_start[b] + i;", "int64_t p = i;"),
    ("v_of_group0", "const uint16_t *v_grp = v_seq + (int64_t)g * n_stride * d;",
     "const uint16_t *v_grp = v_seq;"),
    ("k_of_group0", "const uint16_t *k_grp = k_seq + (int64_t)g * n_stride * d;",
     "const uint16_t *k_grp = k_seq;"),
    ("qblock_min_over_rows", "if (row[g * nv + beta] > best[g * n_valid + beta])",
     "if (row[g * nv + beta] < best[g * n_valid + beta])"),
    ("qblock_first_row_only", "for (int64_t i = i_lo; i <= i_hi; ++i) {",
     "for (int64_t i = i_lo; i <= i_lo; ++i) {"),
    ("qblock_slot_from_zero", "const int64_t qb = q_start / S + slot;",
     "const int64_t qb = slot;"),
    ("backward_no_delta", "const double ds = P[a] * (dP[a] - delta);",
     "const double ds = P[a] * dP[a];"),
    ("backward_dv_unweighted", "dv_grp[j * d + c] += P[a] * oracle_bf16_value(doh[c]);",
     "dv_grp[j * d + c] += oracle_bf16_value(doh[c]);"),
    ("backward_dk_no_scale", "dk_grp[j * d + c] += tau * ds * oracle_bf16_value(qh[c]);",
     "dk_grp[j * d + c] += ds * oracle_bf16_value(qh[c]);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation site not unique: " + name
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(force=True, source=str(path), out=str(tmp_path / "libmutant.so"))
    failures = pins.run_all(oracle.Oracle(lib))
    assert failures, "no pin caught mutant " + name
