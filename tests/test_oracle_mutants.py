"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
its pins catch every one.  Shows the pins constrain the oracle rather than
restate it."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ulys_oracle.c")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("drop_scale", "scores[j] = acc * scale;", "scores[j] = acc;"),
    ("causal_excludes_diagonal", "J->causal ? t + 1 : J->s", "J->causal ? t : J->s"),
    ("gqa_round_robin", "const int64_t g = i / (nq / nkv);\n  const int64_t nkeys = J->causal",
     "const int64_t g = i % nkv;\n  const int64_t nkeys = J->causal"),
    ("no_max_shift_in_lse", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("drop_normalisation", "o_row[e] /= l;", "o_row[e] /= 1.0;"),
    ("k_row_uses_query_head", "const double *krow = J->k + ((j * b + be) * nkv + g) * d;\n    double acc",
     "const double *krow = J->k + ((j * b + be) * nkv + (i % nkv)) * d;\n    double acc"),
    ("pack_heads_strided", "int64_t xi = ((t * b + be) * h + (r * hp + k)) * d + e;\n"
     "            memcpy(dst + yi * elt",
     "int64_t xi = ((t * b + be) * h + (k * P + r)) * d + e;\n"
     "            memcpy(dst + yi * elt"),
    ("seq2head_rank_major_tokens", "int64_t tg = j * sl + t; /* position",
     "int64_t tg = t * P + j; /* position"),
    ("unpack_swaps_groups", "int64_t xi = ((t * b + be) * h + (r * hp + k)) * d + e;\n"
     "            int64_t yi = (((r * sl + t) * b + be) * hp + k) * d + e;\n"
     "            memcpy(dst + xi",
     "int64_t xi = ((t * b + be) * h + ((P - 1 - r) * hp + k)) * d + e;\n"
     "            int64_t yi = (((r * sl + t) * b + be) * hp + k) * d + e;\n"
     "            memcpy(dst + xi"),
    ("bf16_widen_wrong_shift", "<< 16;", "<< 15;"),
    # backward
    ("bwd_drop_scale_dq", "dqrow[e] += ds * krow[e] * scale;\n            dkrow[e]",
     "dqrow[e] += ds * krow[e];\n            dkrow[e]"),
    ("bwd_drop_D", "const double ds = p[j] * (dp[j] - D);\n          const double *krow = J->k",
     "const double ds = p[j] * dp[j];\n          const double *krow = J->k"),
    ("bwd_dv_uses_ds", "dvrow[e] += p[j] * drow[e];\n          }\n        }\n      }\n    }\n  }\n"
     "  free(p); free(dp);\n  J->status = ORC_OK;\n  return NULL;\n}\n\n/*\n * Merge of",
     "dvrow[e] += ds * drow[e];\n          }\n        }\n      }\n    }\n  }\n"
     "  free(p); free(dp);\n  J->status = ORC_OK;\n  return NULL;\n}\n\n/*\n * Merge of"),
    ("bwd_gqa_first_head_only",
     "for (int64_t i = g * G; i < (g + 1) * G; ++i) {\n      for (int64_t t = 0; t < s; ++t) {",
     "for (int64_t i = g * G; i < g * G + 1; ++i) {\n      for (int64_t t = 0; t < s; ++t) {"),
    ("bwd_dp_shifted_feature", "for (int64_t e = 0; e < d; ++e) acc += drow[e] * vrow[e];",
     "for (int64_t e = 0; e < d; ++e) acc += drow[e] * vrow[(e + 1) % d];"),
    ("bwd_rows_causal_skips_diagonal", "for (int64_t t = J->causal ? j : 0; t < s; ++t) {",
     "for (int64_t t = J->causal ? j + 1 : 0; t < s; ++t) {"),
    ("bwd_dk_uses_dout", "dqrow[e] += ds * krow[e] * scale;\n            dkrow[e] += ds * qrow[e] * scale;",
     "dqrow[e] += ds * krow[e] * scale;\n            dkrow[e] += ds * drow[e] * scale;"),
    # KV replication and its backward
    ("pack_kv_strided_heads", "const int64_t g = r * h_kv / P; /* the KV head",
     "const int64_t g = r % h_kv; /* the KV head"),
    ("unpack_kv_sum_drops_a_copy", "for (int64_t r = g * R; r < (g + 1) * R; ++r) /* the ranks",
     "for (int64_t r = g * R; r < (g + 1) * R - 1; ++r) /* the ranks"),
    ("round_bf16_truncates", "q = ldexp(nearbyint(ldexp(m, 8)), e - 8);",
     "q = ldexp(floor(ldexp(m, 8)), e - 8);"),
    # merge of partial attention results
    ("merge_drops_max_in_lse", "lse[li] = m + log(l);", "lse[li] = log(l);"),
    ("merge_swaps_weights", "o[oi + e] = (ea * o_a[oi + e] + eb * o_b[oi + e]) / l;",
     "o[oi + e] = (eb * o_a[oi + e] + ea * o_b[oi + e]) / l;"),
    ("merge_skips_normalisation", "o[oi + e] = (ea * o_a[oi + e] + eb * o_b[oi + e]) / l;",
     "o[oi + e] = (ea * o_a[oi + e] + eb * o_b[oi + e]);"),
    ("merge_lse_row_transposed", "const int64_t li = (be * hp + i) * s + t;",
     "const int64_t li = (t * b + be) * hp + i;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mutated = tmp_path / f"oracle_{name}.c"
    mutated.write_text(src.replace(old, new), encoding="utf-8")
    so = tmp_path / f"liboracle_{name}.so"
    oracle.build(str(mutated), str(so))
    lib = oracle.load(str(so))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"


def test_unmutated_copy_passes(tmp_path):
    so = tmp_path / "liboracle_copy.so"
    oracle.build(SRC, str(so))
    lib = oracle.load(str(so))
    for pin in oracle_pins.ALL_PINS:
        pin(lib)
