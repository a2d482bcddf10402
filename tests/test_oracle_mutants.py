"""The pins are strong enough: plant plausible mistakes in a copy of the oracle
source (on the CPU), rebuild it, and check that at least one pin fails for
every planted mistake.  The real oracle is never modified."""
import importlib.util
import os
import subprocess

import pytest

from tests import test_oracle_pins as pins
from tests import test_oracle_quality as quality

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "msa_oracle.c")

# (name, text in the oracle source, planted replacement)
MUTANTS = [
    ("causal bound drops token t", "for (int64_t i = 0; i <= t; ++i) {", "for (int64_t i = 0; i < t; ++i) {"),
    ("block of a token off by one", "const int64_t b = i / block_size;", "const int64_t b = (i + 1) / block_size;"),
    ("ties go to the higher index", "if (best < 0 || S[b] > S[best]) best = b;",
     "if (best < 0 || S[b] >= S[best]) best = b;"),
    ("one block too few", "for (int round = 0; round < top_k - 1; ++round) {",
     "for (int round = 0; round < top_k - 2; ++round) {"),
    ("local block not forced", "out[j] = (int32_t)c; /* the local block",
     "out[j] = (int32_t)(c > 0 ? c - 1 : 0); /* the local block"),
    ("wrong head to group map", "const int g = h / group_size;", "const int g = h % n_groups;"),
    ("softmax scale dropped", "z[n] = scale * dot;", "z[n] = dot;"),
    ("local block not clipped at t", "i < (int64_t)(s[j] + 1) * block_size && i <= t; ++i) {",
     "i < (int64_t)(s[j] + 1) * block_size && i < n_keys; ++i) {"),
    ("index query of the wrong group", "const uint16_t* q = q_idx + (r * n_groups + g) * (int64_t)index_dim;",
     "const uint16_t* q = q_idx + (r * n_groups + (n_groups - 1 - g)) * (int64_t)index_dim;"),
    ("value of the wrong token", "const uint16_t* vi = v + (idx[m] * n_groups + g) * (int64_t)head_dim;",
     "const uint16_t* vi = v + ((idx[m] > 0 ? idx[m] - 1 : 0) * n_groups + g) * (int64_t)head_dim;"),
    ("key dimension transposed", "const uint16_t* ki = k + (i * n_groups + g) * (int64_t)head_dim;",
     "const uint16_t* ki = k + (g * n_keys + i) * (int64_t)head_dim;"),
    ("mass scores skip token t", "for (int64_t i = 0; i < t + 1; ++i) { /* every causal token */",
     "for (int64_t i = 0; i < t; ++i) { /* every causal token */"),
    ("mass not averaged over the group", "mass[i / block_size] += z[i] / denom / group_size;",
     "mass[i / block_size] += z[i] / denom;"),
    ("mass credited to the previous block", "mass[i / block_size] += z[i] / denom / group_size;",
     "mass[i / block_size > 0 ? i / block_size - 1 : 0] += z[i] / denom / group_size;"),
    ("recall ties go to the higher index", "if (!taken[b] && (best < 0 || P[b] > P[best])) best = b;",
     "if (!taken[b] && (best < 0 || P[b] >= P[best])) best = b;"),
    ("KL with the logarithm ratio flipped",
     "if (s[j] >= 0 && P[s[j]] > 0.0) d += P[s[j]] * (log(P[s[j]]) - ((double)S[s[j]] - lse));",
     "if (s[j] >= 0 && P[s[j]] > 0.0) d += P[s[j]] * (((double)S[s[j]] - lse) - log(P[s[j]]));"),
    ("indexer softmax over every causal block instead of the candidates",
     "        if (s[j] >= 0) sum += exp((double)S[s[j]] - smax);",
     "        if (s[j] >= 0) sum += exp((double)S[s[j]] - smax);\n"
     "      for (int64_t b = 0; b <= pos[r] / block_size; ++b) sum += exp((double)S[b] - smax);"),
    ("candidate mass includes tokens after the query",
     "for (int64_t i = (int64_t)s[jj] * block_size; i < (int64_t)(s[jj] + 1) * block_size && i <= t; ++i) {",
     "for (int64_t i = (int64_t)s[jj] * block_size; i < (int64_t)(s[jj] + 1) * block_size && i < n_keys; ++i) {"),
    ("candidate mass not averaged over the group", "mass[blk[m]] += z[m] / denom / group_size;",
     "mass[blk[m]] += z[m] / denom;"),
    ("candidate mass credited to the next slot's block", "blk[n] = s[jj];",
     "blk[n] = s[jj + 1 < top_k && s[jj + 1] >= 0 ? jj + 1 : jj];"),
    ("coverage misses the last selected block", "for (int j = 0; j < top_k; ++j)\n          if (s[j] >= 0) cov += P[s[j]];",
     "for (int j = 0; j + 1 < top_k; ++j)\n          if (s[j] >= 0) cov += P[s[j]];"),
]

PINS = [
    pins.test_hand_worked_example,
    lambda o: pins.test_pooled_scores_equal_integer_arithmetic(o, 1, 37, 4, 8, 2),
    lambda o: pins.test_selection_equals_dominance_brute_force(o, 0),
    lambda o: pins.test_selection_invariants(o, 8, 4, 200),
    pins.test_ties_go_to_lowest_index,
    pins.test_planted_equal_maxima,
    lambda o: pins.test_short_context_is_dense_attention(o, 4, 3, 12, 4, 1, 8),
    lambda o: pins.test_short_context_is_dense_attention(o, 128, 16, 300, 4, 2, 16),
    pins.test_sparse_rows_equal_dense_attention_over_selected_tokens,
    lambda o: quality.test_block_mass_is_attention_with_block_indicator_values(o, 0, 300, 16, 4, 2, 32),
    quality.test_block_mass_sums_to_one_and_stops_at_the_local_block,
    quality.test_coverage_and_recall_against_sorting,
    quality.test_all_blocks_selected_covers_everything,
    quality.test_kl_hand_example,
    quality.test_kl_vanishes_when_the_indexer_matches_and_is_nonnegative,
    quality.test_selected_mass_hand_example,
    lambda o: quality.test_selected_mass_is_attention_over_the_selection(o, 7, 700, 16, 5, 6, 2, 32),
]


def _mutant_module(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    path_c = tmp_path / "mutant.c"
    path_c.write_text(src.replace(old, new))
    path_so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(path_c), "-o", str(path_so), "-lm"],
                   check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{abs(hash(name))}", os.path.join(ROOT, "oracle",
                                                                                                  "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB_PATH = str(path_so)
    mod._lib = None
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    mod = _mutant_module(tmp_path, name, old, new)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError):
            caught.append(getattr(pin, "__name__", "lambda"))
    assert caught, f"no pin detects the planted mistake: {name}"
