/*
 * oracle_driver.c — runs every function of oracle/msa_oracle.c on small
 * seeded problems, valid and invalid, so that a build with
 * -fsanitize=address,undefined reports any out-of-bounds access, use of
 * uninitialised memory or undefined behaviour in the oracle.  Test
 * infrastructure: built and run by tests/test_sanitizers.py.  Exit status 0
 * iff every call returned what it should and the results pass basic checks.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int msa_oracle_block_scores(int64_t, const int64_t*, const uint16_t*, int, int, const uint16_t*, int64_t, int, float*,
                            int64_t);
int msa_oracle_select(int64_t, const int64_t*, const float*, int, int64_t, int, int, int32_t*);
int msa_oracle_attend(int64_t, const int64_t*, const uint16_t*, int, int, int, const uint16_t*, const uint16_t*,
                      int64_t, const int32_t*, int, int, double, double*);
int msa_oracle_block_mass(int64_t, const int64_t*, const uint16_t*, int, int, int, const uint16_t*, int64_t, int, double,
                          double*, int64_t);
int msa_oracle_selection_quality(int64_t, const int64_t*, const double*, const int32_t*, int, int64_t, int, int,
                                 double*, double*);
int msa_oracle_selected_mass(int64_t, const int64_t*, const uint16_t*, int, int, int, const uint16_t*, int64_t,
                             const int32_t*, int, int, double, double*, int64_t);
int msa_oracle_indexer_kl(int64_t, const int64_t*, const double*, const float*, const int32_t*, int, int64_t, int, int,
                          double*);
void msa_oracle_set_num_threads(int);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static uint16_t bf16_of(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}
static uint16_t dyadic(void) { return bf16_of((float)((int)(next_u64() % 9) - 4) / 4.0f); }
static uint16_t normalish(void) { return bf16_of((float)((double)(next_u64() % 20001) / 5000.0 - 2.0)); }

static int failures = 0;
#define CHECK(cond, what)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "oracle_driver: %s failed\n", what); \
      ++failures;                                          \
    }                                                      \
  } while (0)

static void run_case(int64_t length, int groups, int hq, int d, int di, int bs, int top_k, int64_t n_rows) {
  const int64_t ld = (length - 1) / bs + 1;
  uint16_t* k_idx = malloc(sizeof(uint16_t) * length * di);
  uint16_t* q_idx = malloc(sizeof(uint16_t) * (n_rows ? n_rows : 1) * groups * di);
  uint16_t* q = malloc(sizeof(uint16_t) * (n_rows ? n_rows : 1) * hq * d);
  uint16_t* k = malloc(sizeof(uint16_t) * length * groups * d);
  uint16_t* v = malloc(sizeof(uint16_t) * length * groups * d);
  int64_t* pos = malloc(sizeof(int64_t) * (n_rows ? n_rows : 1));
  float* pooled = malloc(sizeof(float) * (n_rows ? n_rows : 1) * groups * ld);
  int32_t* sel = malloc(sizeof(int32_t) * (n_rows ? n_rows : 1) * groups * top_k);
  double* out = malloc(sizeof(double) * (n_rows ? n_rows : 1) * hq * d);
  double* mass = malloc(sizeof(double) * (n_rows ? n_rows : 1) * groups * ld);
  double* smass = malloc(sizeof(double) * (n_rows ? n_rows : 1) * groups * ld);
  double* cov = malloc(sizeof(double) * (n_rows ? n_rows : 1) * groups);
  double* rec = malloc(sizeof(double) * (n_rows ? n_rows : 1) * groups);
  double* kl = malloc(sizeof(double) * (n_rows ? n_rows : 1) * groups);
  for (int64_t i = 0; i < length * di; ++i) k_idx[i] = dyadic();
  for (int64_t i = 0; i < n_rows * groups * di; ++i) q_idx[i] = dyadic();
  for (int64_t i = 0; i < n_rows * hq * d; ++i) q[i] = normalish();
  for (int64_t i = 0; i < length * groups * d; ++i) k[i] = normalish(), v[i] = normalish();
  for (int64_t r = 0; r < n_rows; ++r) pos[r] = r == 0 ? 0 : r == n_rows - 1 ? length - 1 : (int64_t)(next_u64() % length);
  const double scale = 1.0 / sqrt((double)d);

  CHECK(msa_oracle_block_scores(n_rows, pos, q_idx, groups, di, k_idx, length, bs, pooled, ld) == 0, "block_scores");
  CHECK(msa_oracle_select(n_rows, pos, pooled, groups, ld, bs, top_k, sel) == 0, "select");
  for (int64_t r = 0; r < n_rows; ++r)
    for (int g = 0; g < groups; ++g) {
      const int32_t* s = sel + (r * groups + g) * top_k;
      int last = -1, n = 0;
      for (int j = 0; j < top_k; ++j)
        if (s[j] >= 0) {
          CHECK(s[j] > last && s[j] <= pos[r] / bs, "selection ascending and causal");
          last = s[j];
          ++n;
        }
      const int64_t want = pos[r] / bs + 1 < top_k ? pos[r] / bs + 1 : top_k;
      CHECK(n == want && last == pos[r] / bs, "selection size and local block");
    }
  CHECK(msa_oracle_attend(n_rows, pos, q, hq, groups, d, k, v, length, sel, bs, top_k, scale, out) == 0, "attend");
  for (int64_t i = 0; i < n_rows * hq * d; ++i) CHECK(isfinite(out[i]), "finite output");
  CHECK(msa_oracle_block_mass(n_rows, pos, q, hq, groups, d, k, length, bs, scale, mass, ld) == 0, "block_mass");
  CHECK(msa_oracle_selection_quality(n_rows, pos, mass, sel, groups, ld, bs, top_k, cov, rec) == 0, "quality");
  CHECK(msa_oracle_selected_mass(n_rows, pos, q, hq, groups, d, k, length, sel, bs, top_k, scale, smass, ld) == 0,
        "selected_mass");
  CHECK(msa_oracle_indexer_kl(n_rows, pos, smass, pooled, sel, groups, ld, bs, top_k, kl) == 0, "indexer_kl");
  for (int64_t i = 0; i < n_rows * groups; ++i) {
    CHECK(cov[i] >= -1e-12 && cov[i] <= 1 + 1e-12 && rec[i] >= 0 && rec[i] <= 1, "coverage and recall in [0,1]");
    CHECK(kl[i] >= -1e-9, "KL non-negative");
  }
  /* Rejected arguments: a position past the keys, a selection that is not causal. */
  if (n_rows > 0) {
    const int64_t saved = pos[0];
    pos[0] = length;
    CHECK(msa_oracle_block_scores(n_rows, pos, q_idx, groups, di, k_idx, length, bs, pooled, ld) == 1, "bad position");
    CHECK(msa_oracle_attend(n_rows, pos, q, hq, groups, d, k, v, length, sel, bs, top_k, scale, out) == 1,
          "bad position (attend)");
    pos[0] = saved;
    const int32_t s0 = sel[0];
    sel[0] = (int32_t)(pos[0] / bs + 1);
    CHECK(msa_oracle_attend(n_rows, pos, q, hq, groups, d, k, v, length, sel, bs, top_k, scale, out) == 2,
          "non-causal selection");
    CHECK(msa_oracle_selected_mass(n_rows, pos, q, hq, groups, d, k, length, sel, bs, top_k, scale, smass, ld) == 2,
          "non-causal selection (mass)");
    sel[0] = s0;
  }
  free(k_idx), free(q_idx), free(q), free(k), free(v), free(pos), free(pooled), free(sel), free(out), free(mass);
  free(smass), free(cov), free(rec), free(kl);
}

int main(void) {
  msa_oracle_set_num_threads(2);
  run_case(37, 2, 4, 8, 8, 4, 3, 11);      /* tiny blocks, few slots */
  run_case(300, 1, 8, 16, 32, 128, 16, 9); /* fewer causal blocks than slots */
  run_case(700, 3, 6, 32, 64, 16, 5, 13);  /* many blocks per row */
  run_case(129, 2, 2, 8, 16, 128, 16, 0);  /* no rows */
  run_case(1, 1, 1, 4, 8, 128, 16, 1);     /* a single token */
  if (failures) {
    fprintf(stderr, "oracle_driver: %d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle_driver: ok\n");
  return 0;
}
