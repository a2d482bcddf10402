/*
 * msa_oracle.c — plain, slow CPU oracle of MiniMax Sparse Attention (MSA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or helper with the GPU path, and the GPU path never calls it.
 *
 * What it computes, step by step, in the order of the pages:
 *   "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2 (four inference
 *   steps of MSA, and the softmax-attention equation of the same section):
 *     1. score      s_i = Q_idx[t,g] . K_idx[i]  for every causal key i <= t
 *                   (one Q_idx per GQA group, one K_idx per token shared by
 *                   all groups);
 *     2. pool       block score = max of the token scores inside each
 *                   128-token block (only the causal part of the local block);
 *     3. select     16 blocks per query and group, the local block forced in
 *                   as one of them; equal scores go to the lower block index;
 *     4. attend     exact softmax attention over the tokens of those blocks.
 *
 * Precision.  Inputs are bfloat16 bit patterns.  Every bf16 value is exact in
 * double.  Index scores: each product of two bf16 values is exact in double
 * and the sum is formed in double, then rounded once to float, so the score
 * is the correctly rounded exact dot product (for the dyadic inputs the tests
 * use, it is the exact value).  Pooling and selection compare those floats,
 * which is the precision the GPU path decides in.  Attention: dot products,
 * softmax and the weighted sum are all evaluated in double.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - the score is a plain dot product, no scale and no activation;
 *   - block b covers absolute positions [B*b, B*b + B - 1];
 *   - with c + 1 <= top_k causal blocks, every causal block is selected;
 *   - ties in block score go to the lower block index; -0 compares equal
 *     to +0 and is written as +0;
 *   - the softmax scale is given by the caller (1/sqrt(D) by default).
 * block_size and top_k are parameters here (the GPU path fixes 128 and 16)
 * so that tiny exhaustive cases can be checked.
 *
 * Every function processes a list of query rows of ONE sequence whose keys
 * are given in plain logical order (token i at index i), independently of any
 * cache layout.  Rows are independent; OpenMP spreads them over host cores.
 *
 * Selection quality and the indexer's training target (same page, §2: MSA
 * is judged by selection recall and by how much of the attention the chosen
 * blocks cover; in training, the Main Branch forms a group-averaged
 * importance distribution P over the candidate blocks, the indexer predicts a
 * distribution Q, and the two are aligned by D_KL(P||Q)):
 *     5. dense mass  the DENSE causal softmax probabilities of the tokens of
 *                    block b, summed per block and averaged over the group's
 *                    heads (every causal block);
 *     6. quality     coverage = dense mass on the selected blocks; recall =
 *                    the share of the min(top_k, c+1) largest-mass blocks
 *                    (ties to the lower index) that were selected;
 *     7. P           the Main Branch's own softmax (over the tokens of the
 *                    selected blocks only, as in step 4), summed per selected
 *                    block and averaged over the group's heads: P is a
 *                    distribution over the candidate blocks;
 *     8. D_KL(P||Q)  with Q the indexer's distribution over the same
 *                    candidate blocks: the softmax of their pooled index
 *                    scores.
 * Readings (listed in the design notes): coverage and recall use the dense
 * mass, over every causal block including the local one; the KL's P and Q
 * range over the selected blocks; Q uses the raw pooled scores (no
 * temperature); natural logarithms.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_BAD_SEL 2
#define ORACLE_NO_MEMORY 3

/* bfloat16 bit pattern -> double (exact). */
static double bf16_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Threads for the OpenMP loops below (n <= 0 leaves the setting unchanged). */
void msa_oracle_set_num_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

int msa_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Step 1: one index score, the dot product of a query's Q_idx for one group
 * with one token's K_idx. */
static float index_score(const uint16_t* q_idx, const uint16_t* k_idx, int index_dim) {
  double sum = 0.0;
  for (int d = 0; d < index_dim; ++d) sum += bf16_to_double(q_idx[d]) * bf16_to_double(k_idx[d]);
  return (float)sum;
}

/*
 * Steps 1-2 for n_rows query rows.
 *   pos      [n_rows]                      absolute position t of each row
 *   q_idx    [n_rows][n_groups][index_dim] bf16 bits
 *   k_idx    [n_keys][index_dim]           bf16 bits, n_keys > max t
 *   pooled   [n_rows][n_groups][ld]        out: block scores, -inf for b > t/B
 */
int msa_oracle_block_scores(int64_t n_rows, const int64_t* pos, const uint16_t* q_idx, int n_groups,
                            int index_dim, const uint16_t* k_idx, int64_t n_keys, int block_size,
                            float* pooled, int64_t ld) {
  if (n_rows < 0 || n_groups <= 0 || index_dim <= 0 || block_size <= 0 || !pos || !pooled) return ORACLE_BAD_ARG;
  if (n_rows > 0 && (!q_idx || !k_idx)) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (pos[r] < 0 || pos[r] >= n_keys || pos[r] / block_size >= ld) return ORACLE_BAD_ARG;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t t = pos[r];
    for (int g = 0; g < n_groups; ++g) {
      const uint16_t* q = q_idx + (r * n_groups + g) * (int64_t)index_dim;
      float* out = pooled + (r * n_groups + g) * ld;
      for (int64_t b = 0; b < ld; ++b) out[b] = -INFINITY;
      for (int64_t i = 0; i <= t; ++i) {
        const float s = index_score(q, k_idx + i * (int64_t)index_dim, index_dim);
        const int64_t b = i / block_size;
        if (s > out[b]) out[b] = s;
      }
      /* -0 and +0 are the same score; write +0. */
      for (int64_t b = 0; b <= t / block_size; ++b) out[b] = out[b] + 0.0f;
    }
  }
  return ORACLE_OK;
}

/*
 * Step 3 for n_rows query rows.
 *   pooled [n_rows][n_groups][ld]   block scores (only b < c is read)
 *   sel    [n_rows][n_groups][top_k] out: ascending block ids, -1 padded
 * The top_k - 1 non-local blocks are taken one at a time: each round takes
 * the best block not yet taken, where "best" means the highest score and,
 * among equal scores, the lowest block index (a strictly-greater test while
 * scanning upward keeps the first of equal scores).
 */
int msa_oracle_select(int64_t n_rows, const int64_t* pos, const float* pooled, int n_groups,
                      int64_t ld, int block_size, int top_k, int32_t* sel) {
  if (n_rows < 0 || n_groups <= 0 || block_size <= 0 || top_k <= 0 || !pos || !sel) return ORACLE_BAD_ARG;
  if (n_rows > 0 && !pooled) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (pos[r] < 0 || pos[r] / block_size >= ld) return ORACLE_BAD_ARG;
  int status = ORACLE_OK;

#pragma omp parallel
  {
    unsigned char* taken = (unsigned char*)malloc((size_t)(ld > 0 ? ld : 1));
    if (!taken) {
#pragma omp atomic write
      status = ORACLE_NO_MEMORY;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!taken) continue;
      const int64_t c = pos[r] / block_size;
      for (int g = 0; g < n_groups; ++g) {
        const float* S = pooled + (r * n_groups + g) * ld;
        int32_t* out = sel + (r * n_groups + g) * (int64_t)top_k;
        for (int j = 0; j < top_k; ++j) out[j] = -1;
        if (c + 1 <= top_k) {
          /* Fewer causal blocks than slots: all of them. */
          for (int64_t b = 0; b <= c; ++b) out[b] = (int32_t)b;
          continue;
        }
        memset(taken, 0, (size_t)c);
        for (int round = 0; round < top_k - 1; ++round) {
          int64_t best = -1;
          for (int64_t b = 0; b < c; ++b) {
            if (taken[b]) continue;
            if (best < 0 || S[b] > S[best]) best = b;
          }
          taken[best] = 1;
        }
        int j = 0;
        for (int64_t b = 0; b < c; ++b)
          if (taken[b]) out[j++] = (int32_t)b;
        out[j] = (int32_t)c; /* the local block, always kept, largest id */
      }
    }
    free(taken);
  }
  return status;
}

/*
 * Step 4 for n_rows query rows: for head h of group g = h / (n_q_heads /
 * n_groups), softmax attention of q[r][h] over the tokens of the blocks in
 * sel[r][g], restricted to tokens i <= t.
 *   q    [n_rows][n_q_heads][head_dim]   bf16 bits
 *   k, v [n_keys][n_groups][head_dim]    bf16 bits, logical token order
 *   sel  [n_rows][n_groups][top_k]       block ids, -1 = unused slot
 *   out  [n_rows][n_q_heads][head_dim]   double
 * The softmax subtracts the maximum score before exponentiating (the value
 * of the softmax does not change, only its overflow behaviour).
 */
int msa_oracle_attend(int64_t n_rows, const int64_t* pos, const uint16_t* q, int n_q_heads, int n_groups,
                      int head_dim, const uint16_t* k, const uint16_t* v, int64_t n_keys, const int32_t* sel,
                      int block_size, int top_k, double scale, double* out) {
  if (n_rows < 0 || n_groups <= 0 || n_q_heads <= 0 || n_q_heads % n_groups != 0 || head_dim <= 0 ||
      block_size <= 0 || top_k <= 0 || !pos || !out)
    return ORACLE_BAD_ARG;
  if (n_rows > 0 && (!q || !k || !v || !sel)) return ORACLE_BAD_ARG;
  const int group_size = n_q_heads / n_groups;
  int status = ORACLE_OK;

  /* Validate the selections first: each id is a causal block, no repeats. */
  for (int64_t r = 0; r < n_rows && status == ORACLE_OK; ++r) {
    if (pos[r] < 0 || pos[r] >= n_keys) status = ORACLE_BAD_ARG;
    const int64_t c = pos[r] / block_size;
    for (int g = 0; g < n_groups && status == ORACLE_OK; ++g) {
      const int32_t* s = sel + (r * n_groups + g) * (int64_t)top_k;
      for (int j = 0; j < top_k; ++j) {
        if (s[j] < -1 || s[j] > c) status = ORACLE_BAD_SEL;
        for (int j2 = 0; j2 < j; ++j2)
          if (s[j] >= 0 && s[j2] == s[j]) status = ORACLE_BAD_SEL;
      }
    }
  }
  if (status != ORACLE_OK) return status;

#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)top_k * (size_t)block_size);
    int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)top_k * (size_t)block_size);
    double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
    if (!z || !idx || !acc) {
#pragma omp atomic write
      status = ORACLE_NO_MEMORY;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!z || !idx || !acc) continue;
      const int64_t t = pos[r];
      for (int h = 0; h < n_q_heads; ++h) {
        const int g = h / group_size;
        const int32_t* s = sel + (r * n_groups + g) * (int64_t)top_k;
        const uint16_t* qh = q + (r * n_q_heads + h) * (int64_t)head_dim;
        /* Gather the attended token set I and the scores z_i. */
        int64_t n = 0;
        for (int j = 0; j < top_k; ++j) {
          if (s[j] < 0) continue;
          for (int64_t i = (int64_t)s[j] * block_size; i < (int64_t)(s[j] + 1) * block_size && i <= t; ++i) {
            const uint16_t* ki = k + (i * n_groups + g) * (int64_t)head_dim;
            double dot = 0.0;
            for (int d = 0; d < head_dim; ++d) dot += bf16_to_double(qh[d]) * bf16_to_double(ki[d]);
            z[n] = scale * dot;
            idx[n] = i;
            ++n;
          }
        }
        double* o = out + (r * n_q_heads + h) * (int64_t)head_dim;
        /* Softmax over I, then the probability-weighted sum of values. */
        double zmax = -INFINITY;
        for (int64_t m = 0; m < n; ++m)
          if (z[m] > zmax) zmax = z[m];
        double denom = 0.0;
        for (int d = 0; d < head_dim; ++d) acc[d] = 0.0;
        for (int64_t m = 0; m < n; ++m) {
          const double w = exp(z[m] - zmax);
          denom += w;
          const uint16_t* vi = v + (idx[m] * n_groups + g) * (int64_t)head_dim;
          for (int d = 0; d < head_dim; ++d) acc[d] += w * bf16_to_double(vi[d]);
        }
        for (int d = 0; d < head_dim; ++d) o[d] = n > 0 ? acc[d] / denom : NAN;
      }
    }
    free(z);
    free(idx);
    free(acc);
  }
  return status;
}

/*
 * Step 5: dense attention mass per block.  For each row (position t) and
 * group g, every head h of the group gets the softmax of z_i = scale * q_h.k_i
 * over ALL causal tokens i <= t (not only the selected ones); the mass of
 * block b is the sum of those probabilities over the tokens of b, averaged
 * over the G heads of the group.  out: double [n_rows][n_groups][ld], blocks
 * after the row's own block are 0.
 */
int msa_oracle_block_mass(int64_t n_rows, const int64_t* pos, const uint16_t* q, int n_q_heads, int n_groups,
                          int head_dim, const uint16_t* k, int64_t n_keys, int block_size, double scale,
                          double* out, int64_t ld) {
  if (n_rows < 0 || n_groups <= 0 || n_q_heads <= 0 || n_q_heads % n_groups != 0 || head_dim <= 0 ||
      block_size <= 0 || ld <= 0 || !pos || !out)
    return ORACLE_BAD_ARG;
  if (n_rows > 0 && (!q || !k)) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (pos[r] < 0 || pos[r] >= n_keys || pos[r] / block_size >= ld) return ORACLE_BAD_ARG;
  const int group_size = n_q_heads / n_groups;
  int status = ORACLE_OK;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)n_keys);
    if (!z) {
#pragma omp atomic write
      status = ORACLE_NO_MEMORY;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!z) continue;
      const int64_t t = pos[r];
      for (int g = 0; g < n_groups; ++g) {
        double* mass = out + (r * n_groups + g) * ld;
        for (int64_t b = 0; b < ld; ++b) mass[b] = 0.0;
        for (int j = 0; j < group_size; ++j) {
          const int h = g * group_size + j;
          const uint16_t* qh = q + (r * n_q_heads + h) * (int64_t)head_dim;
          double zmax = -INFINITY;
          for (int64_t i = 0; i < t + 1; ++i) { /* every causal token */
            const uint16_t* key = k + (i * n_groups + g) * (int64_t)head_dim;
            double dot = 0.0;
            for (int d = 0; d < head_dim; ++d) dot += bf16_to_double(qh[d]) * bf16_to_double(key[d]);
            z[i] = scale * dot;
            if (z[i] > zmax) zmax = z[i];
          }
          double denom = 0.0;
          for (int64_t i = 0; i < t + 1; ++i) { /* softmax denominator */
            z[i] = exp(z[i] - zmax);
            denom += z[i];
          }
          for (int64_t i = 0; i < t + 1; ++i) mass[i / block_size] += z[i] / denom / group_size;
        }
      }
    }
    free(z);
  }
  return status;
}

/*
 * Step 6: quality of one selection against the dense mass P.
 *   coverage = sum of P_b over the selected blocks (ids >= 0);
 *   recall   = |selected AND top| / |top|, top = the K = min(top_k, c+1)
 *              blocks of largest P (repeated argmax, strictly greater wins, so
 *              equal masses go to the lower index).
 * mass is double [n_rows][n_groups][ld]; sel int32 [n_rows][n_groups][top_k].
 * Outputs double [n_rows][n_groups].
 */
int msa_oracle_selection_quality(int64_t n_rows, const int64_t* pos, const double* mass, const int32_t* sel,
                                 int n_groups, int64_t ld, int block_size, int top_k, double* coverage,
                                 double* recall) {
  if (n_rows < 0 || n_groups <= 0 || ld <= 0 || block_size <= 0 || top_k <= 0 || !pos || !coverage || !recall)
    return ORACLE_BAD_ARG;
  if (n_rows > 0 && (!mass || !sel)) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (pos[r] < 0 || pos[r] / block_size >= ld) return ORACLE_BAD_ARG;
  int status = ORACLE_OK;
#pragma omp parallel
  {
    char* taken = (char*)malloc((size_t)ld);
    if (!taken) {
#pragma omp atomic write
      status = ORACLE_NO_MEMORY;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!taken) continue;
      const int64_t c = pos[r] / block_size;
      for (int g = 0; g < n_groups; ++g) {
        const int64_t row = r * n_groups + g;
        const double* P = mass + row * ld;
        const int32_t* s = sel + row * (int64_t)top_k;
        double cov = 0.0;
        for (int j = 0; j < top_k; ++j)
          if (s[j] >= 0) cov += P[s[j]];
        /* The K blocks of largest mass. */
        const int64_t K = c + 1 < top_k ? c + 1 : top_k;
        for (int64_t b = 0; b <= c; ++b) taken[b] = 0;
        for (int64_t round = 0; round < K; ++round) {
          int64_t best = -1;
          for (int64_t b = 0; b <= c; ++b)
            if (!taken[b] && (best < 0 || P[b] > P[best])) best = b;
          taken[best] = 1;
        }
        int64_t hits = 0;
        for (int j = 0; j < top_k; ++j)
          if (s[j] >= 0 && s[j] <= c && taken[s[j]]) ++hits;
        coverage[row] = cov;
        recall[row] = (double)hits / (double)K;
      }
    }
    free(taken);
  }
  return status;
}

/*
 * Step 7: the Main Branch's importance of each candidate block.  For each
 * row (position t) and group g, every head h of the group takes the softmax
 * of z_i = scale * q_h.k_i over the tokens it attends in step 4 (the tokens
 * i <= t of the blocks in sel[r][g]); the mass of a selected block is the sum
 * of those probabilities over its tokens, averaged over the G heads.
 * out: double [n_rows][n_groups][ld]; blocks that are not selected (and
 * blocks after the row's own block) are 0, so each row sums to 1 over its
 * selected blocks.  sel int32 [n_rows][n_groups][top_k], -1 = unused slot.
 */
int msa_oracle_selected_mass(int64_t n_rows, const int64_t* pos, const uint16_t* q, int n_q_heads, int n_groups,
                             int head_dim, const uint16_t* k, int64_t n_keys, const int32_t* sel, int block_size,
                             int top_k, double scale, double* out, int64_t ld) {
  if (n_rows < 0 || n_groups <= 0 || n_q_heads <= 0 || n_q_heads % n_groups != 0 || head_dim <= 0 ||
      block_size <= 0 || top_k <= 0 || ld <= 0 || !pos || !out)
    return ORACLE_BAD_ARG;
  if (n_rows > 0 && (!q || !k || !sel)) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < n_rows; ++r) {
    if (pos[r] < 0 || pos[r] >= n_keys || pos[r] / block_size >= ld) return ORACLE_BAD_ARG;
    for (int g = 0; g < n_groups; ++g)
      for (int j = 0; j < top_k; ++j) {
        const int32_t b = sel[(r * n_groups + g) * (int64_t)top_k + j];
        if (b < -1 || b > pos[r] / block_size) return ORACLE_BAD_SEL;
      }
  }
  const int group_size = n_q_heads / n_groups;
  int status = ORACLE_OK;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)top_k * (size_t)block_size);
    int64_t* blk = (int64_t*)malloc(sizeof(int64_t) * (size_t)top_k * (size_t)block_size);
    if (!z || !blk) {
#pragma omp atomic write
      status = ORACLE_NO_MEMORY;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!z || !blk) continue;
      const int64_t t = pos[r];
      for (int g = 0; g < n_groups; ++g) {
        double* mass = out + (r * n_groups + g) * ld;
        for (int64_t b = 0; b < ld; ++b) mass[b] = 0.0;
        const int32_t* s = sel + (r * n_groups + g) * (int64_t)top_k;
        for (int j = 0; j < group_size; ++j) {
          const int h = g * group_size + j;
          const uint16_t* qh = q + (r * n_q_heads + h) * (int64_t)head_dim;
          /* The scores of the attended tokens, as in step 4. */
          int64_t n = 0;
          double zmax = -INFINITY;
          for (int jj = 0; jj < top_k; ++jj) {
            if (s[jj] < 0) continue;
            for (int64_t i = (int64_t)s[jj] * block_size; i < (int64_t)(s[jj] + 1) * block_size && i <= t; ++i) {
              const uint16_t* key = k + (i * n_groups + g) * (int64_t)head_dim;
              double dot = 0.0;
              for (int d = 0; d < head_dim; ++d) dot += bf16_to_double(qh[d]) * bf16_to_double(key[d]);
              z[n] = dot * scale;
              blk[n] = s[jj];
              if (z[n] > zmax) zmax = z[n];
              ++n;
            }
          }
          double denom = 0.0;
          for (int64_t m = 0; m < n; ++m) { /* softmax over the attended tokens */
            z[m] = exp(z[m] - zmax);
            denom += z[m];
          }
          for (int64_t m = 0; m < n; ++m) mass[blk[m]] += z[m] / denom / group_size;
        }
      }
    }
    free(z);
    free(blk);
  }
  return status;
}

/*
 * Step 8: D_KL(P || Q) over the candidate blocks of each row and group.
 *   P = sel_mass (step 7) on the selected blocks;
 *   Q_b = exp(S_b) / sum over the selected blocks b' of exp(S_b'), S the
 *         pooled index scores (step 2);
 *   kl = sum over selected b with P_b > 0 of P_b * (ln P_b - ln Q_b).
 * sel_mass double [n_rows][n_groups][ld]; pooled float [n_rows][n_groups][ld];
 * sel int32 [n_rows][n_groups][top_k].  Output double [n_rows][n_groups].
 */
int msa_oracle_indexer_kl(int64_t n_rows, const int64_t* pos, const double* sel_mass, const float* pooled,
                          const int32_t* sel, int n_groups, int64_t ld, int block_size, int top_k, double* kl) {
  if (n_rows < 0 || n_groups <= 0 || ld <= 0 || block_size <= 0 || top_k <= 0 || !pos || !kl) return ORACLE_BAD_ARG;
  if (n_rows > 0 && (!sel_mass || !pooled || !sel)) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < n_rows; ++r) {
    if (pos[r] < 0 || pos[r] / block_size >= ld) return ORACLE_BAD_ARG;
    for (int g = 0; g < n_groups; ++g)
      for (int j = 0; j < top_k; ++j) {
        const int32_t b = sel[(r * n_groups + g) * (int64_t)top_k + j];
        if (b < -1 || b > pos[r] / block_size) return ORACLE_BAD_SEL;
      }
  }
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int g = 0; g < n_groups; ++g) {
      const int64_t row = r * n_groups + g;
      const double* P = sel_mass + row * ld;
      const float* S = pooled + row * ld;
      const int32_t* s = sel + row * (int64_t)top_k;
      /* ln Q_b = S_b - log sum over the candidates of exp(S_b'). */
      double smax = -INFINITY;
      for (int j = 0; j < top_k; ++j)
        if (s[j] >= 0 && S[s[j]] > smax) smax = S[s[j]];
      double sum = 0.0;
      for (int j = 0; j < top_k; ++j)
        if (s[j] >= 0) sum += exp((double)S[s[j]] - smax);
      const double lse = smax + log(sum);
      double d = 0.0;
      for (int j = 0; j < top_k; ++j)
        if (s[j] >= 0 && P[s[j]] > 0.0) d += P[s[j]] * (log(P[s[j]]) - ((double)S[s[j]] - lse));
      kl[row] = d;
    }
  }
  return ORACLE_OK;
}
