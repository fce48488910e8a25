/*
 * Oracle: standard scaled-dot-product attention in fp64, evaluated by its
 * plain definition on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code, header or constant
 * with the HIP library.
 *
 * What it computes, for every (batch b, head h) and every selected query row i,
 * following "Writing a FlashAttention kernel in Metal", section "Standard
 * attention" (scores, softmax over each row, weighted sum of value rows),
 * section "Blockwise attention and causal masking" (a key after the query is
 * excluded, its score set to minus infinity), and "FlashAttention-2 from
 * PyTorch to Triton", section "What We Are Building" (L is the natural-log
 * logsumexp of the row of scaled scores):
 *
 *   S[i][j] = scale * sum_c Q[i][c] * K[j][c]             for all keys j
 *   S[i][j] = -inf                    if causal and j > i
 *   m_i     = max_j S[i][j]
 *   P[i][j] = exp(S[i][j] - m_i) / sum_k exp(S[i][k] - m_i)
 *   O[i][c] = sum_j P[i][j] * V[j][c]
 *   L[i]    = m_i + log(sum_k exp(S[i][k] - m_i))
 *
 * Subtracting the row maximum before exponentiating is the stabilisation the
 * first page's "Online softmax" section states; it leaves P and L unchanged
 * in exact arithmetic. Nothing is tiled, fused or reordered: each selected
 * row of S and P is materialised in full (all N keys) before O and L are
 * formed from it, and every sum runs over ascending indices.
 *
 * Layout: Q, K, V are contiguous [B][H][N][d] fp64 arrays. With rows == NULL
 * every query row is evaluated and O is [B][H][N][d], L is [B][H][N]. With a
 * list of nrows query indices, only those rows are evaluated and O is
 * [B][H][nrows][d], L is [B][H][nrows] (same row order as the list).
 *
 * Returns 0 on success, 1 on a bad argument, 2 if a row has no admissible key
 * (impossible when queries and keys share positions 0..N-1), 3 on allocation
 * failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int oracle_attention_f64(const double *Q, const double *K, const double *V,
                         double *O, double *L, int64_t B, int64_t H, int64_t N,
                         int64_t d, int causal, double scale,
                         const int64_t *rows, int64_t nrows) {
  if (!Q || !K || !V || !O || !L || B < 1 || H < 1 || N < 1 || d < 1)
    return 1;
  if (rows == NULL) nrows = N;
  if (nrows < 1) return 1;
  for (int64_t r = 0; rows != NULL && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return 1;

  /* S and P for the selected rows of one head, held in full. */
  double *S = (double *)malloc(sizeof(double) * (size_t)nrows * (size_t)N);
  double *P = (double *)malloc(sizeof(double) * (size_t)nrows * (size_t)N);
  if (!S || !P) {
    free(S);
    free(P);
    return 3;
  }
  int status = 0;

  for (int64_t bh = 0; bh < B * H; ++bh) {
    const double *q = Q + bh * N * d;
    const double *k = K + bh * N * d;
    const double *v = V + bh * N * d;
    double *o = O + bh * nrows * d;
    double *lse = L + bh * nrows;

#pragma omp parallel for schedule(dynamic, 4) reduction(| : status)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t i = rows ? rows[r] : r;
      double *s_row = S + r * N;
      double *p_row = P + r * N;

      /* Scores: S = scale * Q K^T, masked above the diagonal when causal. */
      for (int64_t j = 0; j < N; ++j) {
        if (causal && j > i) {
          s_row[j] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += q[i * d + c] * k[j * d + c];
        s_row[j] = scale * dot;
      }

      /* Softmax over the row, shifted by its maximum. */
      double m = -INFINITY;
      for (int64_t j = 0; j < N; ++j)
        if (s_row[j] > m) m = s_row[j];
      if (m == -INFINITY) {
        status |= 2;
        continue;
      }
      double denom = 0.0;
      for (int64_t j = 0; j < N; ++j) denom += exp(s_row[j] - m);
      for (int64_t j = 0; j < N; ++j) p_row[j] = exp(s_row[j] - m) / denom;

      /* Output row: probabilities times value rows. */
      for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < N; ++j) acc += p_row[j] * v[j * d + c];
        o[r * d + c] = acc;
      }

      /* Logsumexp of the scaled scores, natural log. */
      lse[r] = m + log(denom);
    }
    if (status) break;
  }
  free(S);
  free(P);
  return status;
}
