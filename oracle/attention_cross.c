/*
 * Oracle: scaled-dot-product attention between Nq query rows and Nk key/value
 * rows (cross-attention), in fp64, evaluated by its plain definition on the
 * CPU.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the test suite uses it. It shares no code, header or
 * constant with the HIP library.
 *
 * The definition is that of "Writing a FlashAttention kernel in Metal",
 * section "Standard attention" (scores, a softmax over each row, a weighted
 * sum of value rows), with the logsumexp of "FlashAttention-2 from PyTorch to
 * Triton", section "What We Are Building". That page's kernel ("The Triton
 * Kernel" section) takes separate query and key counts and, when causal, keeps
 * key position j for query position i when j <= i, both counted from 0: the
 * causal mask is aligned at the top-left corner of the Nq x Nk score matrix
 * whatever the two counts. For every (b, h) and query row i < Nq:
 *
 *   S[i][j] = scale * sum_c Q[i][c] * K[j][c]          for keys j < Nk
 *   S[i][j] = -inf                   if causal and j > i
 *   P[i][j] = exp(S[i][j] - m_i) / sum_k exp(S[i][k] - m_i),  m_i = max_j S[i][j]
 *   O[i][c] = sum_j P[i][j] * V[j][c]
 *   L[i]    = m_i + log(sum_k exp(S[i][k] - m_i))
 *
 * Every query keeps key 0, so no row is empty. Each row of S and P is held in
 * full before O and L are formed from it; every sum runs over ascending
 * indices.
 *
 * Layout: Q is contiguous [B][H][Nq][d]; K, V are contiguous [B][H][Nk][d];
 * O is [B][H][Nq][d] and L is [B][H][Nq].
 *
 * Returns 0 on success, 1 on a bad argument, 3 on allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

int oracle_attention_cross_f64(const double *Q, const double *K, const double *V,
                               double *O, double *L, int64_t B, int64_t H,
                               int64_t Nq, int64_t Nk, int64_t d, int causal,
                               double scale) {
  if (!Q || !K || !V || !O || !L || B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1)
    return 1;
  double *S = (double *)malloc(sizeof(double) * (size_t)Nq * (size_t)Nk);
  double *P = (double *)malloc(sizeof(double) * (size_t)Nq * (size_t)Nk);
  if (!S || !P) {
    free(S);
    free(P);
    return 3;
  }
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const double *q = Q + bh * Nq * d;
    const double *k = K + bh * Nk * d;
    const double *v = V + bh * Nk * d;
    double *o = O + bh * Nq * d;
    double *lse = L + bh * Nq;

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < Nq; ++i) {
      double *s_row = S + i * Nk;
      double *p_row = P + i * Nk;
      for (int64_t j = 0; j < Nk; ++j) {
        if (causal && j > i) {
          s_row[j] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += q[i * d + c] * k[j * d + c];
        s_row[j] = scale * dot;
      }
      double m = -INFINITY;
      for (int64_t j = 0; j < Nk; ++j)
        if (s_row[j] > m) m = s_row[j];
      double denom = 0.0;
      for (int64_t j = 0; j < Nk; ++j) denom += exp(s_row[j] - m);
      for (int64_t j = 0; j < Nk; ++j) p_row[j] = exp(s_row[j] - m) / denom;
      for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < Nk; ++j) acc += p_row[j] * v[j * d + c];
        o[i * d + c] = acc;
      }
      lse[i] = m + log(denom);
    }
  }
  free(S);
  free(P);
  return 0;
}
