/*
 * Oracle: gradients of standard scaled-dot-product attention in fp64,
 * evaluated by their plain definition on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code, header or constant
 * with the HIP library.
 *
 * The forward function is the one of attention.c ("Writing a FlashAttention
 * kernel in Metal", sections "Standard attention" and "Blockwise attention
 * and causal masking"): O = softmax(scale * Q K^T) V, with keys after the
 * query excluded when causal. Given the gradient dO of a loss with respect to
 * O, this file returns the gradients with respect to Q, K and V by the chain
 * rule through the three steps of that definition, for every (batch, head):
 *
 *   S[i][j]  = scale * sum_c Q[i][c] * K[j][c]      (-inf if causal and j > i)
 *   P[i][j]  = exp(S[i][j] - m_i) / sum_k exp(S[i][k] - m_i),  m_i = max_j S[i][j]
 *   dV[j][c] = sum_i P[i][j] * dO[i][c]              (O = P V, so dV = P^T dO)
 *   dP[i][j] = sum_c dO[i][c] * V[j][c]              (and dP = dO V^T)
 *   dS[i][j] = P[i][j] * (dP[i][j] - sum_k P[i][k] * dP[i][k])
 *                                                    (Jacobian of a row softmax)
 *   dQ[i][c] = scale * sum_j dS[i][j] * K[j][c]      (S = scale Q K^T)
 *   dK[j][c] = scale * sum_i dS[i][j] * Q[i][c]
 *
 * A masked score has P = 0 and hence dS = 0, so it contributes nothing. L is
 * treated as an auxiliary output (saved for the backward, as the third page's
 * "What We Are Building" section describes), not as a differentiated one.
 *
 * Nothing is tiled, fused or reordered: S, P, dP and dS of a head are
 * materialised in full (N x N) and every sum runs over ascending indices.
 *
 * Layout: Q, K, V, dO, dQ, dK, dV are contiguous [B][H][N][d] fp64 arrays.
 * Returns 0 on success, 1 on a bad argument, 2 if a row has no admissible key,
 * 3 on allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

int oracle_attention_bwd_f64(const double *Q, const double *K, const double *V,
                             const double *dO, double *dQ, double *dK, double *dV,
                             int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                             double scale) {
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV || B < 1 || H < 1 || N < 1 || d < 1)
    return 1;
  /* P then dS of one head, each N x N, in full. */
  double *P = (double *)malloc(sizeof(double) * (size_t)N * (size_t)N);
  double *G = (double *)malloc(sizeof(double) * (size_t)N * (size_t)N);
  if (!P || !G) {
    free(P);
    free(G);
    return 3;
  }
  int status = 0;

  for (int64_t bh = 0; bh < B * H; ++bh) {
    const double *q = Q + bh * N * d;
    const double *k = K + bh * N * d;
    const double *v = V + bh * N * d;
    const double *go = dO + bh * N * d;
    double *gq = dQ + bh * N * d;
    double *gk = dK + bh * N * d;
    double *gv = dV + bh * N * d;

#pragma omp parallel for schedule(dynamic, 4) reduction(| : status)
    for (int64_t i = 0; i < N; ++i) {
      double *p_row = P + i * N;
      double *g_row = G + i * N;

      /* Scores, masked above the diagonal when causal. */
      for (int64_t j = 0; j < N; ++j) {
        if (causal && j > i) {
          p_row[j] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += q[i * d + c] * k[j * d + c];
        p_row[j] = scale * dot;
      }

      /* Row softmax, shifted by the row maximum. */
      double m = -INFINITY;
      for (int64_t j = 0; j < N; ++j)
        if (p_row[j] > m) m = p_row[j];
      if (m == -INFINITY) {
        status |= 2;
        continue;
      }
      double denom = 0.0;
      for (int64_t j = 0; j < N; ++j) denom += exp(p_row[j] - m);
      for (int64_t j = 0; j < N; ++j) p_row[j] = exp(p_row[j] - m) / denom;

      /* dP = dO V^T for this row, then the softmax Jacobian applied to it. */
      for (int64_t j = 0; j < N; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += go[i * d + c] * v[j * d + c];
        g_row[j] = dot;
      }
      double pdp = 0.0;
      for (int64_t j = 0; j < N; ++j) pdp += p_row[j] * g_row[j];
      for (int64_t j = 0; j < N; ++j) g_row[j] = p_row[j] * (g_row[j] - pdp);

      /* dQ row: scale * dS K. */
      for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < N; ++j) acc += g_row[j] * k[j * d + c];
        gq[i * d + c] = scale * acc;
      }
    }
    if (status) break;

    /* dV = P^T dO and dK = scale * dS^T Q, one key row at a time. */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < N; ++j) {
      for (int64_t c = 0; c < d; ++c) {
        double av = 0.0, ak = 0.0;
        for (int64_t i = 0; i < N; ++i) {
          av += P[i * N + j] * go[i * d + c];
          ak += G[i * N + j] * q[i * d + c];
        }
        gv[j * d + c] = av;
        gk[j * d + c] = scale * ak;
      }
    }
  }
  free(P);
  free(G);
  return status;
}
