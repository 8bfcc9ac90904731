/*
 * KDA oracle-R: plain, slow, obviously correct fp64 CPU recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do. It shares no code with the HIP kernels.
 *
 * What it computes (Kimi Delta Attention, the channel-wise gated delta rule):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t
 *
 * Source: "Kimi Linear: An Expressive, Efficient Attention Architecture"
 * (paper-graph-ui review), section "The KDA State Update Equation" (the
 * recurrence and the readout o_t = S_t^T q_t, taken after the update); the
 * same recurrence is Eq. 1 of the "L2 Deep Distill" page and section 3.1 of
 * the intelliparadigm.com article.
 *
 * Each token is applied in the order of the review's section "Online
 * Learning Interpretation": decay first, then the error-correcting rank-1
 * step on the decayed state,
 *
 *   Sd  = Diag(alpha_t) S_{t-1}
 *   e   = Sd^T k_t                      (prediction for key k_t)
 *   S_t = Sd - beta_t k_t (e - v_t)^T   (one gradient step, rate beta_t)
 *
 * which expands to exactly the recurrence above.
 *
 * Readings where the pages leave a point open:
 *  - alpha_t arrives as its natural log, log_alpha = log(alpha_t) (the pages
 *    fuse the gate in log space upstream); alpha_t = exp(log_alpha).
 *  - No 1/sqrt(d_k) query scale: the readout is S_t^T q_t as printed.
 *  - The state S is d_k x d_v, stored row-major S[c][j] (key channel c,
 *    value column j fastest).
 *  - Sequences in a packed batch are independent; each starts from its own
 *    h0 (zeros when h0 is NULL).
 *
 * Parallelism: columns j of S evolve independently (every operation above
 * acts on each column separately), so work items are
 * (sequence, head, block of columns). The arithmetic per column is the
 * recurrence above with the sum over c in ascending order.
 *
 * Inputs, arithmetic and outputs are fp64 (bf16 and fp32 inputs are widened
 * exactly by the caller).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_COLS 16 /* columns of S per work item */

/* Runs the recurrence for one (sequence n, head h, column block [j0,j1)). */
static void oracle_block(const double *q, const double *k, const double *v,
                         const double *log_alpha, const double *beta,
                         const double *h0, int64_t t_begin, int64_t t_end,
                         int64_t n, int64_t h, int64_t H, int64_t dk,
                         int64_t dv, int64_t j0, int64_t j1, double *o,
                         double *h_final, double *S, double *a, double *kk,
                         double *qq) {
  const int64_t nb = j1 - j0;
  /* S[c][jj] for jj in [0, nb): local copy of the state block */
  for (int64_t c = 0; c < dk; ++c)
    for (int64_t jj = 0; jj < nb; ++jj)
      S[c * nb + jj] =
          h0 ? h0[((n * H + h) * dk + c) * dv + j0 + jj] : 0.0;

  for (int64_t t = t_begin; t < t_end; ++t) {
    const int64_t base_k = (t * H + h) * dk;
    const int64_t base_v = (t * H + h) * dv;
    const double b = beta[t * H + h];
    for (int64_t c = 0; c < dk; ++c) {
      a[c] = exp(log_alpha[base_k + c]); /* alpha_t[c] */
      kk[c] = k[base_k + c];
      qq[c] = q[base_k + c];
    }
    for (int64_t jj = 0; jj < nb; ++jj) {
      /* decay: Sd = Diag(alpha) S */
      for (int64_t c = 0; c < dk; ++c) S[c * nb + jj] *= a[c];
      /* prediction e_j = sum_c k_c Sd[c][j] */
      double e = 0.0;
      for (int64_t c = 0; c < dk; ++c) e += kk[c] * S[c * nb + jj];
      /* correction S = Sd - beta k (e - v)^T */
      const double err = e - v[base_v + j0 + jj];
      for (int64_t c = 0; c < dk; ++c) S[c * nb + jj] -= b * kk[c] * err;
      /* readout o_j = sum_c q_c S[c][j] (post-update state) */
      double acc = 0.0;
      for (int64_t c = 0; c < dk; ++c) acc += qq[c] * S[c * nb + jj];
      o[base_v + j0 + jj] = acc;
    }
  }
  if (h_final)
    for (int64_t c = 0; c < dk; ++c)
      for (int64_t jj = 0; jj < nb; ++jj)
        h_final[((n * H + h) * dk + c) * dv + j0 + jj] = S[c * nb + jj];
}

/*
 * kda_oracle_forward
 *   q, k        [T_total, H, dk] fp64
 *   v           [T_total, H, dv] fp64
 *   log_alpha   [T_total, H, dk] fp64 (natural log of the decay)
 *   beta        [T_total, H]     fp64
 *   h0          [N, H, dk, dv]   fp64, or NULL for zeros
 *   cu_seqlens  [N + 1]          int64, cu[0] = 0, non-decreasing
 *   o           [T_total, H, dv] fp64 (written)
 *   h_final     [N, H, dk, dv]   fp64 (written; may alias h0; may be NULL)
 *   n_threads   OpenMP threads (<= 0: library default)
 * Returns 0 on success, -1 on a bad argument, -2 on allocation failure.
 */
int kda_oracle_forward(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta,
                       const double *h0, const int64_t *cu_seqlens,
                       int64_t n_seqs, int64_t H, int64_t dk, int64_t dv,
                       double *o, double *h_final, int n_threads) {
  if (!q || !k || !v || !log_alpha || !beta || !cu_seqlens || !o) return -1;
  if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  for (int64_t n = 0; n < n_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  if (cu_seqlens[0] != 0) return -1;

  const int64_t nblk = (dv + KDA_ORACLE_COLS - 1) / KDA_ORACLE_COLS;
  const int64_t items = n_seqs * H * nblk;
  /* h_final may alias h0: a work item reads its h0 block before writing its
   * h_final block and the blocks of different items are disjoint. */
  int failed = 0;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel
  {
    double *S = (double *)malloc(sizeof(double) * dk * KDA_ORACLE_COLS);
    double *a = (double *)malloc(sizeof(double) * dk);
    double *kk = (double *)malloc(sizeof(double) * dk);
    double *qq = (double *)malloc(sizeof(double) * dk);
    const int ok = S && a && kk && qq;
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
    /* every thread reaches the work-sharing loop; one without buffers skips */
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < items; ++it) {
      if (!ok) continue;
      {
        const int64_t jb = it % nblk;
        const int64_t h = (it / nblk) % H;
        const int64_t n = it / (nblk * H);
        const int64_t j0 = jb * KDA_ORACLE_COLS;
        const int64_t j1 = j0 + KDA_ORACLE_COLS < dv ? j0 + KDA_ORACLE_COLS : dv;
        oracle_block(q, k, v, log_alpha, beta, h0, cu_seqlens[n],
                     cu_seqlens[n + 1], n, h, H, dk, dv, j0, j1, o, h_final,
                     S, a, kk, qq);
      }
    }
    free(S);
    free(a);
    free(kk);
    free(qq);
  }
  return failed ? -2 : 0;
}

/* Number of threads an OpenMP parallel region uses by default. */
int kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
