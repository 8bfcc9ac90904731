/* Drives the fp64 oracle (oracle/kda_oracle.c) on small inputs for a build
 * under AddressSanitizer and UndefinedBehaviorSanitizer: packed sequences
 * with empty and partial ones, NULL h0 and h_final, h_final aliasing h0,
 * and rejected arguments. Exits non-zero on a wrong status or a mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_forward(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta,
                       const double *h0, const int64_t *cu_seqlens,
                       int64_t n_seqs, int64_t H, int64_t dk, int64_t dv,
                       double *o, double *h_final, int n_threads);

static double rnd(uint64_t *s) {   /* splitmix64 -> [-1, 1) */
  uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) / 4503599627370496.0 - 1.0;
}

static double *alloc_fill(int64_t n, uint64_t *s, double scale, double shift) {
  double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = scale * rnd(s) + shift;
  return p;
}

int main(void) {
  const int64_t H = 3, dk = 8, dv = 12, N = 4;
  const int64_t cu[5] = {0, 5, 5, 70, 71};   /* one empty sequence */
  const int64_t T = cu[N];
  uint64_t s = 42;
  double *q = alloc_fill(T * H * dk, &s, 1.0, 0.0);
  double *k = alloc_fill(T * H * dk, &s, 0.3, 0.0);
  double *v = alloc_fill(T * H * dv, &s, 1.0, 0.0);
  double *la = alloc_fill(T * H * dk, &s, 0.05, -0.06);
  double *b = alloc_fill(T * H, &s, 0.5, 0.5);
  double *h0 = alloc_fill(N * H * dk * dv, &s, 0.02, 0.0);
  double *o1 = (double *)calloc((size_t)(T * H * dv), sizeof(double));
  double *o2 = (double *)calloc((size_t)(T * H * dv), sizeof(double));
  double *hf = (double *)calloc((size_t)(N * H * dk * dv), sizeof(double));
  double *hin = (double *)malloc(sizeof(double) * (size_t)(N * H * dk * dv));
  int bad = 0;
  if (kda_oracle_forward(q, k, v, la, b, h0, cu, N, H, dk, dv, o1, hf, 2) != 0) bad |= 1;
  /* h_final aliasing h0 gives the same outputs and final states */
  memcpy(hin, h0, sizeof(double) * (size_t)(N * H * dk * dv));
  if (kda_oracle_forward(q, k, v, la, b, hin, cu, N, H, dk, dv, o2, hin, 1) != 0) bad |= 2;
  if (memcmp(o1, o2, sizeof(double) * (size_t)(T * H * dv)) != 0) bad |= 4;
  if (memcmp(hf, hin, sizeof(double) * (size_t)(N * H * dk * dv)) != 0) bad |= 8;
  /* NULL h0 and NULL h_final */
  if (kda_oracle_forward(q, k, v, la, b, NULL, cu, N, H, dk, dv, o2, NULL, 0) != 0) bad |= 16;
  for (int64_t i = 0; i < T * H * dv; ++i)
    if (!isfinite(o2[i])) bad |= 32;
  /* rejected arguments */
  const int64_t cu_bad[3] = {0, 7, 3};
  const int64_t cu_off[3] = {1, 2, 3};
  if (kda_oracle_forward(q, k, v, la, b, h0, cu_bad, 2, H, dk, dv, o2, hf, 1) != -1) bad |= 64;
  if (kda_oracle_forward(q, k, v, la, b, h0, cu_off, 2, H, dk, dv, o2, hf, 1) != -1) bad |= 128;
  if (kda_oracle_forward(NULL, k, v, la, b, h0, cu, N, H, dk, dv, o2, hf, 1) != -1) bad |= 256;
  if (kda_oracle_forward(q, k, v, la, b, h0, cu, N, 0, dk, dv, o2, hf, 1) != -1) bad |= 512;
  free(q); free(k); free(v); free(la); free(b); free(h0);
  free(o1); free(o2); free(hf); free(hin);
  if (bad) fprintf(stderr, "oracle driver: failures 0x%x\n", bad);
  else printf("oracle driver ok\n");
  return bad ? 1 : 0;
}
