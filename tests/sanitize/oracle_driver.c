/* The oracle's C core under AddressSanitizer / UndefinedBehaviorSanitizer
 * (test infrastructure): one-sided Jacobi SVD of random pages of every
 * shape the tests use, batched and single, and the bf16 rounding helpers;
 * the factors must reproduce the page.  Exit status 0 when they do. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int pkvo_svd(const double* X, int n, int m, double* U, double* S, double* Wt);
int pkvo_svd_batch(const double* X, int64_t n_pages, int n, int m, double* U, double* S, double* Wt);
void pkvo_bf16_encode(const double* x, uint16_t* out, int64_t n);
void pkvo_bf16_decode(const uint16_t* b, double* out, int64_t n);
void pkvo_round_array(double* x, int64_t n, int mode);

static double frand(unsigned* s) {
  *s = *s * 1664525u + 1013904223u;
  return ((*s >> 8) & 0xffff) / 32768.0 - 1.0;
}

int main(void) {
  unsigned seed = 7;
  int bad = 0;
  const int shapes[][2] = {{64, 128}, {8, 8}, {1, 5}, {32, 128}};
  for (int sh = 0; sh < 4; ++sh) {
    const int n = shapes[sh][0], m = shapes[sh][1], pages = 3;
    double* X = malloc(sizeof(double) * pages * n * m);
    double* U = malloc(sizeof(double) * pages * n * n);
    double* S = malloc(sizeof(double) * pages * n);
    double* Wt = malloc(sizeof(double) * pages * n * m);
    for (int i = 0; i < pages * n * m; ++i) X[i] = frand(&seed);
    if (pkvo_svd_batch(X, pages, n, m, U, S, Wt) != 0) bad++;
    for (int p = 0; p < pages; ++p) {
      double err = 0, nrm = 0;
      for (int i = 0; i < n; ++i)
        for (int j = 0; j < m; ++j) {
          double acc = 0;
          for (int k = 0; k < n; ++k) acc += U[p * n * n + i * n + k] * S[p * n + k] * Wt[p * n * m + k * m + j];
          const double x = X[p * n * m + i * m + j];
          err += (acc - x) * (acc - x);
          nrm += x * x;
        }
      if (!(sqrt(err) <= 1e-10 * sqrt(nrm))) {
        fprintf(stderr, "shape %dx%d page %d: reconstruction %g\n", n, m, p, sqrt(err / nrm));
        bad++;
      }
    }
    if (pkvo_svd(X, n, m, U, S, Wt) < 0) bad++;  /* (returns its sweep count) */
    free(X);
    free(U);
    free(S);
    free(Wt);
  }
  /* normal values round to within half a bf16 step; a subnormal is kept
     to the subnormal step 2^-133 */
  double v[5] = {1.0, -2.5, 3.14159, 1e-40, 65504.0}, w[5];
  uint16_t b[5];
  pkvo_bf16_encode(v, b, 5);
  pkvo_bf16_decode(b, w, 5);
  for (int i = 0; i < 5; ++i)
    if (fabs(w[i] - v[i]) > fmax(fabs(v[i]) * 0.004, ldexp(1.0, -134))) bad++;
  pkvo_round_array(v, 5, 0);
  for (int i = 0; i < 5; ++i)
    if (v[i] != w[i]) bad++;
  if (bad) fprintf(stderr, "%d oracle checks failed\n", bad);
  else printf("oracle driver: all checks passed\n");
  return bad ? 1 : 0;
}
