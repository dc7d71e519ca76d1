/*
 * PuzzleKV CPU oracle: double-precision reference arithmetic.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP path in long_context_decode_pkv_amd/.
 *
 * What it computes (source: "PuzzleKV: Page-Wise Low-Rank Decomposition for KV
 * Cache Compression"):
 *   - the truncated SVD of a page, X = U Sigma W^T (Sec. 3.2, "Truncated SVD"),
 *     obtained here by one-sided Jacobi rotations (Hestenes 1958) in cyclic
 *     row order with a relative orthogonality threshold (Demmel & Veselic 1992).
 *     The page itself reaches its factors through the Gram matrix X X^T
 *     (Sec. 3.3, text after Eq. 3); the oracle deliberately does not, so the
 *     two routes can be compared.
 *   - round-to-nearest-even conversion of a double to bfloat16 or float32,
 *     used to build the "stored" variant of the factors (a storage dtype is
 *     part of the cache definition; the pages do not state a rounding mode,
 *     nearest-even is the reading taken).
 *
 * Everything else the oracle needs (classification, reconstruction, naive
 * softmax attention, page-wise Eq. 4/5 states) lives in oracle/__init__.py.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define PKVO_MAX_SWEEPS 40
#define PKVO_ORTH_TOL 1e-15
/* rows whose squared norm is below this fraction of ||X||_F^2 are numerically
 * zero (sigma < 1e-15 ||X||_F) and are not rotated further */
#define PKVO_NULL_ROW 1e-30

/* ------------------------------------------------------------------ */
/* Rounding to the storage dtypes (nearest, ties to even).              */
/* ------------------------------------------------------------------ */

/* Nearest bfloat16 (1 sign, 8 exponent, 7 fraction bits) to x, ties to
 * even, returned as its 16-bit pattern.  Works directly from the double so
 * there is exactly one rounding. */
uint16_t pkvo_bf16_bits(double x) {
  if (isnan(x)) return (uint16_t)0x7fc0;
  double ax = fabs(x);
  double v;
  if (ax == 0.0) {
    v = 0.0;
  } else {
    int e;
    double f = frexp(ax, &e); /* ax = f * 2^e, f in [0.5, 1) */
    if (e - 1 < -126) {
      /* below the smallest normal: fixed quantum 2^-133 */
      v = nearbyint(ax * 0x1p133) * 0x1p-133;
    } else {
      double m = nearbyint(f * 256.0); /* 8 significant bits */
      v = ldexp(m, e - 8);
    }
  }
  float fv = (float)v; /* exact: v has at most 8 significant bits (or inf) */
  uint32_t u;
  memcpy(&u, &fv, 4);
  uint16_t b = (uint16_t)(u >> 16);
  if (signbit(x)) b |= 0x8000u;
  return b;
}

double pkvo_bf16_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* In-place rounding of n doubles: mode 0 = bfloat16, 1 = float32, 2 = none. */
void pkvo_round_array(double* x, int64_t n, int mode) {
  if (mode == 2) return;
  for (int64_t i = 0; i < n; ++i) {
    if (mode == 0)
      x[i] = pkvo_bf16_to_double(pkvo_bf16_bits(x[i]));
    else
      x[i] = (double)(float)x[i];
  }
}

void pkvo_bf16_encode(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = pkvo_bf16_bits(x[i]);
}

void pkvo_bf16_decode(const uint16_t* b, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = pkvo_bf16_to_double(b[i]);
}

/* ------------------------------------------------------------------ */
/* One-sided Jacobi SVD of a short, wide matrix.                        */
/* ------------------------------------------------------------------ */

static double dot(const double* a, const double* b, int m) {
  double s = 0.0;
  for (int k = 0; k < m; ++k) s += a[k] * b[k];
  return s;
}

/*
 * X: n x m row-major, n <= m.  On success returns the number of sweeps used
 * (>= 1) and writes
 *   U  : n x n row-major, orthonormal columns,
 *   S  : n singular values, descending (stable order for ties),
 *   Wt : n x m row-major, row i = w_i^T (zero row when S[i] == 0),
 * with X = U diag(S) Wt.  Returns -1 for bad arguments and -2 when the sweep
 * cap is hit without convergence (the caller must treat that as fatal).
 *
 * Method: the rows of A (initially X) are rotated pairwise until every pair
 * is orthogonal to PKVO_ORTH_TOL relative to the product of their norms (or
 * one of the two is numerically zero).  The
 * accumulated rotations form U, the final rows are sigma_i w_i^T.
 */
int pkvo_svd(const double* X, int n, int m, double* U, double* S, double* Wt) {
  if (n <= 0 || m <= 0 || n > m) return -1;
  double* A = (double*)malloc(sizeof(double) * (size_t)n * m);
  double* V = (double*)malloc(sizeof(double) * (size_t)n * n);
  double* nrm = (double*)malloc(sizeof(double) * n);
  int* order = (int*)malloc(sizeof(int) * n);
  if (!A || !V || !nrm || !order) {
    free(A); free(V); free(nrm); free(order);
    return -1;
  }
  memcpy(A, X, sizeof(double) * (size_t)n * m);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) V[i * n + j] = (i == j) ? 1.0 : 0.0;

  const double null_row = PKVO_NULL_ROW * dot(X, X, n * m);
  int sweeps = 0, converged = 0;
  while (sweeps < PKVO_MAX_SWEEPS) {
    ++sweeps;
    int rotated = 0;
    for (int i = 0; i < n - 1; ++i) {
      for (int j = i + 1; j < n; ++j) {
        double* ai = A + (size_t)i * m;
        double* aj = A + (size_t)j * m;
        double alpha = dot(ai, ai, m);
        double beta = dot(aj, aj, m);
        double gamma = dot(ai, aj, m);
        if (gamma == 0.0 || fabs(gamma) <= PKVO_ORTH_TOL * sqrt(alpha * beta)) continue;
        if (alpha <= null_row || beta <= null_row) continue;
        rotated = 1;
        /* rotation that makes rows i and j orthogonal:
         * t solves t^2 + 2 zeta t - 1 = 0, smaller root */
        double zeta = (beta - alpha) / (2.0 * gamma);
        double t = copysign(1.0, zeta) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        double c = 1.0 / sqrt(1.0 + t * t);
        double s = c * t;
        for (int k = 0; k < m; ++k) {
          double x = ai[k], y = aj[k];
          ai[k] = c * x - s * y;
          aj[k] = s * x + c * y;
        }
        for (int k = 0; k < n; ++k) {
          double x = V[k * n + i], y = V[k * n + j];
          V[k * n + i] = c * x - s * y;
          V[k * n + j] = s * x + c * y;
        }
      }
    }
    if (!rotated) {
      converged = 1;
      break;
    }
  }
  if (!converged) {
    free(A); free(V); free(nrm); free(order);
    return -2;
  }
  for (int i = 0; i < n; ++i) {
    nrm[i] = sqrt(dot(A + (size_t)i * m, A + (size_t)i * m, m));
    order[i] = i;
  }
  /* stable insertion sort, descending */
  for (int i = 1; i < n; ++i) {
    int key = order[i];
    int j = i - 1;
    while (j >= 0 && nrm[order[j]] < nrm[key]) {
      order[j + 1] = order[j];
      --j;
    }
    order[j + 1] = key;
  }
  for (int o = 0; o < n; ++o) {
    int i = order[o];
    S[o] = nrm[i];
    for (int k = 0; k < n; ++k) U[k * n + o] = V[k * n + i];
    for (int k = 0; k < m; ++k)
      Wt[(size_t)o * m + k] = (nrm[i] > 0.0) ? A[(size_t)i * m + k] / nrm[i] : 0.0;
  }
  free(A); free(V); free(nrm); free(order);
  return sweeps;
}

/* Batched form over independent pages; returns 0, or the first failing
 * page's status.  Pages are independent so the loop is parallel. */
int pkvo_svd_batch(const double* X, int64_t n_pages, int n, int m, double* U, double* S,
                   double* Wt) {
  int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < n_pages; ++p) {
    int rc = pkvo_svd(X + (size_t)p * n * m, n, m, U + (size_t)p * n * n, S + (size_t)p * n,
                      Wt + (size_t)p * n * m);
    if (rc < 0) {
#pragma omp critical
      { if (status == 0) status = rc; }
    }
  }
  return status;
}

int pkvo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
