/*
 * Drives every entry point of the CPU oracle (oracle/gmla_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer: all argument paths (causal and
 * not, row subsets, chunk offsets Tq < Tk, weights and log-sum-exp outputs, several
 * threads, invalid arguments), with a few exact checks.  Exit status 0 = clean.
 * Test infrastructure: built and run by tests/test_oracle_sanitized.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gmla_oracle_attend_head(int64_t Tq, int64_t Tk, int64_t D, double scale, int causal,
                            const double* q, int64_t ldq, const double* k, int64_t ldk,
                            const double* v, int64_t ldv, const int64_t* rows, int64_t nrows,
                            double* out, double* lse, double* probs, int nthreads);
int gmla_oracle_linear(int64_t M, int64_t N, int64_t K, const double* x, const double* w, double* y,
                       int nthreads);
int gmla_oracle_gate(int64_t n, const double* g, const double* o, double* out);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double rnd(void) {  /* xorshift64*, uniform in [-1, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}
static double* fill(int64_t n) {
  double* p = (double*)malloc((size_t)n * sizeof(double));
  for (int64_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  const int64_t D = 12;
  const int64_t sizes[][2] = {{1, 1}, {5, 5}, {17, 40}, {64, 64}, {3, 100}};
  for (int si = 0; si < 5; ++si) {
    const int64_t Tq = sizes[si][0], Tk = sizes[si][1];
    double* q = fill(Tq * D);
    double* k = fill(Tk * D);
    double* v = fill(Tk * D);
    double* out = (double*)calloc((size_t)(Tq * D), sizeof(double));
    double* lse = (double*)calloc((size_t)Tq, sizeof(double));
    double* probs = (double*)calloc((size_t)(Tq * Tk), sizeof(double));
    for (int causal = 0; causal < 2; ++causal)
      for (int threads = 1; threads <= 3; threads += 2) {
        CHECK(gmla_oracle_attend_head(Tq, Tk, D, 0.3, causal, q, D, k, D, v, D, NULL, 0, out, lse,
                                      probs, threads) == 0);
        for (int64_t i = 0; i < Tq; ++i) {
          double sum = 0.0;
          for (int64_t s = 0; s < Tk; ++s) sum += probs[i * Tk + s];
          CHECK(fabs(sum - 1.0) < 1e-12);
          if (causal)
            for (int64_t s = i + (Tk - Tq) + 1; s < Tk; ++s) CHECK(probs[i * Tk + s] == 0.0);
        }
      }
    const int64_t rows[2] = {Tq - 1, 0};
    double* out2 = (double*)calloc((size_t)(2 * D), sizeof(double));  /* nrows x D */
    CHECK(gmla_oracle_attend_head(Tq, Tk, D, 0.3, 1, q, D, k, D, v, D, rows, 2, out2, NULL, NULL,
                                  2) == 0);
    free(out2);
    free(q); free(k); free(v); free(out); free(lse); free(probs);
  }
  /* one key: the output is that key's value row */
  {
    double q[4] = {1, 2, 3, 4}, k[4] = {4, 3, 2, 1}, v[4] = {0.5, -1, 2, 7}, o[4];
    CHECK(gmla_oracle_attend_head(1, 1, 4, 0.5, 1, q, 4, k, 4, v, 4, NULL, 0, o, NULL, NULL, 1) == 0);
    for (int d = 0; d < 4; ++d) CHECK(o[d] == v[d]);
  }
  /* invalid arguments are refused */
  {
    double a[8] = {0}, o[8];
    const int64_t bad_row[1] = {5};
    CHECK(gmla_oracle_attend_head(2, 1, 4, 0.5, 1, a, 4, a, 4, a, 4, NULL, 0, o, NULL, NULL, 1) == -1);
    CHECK(gmla_oracle_attend_head(1, 1, 4, 0.5, 2, a, 4, a, 4, a, 4, NULL, 0, o, NULL, NULL, 1) == -1);
    CHECK(gmla_oracle_attend_head(1, 1, 4, 0.5, 1, a, 4, a, 4, a, 4, bad_row, 1, o, NULL, NULL, 1) == -1);
    CHECK(gmla_oracle_linear(0, 1, 1, a, a, o, 1) == -1);
    CHECK(gmla_oracle_gate(-1, a, a, o) == -1);
  }
  /* linear and gate */
  {
    const int64_t M = 7, N = 5, K = 9;
    double* x = fill(M * K);
    double* w = fill(N * K);
    double* y = (double*)malloc((size_t)(M * N) * sizeof(double));
    CHECK(gmla_oracle_linear(M, N, K, x, w, y, 3) == 0);
    double acc = 0.0;
    for (int64_t kk = 0; kk < K; ++kk) acc += x[2 * K + kk] * w[4 * K + kk];
    CHECK(y[2 * N + 4] == acc);
    double* g = fill(M * N);
    double* z = (double*)malloc((size_t)(M * N) * sizeof(double));
    CHECK(gmla_oracle_gate(M * N, g, y, z) == 0);
    CHECK(gmla_oracle_gate(0, NULL, NULL, NULL) == 0);
    free(x); free(w); free(y); free(g); free(z);
  }
  printf("oracle sanitized run clean\n");
  return 0;
}
