/*
 * gmla_oracle.c -- plain, slow CPU reference for the causal softmax attention of
 * a Gated MLA layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this file's library.  The GPU library shares no code,
 * header, table or helper with it, and never calls it.
 *
 * Everything is double precision, written as the definitions read, one output row
 * at a time, with no blocking, fusion or reordering beyond the definitions:
 *
 *   Scores   S[t,s] = scale * sum_d Q[t,d] K[s,d]
 *            ("Gated MLA", section "Start from familiar attention": softmax of
 *            Q K^T / sqrt(D_h) + M; "Kimi K3 - Softmax over keys", the eager
 *            attention code: einsum of query and key, times scaling).
 *   Mask     M[t,s] = 0 if s <= t, -inf if s > t ("Kimi K2 - Construct causal
 *            mask", the formula for M).  A masked key therefore has weight exactly
 *            zero; the oracle skips it.  With Tq queries against Tk keys, query i
 *            sits at absolute position t = i + (Tk - Tq), as positions start at the
 *            cached length on that page's position-id code; one decode query at
 *            position p sees keys 0..p ("Kimi K3 - Softmax over keys": S is
 *            [B, 96, 1, 1001] at p = 1000).
 *   Softmax  A[t,s] = exp S[t,s] / sum_{u<=t} exp S[t,u], A[t,s] = 0 for s > t
 *            ("Kimi K3 - Softmax over keys", the formula).  The row maximum is
 *            subtracted before exp, which leaves A unchanged exactly in real
 *            arithmetic.
 *   Mixing   O[t,:] = sum_s A[t,s] V[s,:]  (same code: einsum of probs and value;
 *            "Le Transformer et l'attention", step "Agréger").
 *   Linear   Y = X W^T with W stored [out, in]  ("Gated MLA", C = X W_c^T,
 *            K = C W_k^T, V = C W_v^T, Y = [...] W_o^T).
 *   Gate     sigmoid(x) = 1 / (1 + exp(-x)), applied channel-wise ("Gated MLA",
 *            section "The channel-wise output gate").
 *
 * Rows are independent, so the only parallelism is a pool of threads that each take
 * whole output rows.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <unistd.h>

/* ------------------------------------------------------------------------- */
/* Threading: run fn(ctx, row) for row in [0, nrows) on nthreads threads.     */
/* ------------------------------------------------------------------------- */

typedef void (*row_fn)(void* ctx, int64_t row, void* scratch);

typedef struct {
  row_fn fn;
  void* ctx;
  int64_t nrows;
  int64_t next;
  size_t scratch_bytes;
  pthread_mutex_t lock;
  int failed;
} pool_t;

static void* pool_worker(void* arg) {
  pool_t* p = (pool_t*)arg;
  void* scratch = NULL;
  if (p->scratch_bytes) {
    scratch = malloc(p->scratch_bytes);
    if (!scratch) {
      pthread_mutex_lock(&p->lock);
      p->failed = 1;
      pthread_mutex_unlock(&p->lock);
      return NULL;
    }
  }
  for (;;) {
    pthread_mutex_lock(&p->lock);
    int64_t row = p->next++;
    pthread_mutex_unlock(&p->lock);
    if (row >= p->nrows) break;
    p->fn(p->ctx, row, scratch);
  }
  free(scratch);
  return NULL;
}

static int run_rows(row_fn fn, void* ctx, int64_t nrows, size_t scratch_bytes, int nthreads) {
  if (nthreads <= 0) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = n > 0 ? (int)n : 1;
  }
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
  pool_t p;
  p.fn = fn;
  p.ctx = ctx;
  p.nrows = nrows;
  p.next = 0;
  p.scratch_bytes = scratch_bytes;
  p.failed = 0;
  pthread_mutex_init(&p.lock, NULL);
  pthread_t tids[256];
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&tids[i], NULL, pool_worker, &p) != 0) break;
    ++started;
  }
  if (started == 0) pool_worker(&p); /* no thread could start: do the work here */
  for (int i = 0; i < started; ++i) pthread_join(tids[i], NULL);
  pthread_mutex_destroy(&p.lock);
  return p.failed ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* Attention for one head.                                                    */
/* ------------------------------------------------------------------------- */

typedef struct {
  int64_t Tq, Tk, D;
  double scale;
  int causal;
  const double *q, *k, *v;
  int64_t ldq, ldk, ldv;
  const int64_t* rows;
  double* out;
  double* lse;
  double* probs;
} attend_ctx;

static void attend_row(void* vctx, int64_t r, void* scratch) {
  const attend_ctx* c = (const attend_ctx*)vctx;
  double* s = (double*)scratch; /* one score per key */
  const int64_t i = c->rows ? c->rows[r] : r;
  const int64_t t = i + (c->Tk - c->Tq); /* absolute position of query i */
  /* keys 0..last are visible */
  const int64_t last = c->causal ? t : c->Tk - 1;
  const double* qi = c->q + i * c->ldq;

  /* scores of the visible keys */
  for (int64_t j = 0; j <= last; ++j) {
    const double* kj = c->k + j * c->ldk;
    double dot = 0.0;
    for (int64_t d = 0; d < c->D; ++d) dot += qi[d] * kj[d];
    s[j] = c->scale * dot;
  }
  /* softmax over the visible keys */
  double m = -INFINITY;
  for (int64_t j = 0; j <= last; ++j)
    if (s[j] > m) m = s[j];
  double z = 0.0;
  for (int64_t j = 0; j <= last; ++j) {
    s[j] = exp(s[j] - m);
    z += s[j];
  }
  for (int64_t j = 0; j <= last; ++j) s[j] /= z;
  /* weighted sum of the values */
  double* o = c->out + r * c->D;
  for (int64_t d = 0; d < c->D; ++d) o[d] = 0.0;
  for (int64_t j = 0; j <= last; ++j) {
    const double* vj = c->v + j * c->ldv;
    for (int64_t d = 0; d < c->D; ++d) o[d] += s[j] * vj[d];
  }
  if (c->lse) c->lse[r] = m + log(z);
  if (c->probs) {
    double* a = c->probs + r * c->Tk;
    for (int64_t j = 0; j < c->Tk; ++j) a[j] = j <= last ? s[j] : 0.0;
  }
}

/*
 * Attention of Tq queries against Tk keys for one head.
 *   q: Tq rows of D values, row stride ldq (elements); k, v: Tk rows, strides ldk, ldv.
 *   rows: the query indices to compute (NULL: all Tq, in order); nrows of them.
 *   out: nrows x D.  lse (nullable): nrows log-sum-exp values of the scaled scores.
 *   probs (nullable): nrows x Tk attention weights, zero for masked keys.
 * Returns 0, or -1 on invalid arguments or allocation failure.
 */
int gmla_oracle_attend_head(int64_t Tq, int64_t Tk, int64_t D, double scale, int causal,
                            const double* q, int64_t ldq, const double* k, int64_t ldk,
                            const double* v, int64_t ldv, const int64_t* rows, int64_t nrows,
                            double* out, double* lse, double* probs, int nthreads) {
  if (Tq <= 0 || Tk <= 0 || D <= 0 || Tq > Tk || !q || !k || !v || !out) return -1;
  if (causal != 0 && causal != 1) return -1;
  if (!rows) nrows = Tq;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= Tq) return -1;
  attend_ctx c = {Tq, Tk, D, scale, causal, q, k, v, ldq, ldk, ldv, rows, out, lse, probs};
  return run_rows(attend_row, &c, nrows, (size_t)Tk * sizeof(double), nthreads);
}

/* ------------------------------------------------------------------------- */
/* Y = X W^T                                                                  */
/* ------------------------------------------------------------------------- */

typedef struct {
  int64_t N, K;
  const double *x, *w;
  double* y;
} linear_ctx;

static void linear_row(void* vctx, int64_t i, void* scratch) {
  (void)scratch;
  const linear_ctx* c = (const linear_ctx*)vctx;
  const double* xi = c->x + i * c->K;
  double* yi = c->y + i * c->N;
  for (int64_t j = 0; j < c->N; ++j) {
    const double* wj = c->w + j * c->K; /* row j of W is output feature j */
    double acc = 0.0;
    for (int64_t kk = 0; kk < c->K; ++kk) acc += xi[kk] * wj[kk];
    yi[j] = acc;
  }
}

/* Y[M,N] = X[M,K] W[N,K]^T, all row-major.  Returns 0 or -1. */
int gmla_oracle_linear(int64_t M, int64_t N, int64_t K, const double* x, const double* w, double* y,
                       int nthreads) {
  if (M <= 0 || N <= 0 || K <= 0 || !x || !w || !y) return -1;
  linear_ctx c = {N, K, x, w, y};
  return run_rows(linear_row, &c, M, 0, nthreads);
}

/* ------------------------------------------------------------------------- */
/* Channel-wise sigmoid gate: out = sigmoid(g) * o, elementwise.              */
/* ------------------------------------------------------------------------- */

int gmla_oracle_gate(int64_t n, const double* g, const double* o, double* out) {
  if (n < 0 || (n > 0 && (!g || !o || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = o[i] / (1.0 + exp(-g[i]));
  return 0;
}
