/*
 * Gated triangle self-attention with pair bias: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may build, load or call this file.  It shares
 * no code, header, table or constant with the GPU library and must stay slow
 * and obvious: one (row, head) pair per task, one full query-by-key logit block
 * in fp64, libm exp/log, no blocking, no fusion, no reordering beyond the
 * definition below.
 *
 * What it computes (starting node).  The pages describe triangle attention in
 * words only: a pair (i, j) attends over a third node k, the cost is cubic in
 * the number of tokens (TurboPairFormer news item, "Dove si impiega il
 * tempo"), the attention is gated (HelixFold review, "Fused Gated
 * Self-Attention"), and the backward produces gradients for query, key, value
 * and pair bias from the probability tiles (TurboPairFormer news item, same
 * section).  The formula taken here is the plainest one those statements
 * support:
 *
 *   s[i,h,j,k]  = (q[i,h,j,:] . k[i,h,k,:]) / sqrt(c) + b[h,j,k]
 *                 (replaced by -1e9 when mask[i,k] == 0)
 *   p[i,h,j,:]  = softmax over k of s[i,h,j,:]
 *   lse[i,h,j]  = log sum_k exp(s[i,h,j,k])
 *   a[i,h,j,:]  = sum_k p[i,h,j,k] v[i,h,k,:]
 *   o[i,j,h,:]  = sigmoid(g[i,j,h,:]) * a[i,h,j,:]
 *
 * Backward, given do[i,j,h,:]:
 *   da   = do * sigmoid(g)                       (gradient reaching a)
 *   dg   = do * a * sigmoid(g) * (1 - sigmoid(g))
 *   dv[k]  = sum_j p[j,k] da[j]
 *   dp[j,k] = da[j] . v[k]
 *   D[j]   = sum_k p[j,k] dp[j,k]                (also checked against da[j].a[j])
 *   ds[j,k] = p[j,k] (dp[j,k] - D[j]), and 0 where the logit was replaced
 *   dq[j]  = sum_k ds[j,k] k[k] / sqrt(c)
 *   dk[k]  = sum_j ds[j,k] q[j] / sqrt(c)
 *   db[h,j,k] = sum_i ds[i,h,j,k]
 *
 * Layouts (row-major, the same as the GPU boundary):
 *   q        [rows][H][nq][c]      k, v   [rows][H][nk][c]
 *   bias     [H][nq][nk]           gate, out, dout, dgate  [rows][nq][H][c]
 *   mask     [rows][nk] (NULL = every key valid)
 *   attn, dq [rows][H][nq][c]      dk, dv [rows][H][nk][c]
 *   lse, D   [rows][H][nq]         dbias  [H][nq][nk] (sum over the rows given)
 * Queries and keys have separate counts so that a caller can evaluate a
 * subset of queries (all keys) exactly: every quantity above for a query j
 * depends only on that query's own row of logits.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define MASKED_LOGIT (-1e9)

typedef struct {
  int rows, H, nq, nk, c;
  const double *q, *k, *v, *bias, *gate, *dout;
  const uint8_t *mask;
  double *out, *attn, *lse;                 /* forward outputs */
  double *dq, *dk, *dv, *dgate, *D;         /* backward outputs */
  double *dbias_part;                       /* per-thread [H][nq][nk] */
  double max_d_mismatch;                    /* per-thread */
  int next_task, n_tasks, backward;
  pthread_mutex_t *lock;
} job_t;

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* logits and probabilities of one (row, head) block; returns 1 per replaced logit in rep */
static void block_probs(const job_t *J, int i, int h, double *S, double *P, uint8_t *rep, double *lse_out)
{
  const int nq = J->nq, nk = J->nk, c = J->c, H = J->H;
  const double *Q = J->q + ((size_t)i * H + h) * nq * c;
  const double *K = J->k + ((size_t)i * H + h) * nk * c;
  const double inv_sqrt_c = 1.0 / sqrt((double)c);
  for (int j = 0; j < nq; j++) {
    for (int kk = 0; kk < nk; kk++) {
      double dot = 0.0;
      for (int x = 0; x < c; x++) dot += Q[(size_t)j * c + x] * K[(size_t)kk * c + x];
      double s = dot * inv_sqrt_c + J->bias[((size_t)h * nq + j) * nk + kk];
      int r = (J->mask != NULL && J->mask[(size_t)i * nk + kk] == 0);
      if (r) s = MASKED_LOGIT;
      S[(size_t)j * nk + kk] = s;
      rep[(size_t)j * nk + kk] = (uint8_t)r;
    }
    double m = -INFINITY;
    for (int kk = 0; kk < nk; kk++) if (S[(size_t)j * nk + kk] > m) m = S[(size_t)j * nk + kk];
    double l = 0.0;
    for (int kk = 0; kk < nk; kk++) {
      double e = exp(S[(size_t)j * nk + kk] - m);
      P[(size_t)j * nk + kk] = e;
      l += e;
    }
    for (int kk = 0; kk < nk; kk++) P[(size_t)j * nk + kk] /= l;
    lse_out[j] = m + log(l);
  }
}

static void do_task(job_t *J, int task, double *S, double *P, uint8_t *rep, double *dA, double *dP,
                    double *dbias, double *max_mis)
{
  const int H = J->H, nq = J->nq, nk = J->nk, c = J->c;
  const int i = task / H, h = task % H;
  const double *V = J->v + ((size_t)i * H + h) * nk * c;
  const double *Q = J->q + ((size_t)i * H + h) * nq * c;
  const double *K = J->k + ((size_t)i * H + h) * nk * c;
  const double inv_sqrt_c = 1.0 / sqrt((double)c);
  double *lse = J->lse + ((size_t)i * H + h) * nq;
  block_probs(J, i, h, S, P, rep, lse);

  /* a = P v ; o = sigmoid(g) * a */
  double *A = J->attn + ((size_t)i * H + h) * nq * c;
  for (int j = 0; j < nq; j++)
    for (int x = 0; x < c; x++) {
      double acc = 0.0;
      for (int kk = 0; kk < nk; kk++) acc += P[(size_t)j * nk + kk] * V[(size_t)kk * c + x];
      A[(size_t)j * c + x] = acc;
    }
  for (int j = 0; j < nq; j++)
    for (int x = 0; x < c; x++) {
      size_t gi = (((size_t)i * nq + j) * H + h) * c + x;
      J->out[gi] = sigmoid(J->gate[gi]) * A[(size_t)j * c + x];
    }
  if (!J->backward) return;

  /* gate backward */
  for (int j = 0; j < nq; j++)
    for (int x = 0; x < c; x++) {
      size_t gi = (((size_t)i * nq + j) * H + h) * c + x;
      double sg = sigmoid(J->gate[gi]);
      dA[(size_t)j * c + x] = J->dout[gi] * sg;
      J->dgate[gi] = J->dout[gi] * A[(size_t)j * c + x] * sg * (1.0 - sg);
    }
  /* dv = P^T dA */
  double *dV = J->dv + ((size_t)i * H + h) * nk * c;
  for (int kk = 0; kk < nk; kk++)
    for (int x = 0; x < c; x++) {
      double acc = 0.0;
      for (int j = 0; j < nq; j++) acc += P[(size_t)j * nk + kk] * dA[(size_t)j * c + x];
      dV[(size_t)kk * c + x] = acc;
    }
  /* dp = dA v^T ; D = sum_k P dp ; ds = P (dp - D) (zero where replaced) */
  double *Dout = J->D + ((size_t)i * H + h) * nq;
  for (int j = 0; j < nq; j++) {
    double Dj = 0.0;
    for (int kk = 0; kk < nk; kk++) {
      double dp = 0.0;
      for (int x = 0; x < c; x++) dp += dA[(size_t)j * c + x] * V[(size_t)kk * c + x];
      dP[(size_t)j * nk + kk] = dp;
      Dj += P[(size_t)j * nk + kk] * dp;
    }
    Dout[j] = Dj;
    double alt = 0.0, scale = 0.0;
    for (int x = 0; x < c; x++) {
      alt += dA[(size_t)j * c + x] * A[(size_t)j * c + x];
      scale += fabs(dA[(size_t)j * c + x] * A[(size_t)j * c + x]);
    }
    double mis = fabs(alt - Dj) / (scale > 0 ? scale : 1.0);
    if (mis > *max_mis) *max_mis = mis;
    for (int kk = 0; kk < nk; kk++) {
      size_t e = (size_t)j * nk + kk;
      dP[e] = rep[e] ? 0.0 : P[e] * (dP[e] - Dj); /* dP now holds ds */
    }
  }
  /* dq = ds k / sqrt(c) ; dk = ds^T q / sqrt(c) ; dbias += ds */
  double *dQ = J->dq + ((size_t)i * H + h) * nq * c;
  double *dK = J->dk + ((size_t)i * H + h) * nk * c;
  for (int j = 0; j < nq; j++)
    for (int x = 0; x < c; x++) {
      double acc = 0.0;
      for (int kk = 0; kk < nk; kk++) acc += dP[(size_t)j * nk + kk] * K[(size_t)kk * c + x];
      dQ[(size_t)j * c + x] = acc * inv_sqrt_c;
    }
  for (int kk = 0; kk < nk; kk++)
    for (int x = 0; x < c; x++) {
      double acc = 0.0;
      for (int j = 0; j < nq; j++) acc += dP[(size_t)j * nk + kk] * Q[(size_t)j * c + x];
      dK[(size_t)kk * c + x] = acc * inv_sqrt_c;
    }
  for (int j = 0; j < nq; j++)
    for (int kk = 0; kk < nk; kk++)
      dbias[((size_t)h * nq + j) * nk + kk] += dP[(size_t)j * nk + kk];
}

typedef struct { job_t *J; int tid; double max_mis; } worker_arg;

static void *worker(void *p)
{
  worker_arg *W = (worker_arg *)p;
  job_t *J = W->J;
  size_t blk = (size_t)J->nq * J->nk;
  double *S = malloc(blk * sizeof(double)), *P = malloc(blk * sizeof(double));
  double *dP = J->backward ? malloc(blk * sizeof(double)) : NULL;
  double *dA = J->backward ? malloc((size_t)J->nq * J->c * sizeof(double)) : NULL;
  uint8_t *rep = malloc(blk);
  double *dbias = J->backward ? J->dbias_part + (size_t)W->tid * J->H * blk : NULL;
  W->max_mis = 0.0;
  for (;;) {
    pthread_mutex_lock(J->lock);
    int t = J->next_task++;
    pthread_mutex_unlock(J->lock);
    if (t >= J->n_tasks) break;
    do_task(J, t, S, P, rep, dA, dP, dbias, &W->max_mis);
  }
  free(S); free(P); free(dP); free(dA); free(rep);
  return NULL;
}

static int run(job_t *J, int threads)
{
  if (threads <= 0) threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (threads < 1) threads = 1;
  if (threads > J->n_tasks) threads = J->n_tasks > 0 ? J->n_tasks : 1;
  size_t blk = (size_t)J->H * J->nq * J->nk;
  pthread_mutex_t lock = PTHREAD_MUTEX_INITIALIZER;
  J->lock = &lock;
  J->next_task = 0;
  if (J->backward) {
    J->dbias_part = calloc((size_t)threads * blk, sizeof(double));
    if (!J->dbias_part) return -1;
  }
  pthread_t *th = malloc(sizeof(pthread_t) * threads);
  worker_arg *wa = malloc(sizeof(worker_arg) * threads);
  for (int t = 0; t < threads; t++) {
    wa[t].J = J; wa[t].tid = t; wa[t].max_mis = 0.0;
    pthread_create(&th[t], NULL, worker, &wa[t]);
  }
  J->max_d_mismatch = 0.0;
  for (int t = 0; t < threads; t++) {
    pthread_join(th[t], NULL);
    if (wa[t].max_mis > J->max_d_mismatch) J->max_d_mismatch = wa[t].max_mis;
  }
  free(th); free(wa);
  return threads;
}

/* Forward over every (row, head).  Returns the number of threads used. */
int oracle_fwd(int rows, int H, int nq, int nk, int c,
               const double *q, const double *k, const double *v, const double *bias,
               const double *gate, const uint8_t *mask,
               double *out, double *attn, double *lse, int threads)
{
  job_t J; memset(&J, 0, sizeof J);
  J.rows = rows; J.H = H; J.nq = nq; J.nk = nk; J.c = c;
  J.q = q; J.k = k; J.v = v; J.bias = bias; J.gate = gate; J.mask = mask;
  J.out = out; J.attn = attn; J.lse = lse;
  J.n_tasks = rows * H; J.backward = 0;
  return run(&J, threads);
}

/* Forward and backward.  dbias is the sum over the rows given.  *d_mismatch
 * receives the largest relative gap between the two forms of D. */
int oracle_bwd(int rows, int H, int nq, int nk, int c,
               const double *q, const double *k, const double *v, const double *bias,
               const double *gate, const uint8_t *mask, const double *dout,
               double *out, double *attn, double *lse,
               double *dq, double *dk, double *dv, double *dbias, double *dgate, double *D,
               double *d_mismatch, int threads)
{
  job_t J; memset(&J, 0, sizeof J);
  J.rows = rows; J.H = H; J.nq = nq; J.nk = nk; J.c = c;
  J.q = q; J.k = k; J.v = v; J.bias = bias; J.gate = gate; J.mask = mask; J.dout = dout;
  J.out = out; J.attn = attn; J.lse = lse;
  J.dq = dq; J.dk = dk; J.dv = dv; J.dgate = dgate; J.D = D;
  J.n_tasks = rows * H; J.backward = 1;
  int used = run(&J, threads);
  if (used < 0) return used;
  size_t blk = (size_t)H * nq * nk;
  for (size_t e = 0; e < blk; e++) {
    double s = 0.0;
    for (int t = 0; t < used; t++) s += J.dbias_part[(size_t)t * blk + e];
    dbias[e] = s;
  }
  free(J.dbias_part);
  if (d_mismatch) *d_mismatch = J.max_d_mismatch;
  return used;
}
