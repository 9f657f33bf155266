/*
 * KDA recurrence in plain C, fp64 -- TEST INFRASTRUCTURE (CPU oracle).
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg use it; the
 * GPU library neither links nor calls it, and the two share no source.
 *
 * Same definition as oracle/sequential.py (recurrent-form entry of the "xhh.club"
 * tag page 结构; -5 log-decay floor from its chunkwise-form entry), one token at a
 * time:
 *     gt = min(0, max(-5, g)),  S' = Diag(exp(gt)) S,  u = beta (v - S'^T k),
 *     S  = S' + k u^T,          o  = S^T q.
 * Column j of S evolves from column j alone (u_j needs only S'[:, j]), so the work
 * splits exactly into independent (batch, head, column block) units, which run on
 * POSIX threads.  Inputs are the stored bytes: q/k/v as bf16 bit patterns or fp32,
 * g/beta/S0 fp32.  Results are fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define COLS 16   /* value columns per work unit */

static double ld(const void *p, int bf16, size_t i) {
  if (bf16) {
    uint32_t b = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
  }
  return (double)((const float *)p)[i];
}

typedef struct {
  int B, T, H, dk, dv, bf16;
  const void *q, *k, *v;
  const float *g, *beta, *S0;
  double *o, *S_out, *ckpt;
  int ckpt_every;
  int n_units;
  int next;  /* shared work counter */
  pthread_mutex_t mu;
} job_t;

static void run_unit(job_t *J, int unit) {
  const int ncb = (J->dv + COLS - 1) / COLS;
  const int cb = unit % ncb, bh = unit / ncb;
  const int h = bh % J->H, b = bh / J->H;
  const int dk = J->dk, dv = J->dv, H = J->H;
  const int c0 = cb * COLS, nc = (dv - c0) < COLS ? (dv - c0) : COLS;
  double *S = (double *)malloc(sizeof(double) * (size_t)dk * COLS);
  double *a = (double *)malloc(sizeof(double) * (size_t)dk);
  double *kk = (double *)malloc(sizeof(double) * (size_t)dk);
  double *qq = (double *)malloc(sizeof(double) * (size_t)dk);
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < nc; ++j)
      S[i * COLS + j] = J->S0 ? (double)J->S0[(((size_t)b * H + h) * dk + i) * dv + c0 + j] : 0.0;
  for (int t = 0; t < J->T; ++t) {
    const size_t tok = ((size_t)b * J->T + t) * H + h;   /* (b, t, h) */
    const double bt = (double)J->beta[tok];
    for (int i = 0; i < dk; ++i) {
      double gi = (double)J->g[tok * dk + i];
      gi = gi < -5.0 ? -5.0 : gi;
      gi = gi > 0.0 ? 0.0 : gi;
      a[i] = exp(gi);
      kk[i] = ld(J->k, J->bf16, tok * dk + i);
      qq[i] = ld(J->q, J->bf16, tok * dk + i);
    }
    double e[COLS], u[COLS], oo[COLS];
    for (int j = 0; j < nc; ++j) e[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
      double *row = S + i * COLS;
      for (int j = 0; j < nc; ++j) {
        row[j] *= a[i];
        e[j] += row[j] * kk[i];
      }
    }
    for (int j = 0; j < nc; ++j) u[j] = bt * (ld(J->v, J->bf16, tok * dv + c0 + j) - e[j]);
    for (int j = 0; j < nc; ++j) oo[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
      double *row = S + i * COLS;
      for (int j = 0; j < nc; ++j) {
        row[j] += kk[i] * u[j];
        oo[j] += row[j] * qq[i];
      }
    }
    if (J->o)
      for (int j = 0; j < nc; ++j) J->o[tok * dv + c0 + j] = oo[j];
    if (J->ckpt && J->ckpt_every > 0 && (t + 1) % J->ckpt_every == 0) {
      const size_t m = (size_t)(t + 1) / J->ckpt_every - 1, nm = (size_t)J->T / J->ckpt_every;
      double *dst = J->ckpt + (((size_t)b * nm + m) * H + h) * (size_t)dk * dv;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nc; ++j) dst[(size_t)i * dv + c0 + j] = S[i * COLS + j];
    }
  }
  if (J->S_out)
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < nc; ++j)
        J->S_out[(((size_t)b * H + h) * dk + i) * dv + c0 + j] = S[i * COLS + j];
  free(S);
  free(a);
  free(kk);
  free(qq);
}

static void *worker(void *arg) {
  job_t *J = (job_t *)arg;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    const int u = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (u >= J->n_units) break;
    run_unit(J, u);
  }
  return NULL;
}

static void run_all(job_t *J, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > J->n_units) nthreads = J->n_units;
  pthread_mutex_init(&J->mu, NULL);
  J->next = 0;
  if (nthreads <= 1) {
    worker(J);
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&J->mu);
}

/* Prefill over [B,T,H,*] token-major inputs.  o: [B,T,H,dv] or NULL; S_out:
 * [B,H,dk,dv] or NULL; ckpt: [B, T/ckpt_every, H, dk, dv] or NULL (state after the
 * first m*ckpt_every tokens).  Returns 0, or -1 on bad arguments. */
int kda_oracle_prefill(int B, int T, int H, int dk, int dv, int in_bf16, const void *q,
                       const void *k, const void *v, const float *g, const float *beta,
                       const float *S0, double *o, double *S_out, int ckpt_every, double *ckpt,
                       int nthreads) {
  if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1 || !q || !k || !v || !g || !beta) return -1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv; J.bf16 = in_bf16;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S0;
  J.o = o; J.S_out = S_out; J.ckpt = ckpt; J.ckpt_every = ckpt_every;
  J.n_units = B * H * ((dv + COLS - 1) / COLS);
  if (J.n_units == 0) return 0;
  run_all(&J, nthreads);
  return 0;
}

/* One decode step for N sequences: inputs [N,H,*] (T = 1), state [N,H,dk,dv] fp64 in
 * and out, o [N,H,dv] fp64. */
typedef struct {
  int N, H, dk, dv, bf16;
  const void *q, *k, *v;
  const float *g, *beta;
  double *state, *o;
  int n_units, next;
  pthread_mutex_t mu;
} djob_t;

static void *dworker(void *arg) {
  djob_t *J = (djob_t *)arg;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    const int u = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (u >= J->n_units) break;
    const size_t nh = (size_t)u, dk = (size_t)J->dk, dv = (size_t)J->dv;
    double *S = J->state + nh * dk * dv;
    double *e = (double *)calloc(dv, sizeof(double));
    double *oo = (double *)calloc(dv, sizeof(double));
    for (size_t i = 0; i < dk; ++i) {
      double gi = (double)J->g[nh * dk + i];
      gi = gi < -5.0 ? -5.0 : (gi > 0.0 ? 0.0 : gi);
      const double a = exp(gi), ki = ld(J->k, J->bf16, nh * dk + i);
      for (size_t j = 0; j < dv; ++j) {
        S[i * dv + j] *= a;
        e[j] += S[i * dv + j] * ki;
      }
    }
    const double bt = (double)J->beta[nh];
    for (size_t j = 0; j < dv; ++j) e[j] = bt * (ld(J->v, J->bf16, nh * dv + j) - e[j]);
    for (size_t i = 0; i < dk; ++i) {
      const double ki = ld(J->k, J->bf16, nh * dk + i), qi = ld(J->q, J->bf16, nh * dk + i);
      for (size_t j = 0; j < dv; ++j) {
        S[i * dv + j] += ki * e[j];
        oo[j] += S[i * dv + j] * qi;
      }
    }
    for (size_t j = 0; j < dv; ++j) J->o[nh * dv + j] = oo[j];
    free(e);
    free(oo);
  }
  return NULL;
}

int kda_oracle_decode_step(int N, int H, int dk, int dv, int in_bf16, const void *q, const void *k,
                           const void *v, const float *g, const float *beta, double *state,
                           double *o, int nthreads) {
  if (N < 0 || H < 0 || dk < 1 || dv < 1 || !q || !k || !v || !g || !beta || !state || !o)
    return -1;
  djob_t J;
  memset(&J, 0, sizeof J);
  J.N = N; J.H = H; J.dk = dk; J.dv = dv; J.bf16 = in_bf16;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.state = state; J.o = o;
  J.n_units = N * H;
  if (J.n_units == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > J.n_units) nthreads = J.n_units;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads <= 1) {
    dworker(&J);
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, dworker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&J.mu);
  return 0;
}
