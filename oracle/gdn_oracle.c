/*
 * gdn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64, token-by-token CPU implementation of the gated delta
 * rule (the GatedDeltaNet linear-attention core that the XTuner / Ascend 910C
 * Qwen3.5-2B training article rebuilds natively, section 3.1.2 "GDN linear
 * attention rebuilt natively in Ascend C", Fig. 7 and Fig. 8).
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header or build step with the
 * HIP library under linear_attention_gated_amd/.
 *
 * What it computes, per sequence n and head h, independently:
 *
 *   S <- initial state (d_v x d_k; zeros when h0 is NULL)
 *   for each token t of the sequence, in order:
 *       a   = exp(g_t)
 *       S   = a * S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *       o_t = scale * S q_t
 *   final state = S
 *
 * The article names the operator but prints no formula; the recurrence above
 * is the standard gated delta rule of GatedDeltaNet, written out literally:
 * the decay multiplies the previous state before the delta correction.
 *
 * States cross the interface transposed, as the d_k x d_v matrix h = S^T,
 * stored [N][H][d_k][d_v] (element (i, j) is S[j][i]).
 *
 * The backward is reverse-mode differentiation of the same loop for the loss
 *   L = sum_t <do_t, o_t> + <dS_T, S_T>      (dS_T = dht^T, zero if absent)
 * With Y = dL/dS_t (d_v x d_k), walking t = T..1:
 *   Y    += scale * do_t q_t^T
 *   dq_t  = scale * S_t^T do_t
 *   e     = S_{t-1} k_t,  w = Y k_t                      (both length d_v)
 *   dv_t  = beta_t w
 *   dbeta = w . (v_t - a e)
 *   dk_t  = beta_t Y^T v_t - a beta_t (S_{t-1}^T w + Y^T e)
 *   dg_t  = a (<Y, S_{t-1}>_F - beta_t w . e)
 *   Y     = a (Y - beta_t w k_t^T)                        (now dL/dS_{t-1})
 * and dh0 = Y^T after the first token.  S_{t-1} is recomputed per segment of
 * CKPT tokens from a forward checkpoint taken at the segment start.
 *
 * Layouts (all fp64, contiguous, last index fastest):
 *   q, k, dq, dk: [total_tokens][H][dk];  v, o, do, dv: [total_tokens][H][dv]
 *   g, beta, dg, dbeta: [total_tokens][H]
 *   h0, ht, dht, dh0: [N][H][dk][dv]
 * Sequence n covers tokens [cu[n], cu[n+1]).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define CKPT 64

typedef struct {
  int64_t nseq, H, dk, dv;
  const int64_t* cu;
  double scale;
  const double *q, *k, *v, *g, *beta, *h0, *dO, *dht;
  double *o, *ht, *dq, *dk_, *dv_, *dg, *dbeta, *dh0;
  int backward;
  int64_t next_unit; /* work counter, taken atomically */
  int status;
} job_t;

/* S (dv x dk, row-major) <- a S (I - b k k^T) + b v k^T, literally:
 * first the delta-corrected product S (I - b k k^T) = S - b (S k) k^T,
 * then the decay, then the write. */
static void step_state(double* S, int64_t dk, int64_t dv, const double* kt,
                       const double* vt, double a, double b, double* e) {
  for (int64_t j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int64_t i = 0; i < dk; ++i) acc += S[j * dk + i] * kt[i];
    e[j] = acc;
  }
  for (int64_t j = 0; j < dv; ++j)
    for (int64_t i = 0; i < dk; ++i)
      S[j * dk + i] = a * (S[j * dk + i] - b * e[j] * kt[i]) + b * vt[j] * kt[i];
}

static void load_state(double* S, const double* h, int64_t dk, int64_t dv) {
  /* h is [dk][dv] holding S^T */
  if (!h) {
    memset(S, 0, sizeof(double) * dk * dv);
    return;
  }
  for (int64_t i = 0; i < dk; ++i)
    for (int64_t j = 0; j < dv; ++j) S[j * dk + i] = h[i * dv + j];
}

static void store_state(double* h, const double* S, int64_t dk, int64_t dv) {
  for (int64_t i = 0; i < dk; ++i)
    for (int64_t j = 0; j < dv; ++j) h[i * dv + j] = S[j * dk + i];
}

static int fwd_unit(job_t* J, int64_t n, int64_t hh) {
  const int64_t H = J->H, dk = J->dk, dv = J->dv;
  const int64_t t0 = J->cu[n], t1 = J->cu[n + 1];
  double* S = (double*)malloc(sizeof(double) * dk * dv);
  double* e = (double*)malloc(sizeof(double) * dv);
  if (!S || !e) { free(S); free(e); return -1; }
  load_state(S, J->h0 ? J->h0 + (n * H + hh) * dk * dv : NULL, dk, dv);
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t th = t * H + hh;
    const double* qt = J->q + th * dk;
    const double* kt = J->k + th * dk;
    const double* vt = J->v + th * dv;
    step_state(S, dk, dv, kt, vt, exp(J->g[th]), J->beta[th], e);
    double* ot = J->o + th * dv;
    for (int64_t j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int64_t i = 0; i < dk; ++i) acc += S[j * dk + i] * qt[i];
      ot[j] = J->scale * acc;
    }
  }
  if (J->ht) store_state(J->ht + (n * H + hh) * dk * dv, S, dk, dv);
  free(S);
  free(e);
  return 0;
}

static int bwd_unit(job_t* J, int64_t n, int64_t hh) {
  const int64_t H = J->H, dk = J->dk, dv = J->dv, D2 = dk * dv;
  const int64_t t0 = J->cu[n], t1 = J->cu[n + 1], len = t1 - t0;
  const int64_t nseg = (len + CKPT - 1) / CKPT;
  /* checkpoints: state entering each segment */
  double* ck = (double*)malloc(sizeof(double) * D2 * (nseg > 0 ? nseg : 1));
  /* states inside one segment: seg[0] = entering state, seg[u+1] = after token u */
  double* seg = (double*)malloc(sizeof(double) * D2 * (CKPT + 1));
  double* Y = (double*)malloc(sizeof(double) * D2);
  double* e = (double*)malloc(sizeof(double) * dv);
  double* w = (double*)malloc(sizeof(double) * dv);
  if (!ck || !seg || !Y || !e || !w) {
    free(ck); free(seg); free(Y); free(e); free(w);
    return -1;
  }
  /* forward sweep storing checkpoints */
  double* S = seg; /* reuse as running state */
  load_state(S, J->h0 ? J->h0 + (n * H + hh) * D2 : NULL, dk, dv);
  for (int64_t s = 0; s < nseg; ++s) {
    memcpy(ck + s * D2, S, sizeof(double) * D2);
    const int64_t a0 = t0 + s * CKPT;
    const int64_t a1 = (a0 + CKPT < t1) ? a0 + CKPT : t1;
    for (int64_t t = a0; t < a1; ++t) {
      const int64_t th = t * H + hh;
      step_state(S, dk, dv, J->k + th * dk, J->v + th * dv, exp(J->g[th]), J->beta[th], e);
    }
  }
  /* Y = dL/dS_T = dht^T */
  load_state(Y, J->dht ? J->dht + (n * H + hh) * D2 : NULL, dk, dv);
  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t a0 = t0 + s * CKPT;
    const int64_t a1 = (a0 + CKPT < t1) ? a0 + CKPT : t1;
    /* recompute the segment's states from its checkpoint */
    memcpy(seg, ck + s * D2, sizeof(double) * D2);
    for (int64_t t = a0; t < a1; ++t) {
      const int64_t u = t - a0;
      const int64_t th = t * H + hh;
      memcpy(seg + (u + 1) * D2, seg + u * D2, sizeof(double) * D2);
      step_state(seg + (u + 1) * D2, dk, dv, J->k + th * dk, J->v + th * dv, exp(J->g[th]),
                 J->beta[th], e);
    }
    for (int64_t t = a1 - 1; t >= a0; --t) {
      const int64_t u = t - a0;
      const int64_t th = t * H + hh;
      const double* St = seg + (u + 1) * D2;
      const double* Sp = seg + u * D2;
      const double* qt = J->q + th * dk;
      const double* kt = J->k + th * dk;
      const double* vt = J->v + th * dv;
      const double* dot = J->dO + th * dv;
      const double a = exp(J->g[th]), b = J->beta[th];
      /* Y += scale do q^T ; dq = scale S_t^T do */
      for (int64_t j = 0; j < dv; ++j)
        for (int64_t i = 0; i < dk; ++i) Y[j * dk + i] += J->scale * dot[j] * qt[i];
      double* dqt = J->dq + th * dk;
      for (int64_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) acc += St[j * dk + i] * dot[j];
        dqt[i] = J->scale * acc;
      }
      /* e = S_{t-1} k, w = Y k */
      for (int64_t j = 0; j < dv; ++j) {
        double ae = 0.0, aw = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
          ae += Sp[j * dk + i] * kt[i];
          aw += Y[j * dk + i] * kt[i];
        }
        e[j] = ae;
        w[j] = aw;
      }
      double* dvt = J->dv_ + th * dv;
      double db = 0.0, we = 0.0;
      for (int64_t j = 0; j < dv; ++j) {
        dvt[j] = b * w[j];
        db += w[j] * (vt[j] - a * e[j]);
        we += w[j] * e[j];
      }
      J->dbeta[th] = db;
      double* dkt = J->dk_ + th * dk;
      for (int64_t i = 0; i < dk; ++i) {
        double yv = 0.0, sw = 0.0, ye = 0.0;
        for (int64_t j = 0; j < dv; ++j) {
          yv += Y[j * dk + i] * vt[j];
          sw += Sp[j * dk + i] * w[j];
          ye += Y[j * dk + i] * e[j];
        }
        dkt[i] = b * yv - a * b * (sw + ye);
      }
      double ys = 0.0;
      for (int64_t x = 0; x < D2; ++x) ys += Y[x] * Sp[x];
      J->dg[th] = a * (ys - b * we);
      /* Y <- a (Y - b w k^T) */
      for (int64_t j = 0; j < dv; ++j)
        for (int64_t i = 0; i < dk; ++i) Y[j * dk + i] = a * (Y[j * dk + i] - b * w[j] * kt[i]);
    }
  }
  if (J->dh0) store_state(J->dh0 + (n * H + hh) * D2, Y, dk, dv);
  free(ck); free(seg); free(Y); free(e); free(w);
  return 0;
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int64_t units = J->nseq * J->H;
  for (;;) {
    int64_t u = __atomic_fetch_add(&J->next_unit, 1, __ATOMIC_RELAXED);
    if (u >= units) break;
    int rc = J->backward ? bwd_unit(J, u / J->H, u % J->H) : fwd_unit(J, u / J->H, u % J->H);
    if (rc) __atomic_store_n(&J->status, rc, __ATOMIC_RELAXED);
  }
  return NULL;
}

static int run(job_t* J, int nthreads) {
  const int64_t units = J->nseq * J->H;
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  J->next_unit = 0;
  J->status = 0;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  if (!th) return -1;
  int started = 0;
  for (int i = 1; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, worker, J) != 0) break;
    ++started;
  }
  worker(J);
  for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
  free(th);
  return J->status;
}

/* Number of threads a call with this problem and request would use. */
int gdn_oracle_threads(int64_t nseq, int64_t H, int nthreads) {
  const int64_t units = nseq * H;
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  return nthreads;
}

int gdn_oracle_fwd(int64_t nseq, const int64_t* cu, int64_t H, int64_t dk, int64_t dv,
                   double scale, const double* q, const double* k, const double* v,
                   const double* g, const double* beta, const double* h0, double* o,
                   double* ht, int nthreads) {
  job_t J;
  memset(&J, 0, sizeof(J));
  J.nseq = nseq; J.cu = cu; J.H = H; J.dk = dk; J.dv = dv; J.scale = scale;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.o = o; J.ht = ht;
  J.backward = 0;
  return run(&J, nthreads);
}

int gdn_oracle_bwd(int64_t nseq, const int64_t* cu, int64_t H, int64_t dk, int64_t dv,
                   double scale, const double* q, const double* k, const double* v,
                   const double* g, const double* beta, const double* h0, const double* dO,
                   const double* dht, double* dq, double* dk_, double* dv_, double* dg,
                   double* dbeta, double* dh0, int nthreads) {
  job_t J;
  memset(&J, 0, sizeof(J));
  J.nseq = nseq; J.cu = cu; J.H = H; J.dk = dk; J.dv = dv; J.scale = scale;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.dO = dO; J.dht = dht;
  J.dq = dq; J.dk_ = dk_; J.dv_ = dv_; J.dg = dg; J.dbeta = dbeta; J.dh0 = dh0;
  J.backward = 1;
  return run(&J, nthreads);
}
