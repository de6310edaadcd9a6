/*
 * la_oracle.c -- plain, slow, fp64 CPU oracle for causal linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the bench use it.  It shares no code with the HIP library.
 *
 * What it computes (one head at a time, token by token):
 *
 *   S   <- a_t * S + phi(k_t) v_t^T           S is d_k x d_v, rows = key dim
 *   o_t <- phi(q_t)^T S                       read AFTER the write (self-inclusive)
 *
 * Sources (titles and sections of the pages this follows):
 *  - "Linear / Sparse Attention - minimal runnable implementation",
 *    linear_attn_recurrent: the d_k x d_v state, the outer-product write
 *    k v^T and the update-then-read order.
 *  - CS336 lecture 4 code 1 "linear attention", section 4 (forgetting):
 *    gated_linear_attention_recurrent: the decayed recurrence
 *    S_t = gamma_t S_{t-1} + k_t v_t^T with gamma_t in (0, 1]; the decay
 *    multiplies the previous state only, never the current write.
 *  - "adv13 -- Linear Attention / SSM", section 3.2 / 4.2: the feature map
 *    phi is applied to q and k (not v); phi(x) = elu(x) + 1 (alpha = 1).
 *  - Linear/sparse attention tutorial, section 2.4: RetNet keeps one fixed
 *    gamma per head; section 3.3 / 4.2: the Mamba-style scalar decay
 *    a_t = exp(Delta_t * A) with Delta_t = softplus(g_t), here A = -1, so
 *    a_t = exp(-softplus(g_t)).
 *
 * The normalised variant (the linear/sparse attention tutorial, section 2.2,
 * boxed recurrence) also carries z_t = a_t z_{t-1} + phi(k_t) (the decay acts
 * on z as on S: z is S's extra value column of ones, tutorial section 6.2)
 * and returns o_t = phi(q_t)^T S_t / phi(q_t)^T z_t, with no term added to the
 * denominator (the pages give none).
 *
 * The delta rule (DeltaNet; with a_t, Gated DeltaNet) is the second
 * recurrence here ("Linear / Sparse Attention - minimal runnable
 * implementation", delta_rule_recurrent; the tutorial, section 5.1-5.2, Q15
 * and Q17).  The pages write it with a d_v x d_k state S' that maps keys to
 * values, S'_t = a_t S'_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T; the
 * state here is its transpose S = S'^T (d_k x d_v, the orientation of the
 * linear-attention state), so the same step reads
 *
 *   S   <- a_t (S - beta_t k_t (k_t^T S)) + beta_t k_t v_t^T
 *   o_t <- q_t^T S                            read AFTER the write
 *
 * (the erase acts on the decayed previous state, the write is undecayed;
 * the keys are taken as given: the pages normalise them before the call).
 *
 * Decay kinds (same numbering as the library's public enum, redeclared here
 * on purpose so that the two sides share no header):
 *   0 none        a_t = 1
 *   1 per head    a_t = gamma[h]                   (data: gamma[H])
 *   2 log decay   a_t = exp(log_a[b,h,t])          (data: log_a[B,H,L])
 *   3 gate        a_t = exp(-softplus(g[b,h,t]))   (data: g[B,H,L])
 *   4 per channel a_t = diag(exp(log_a[b,h,t,:]))  (data: log_a[B,H,L,dk])
 *     GLA's data-dependent diagonal gate (the tutorial, section 2.4):
 *     S_t = diag(alpha_t) S_{t-1} + k_t v_t^T, one factor per key channel
 *     (row of S), so it scales the previous state row by row.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_PHI_IDENTITY 0
#define ORACLE_PHI_ELU1 1

#define ORACLE_DECAY_NONE 0
#define ORACLE_DECAY_HEAD 1
#define ORACLE_DECAY_LOG 2
#define ORACLE_DECAY_GATE 3
#define ORACLE_DECAY_CHANNEL 4

/* phi(x) = elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) for x <= 0. */
static double oracle_phi(int phi, double x) {
  if (phi == ORACLE_PHI_ELU1) return x > 0.0 ? x + 1.0 : exp(x);
  return x;
}

/* softplus(g) = log(1 + e^g), written so that neither branch overflows. */
static double oracle_softplus(double g) {
  return (g > 0.0 ? g : 0.0) + log1p(exp(-fabs(g)));
}

/* Decay a_t of token t of head (b,h).  `dh` points at the head's decay data:
 * gamma[h] for kind 1, the head's [L] row for kinds 2 and 3. */
static double oracle_decay(int kind, const double* dh, int t) {
  switch (kind) {
    case ORACLE_DECAY_HEAD: return dh[0];
    case ORACLE_DECAY_LOG: return exp(dh[t]);
    case ORACLE_DECAY_GATE: return exp(-oracle_softplus(dh[t]));
    default: return 1.0;
  }
}

/*
 * One head, L tokens, token by token.
 *   q, k : [L, dk]   v : [L, dv]   out : [L, dv]   S : [dk, dv] (in: S_0, out: S_L)
 *   dh   : decay data of this head (see oracle_decay), may be NULL for kind 0;
 *          for kind 4 the head's [L, dk] log_a rows
 *   z    : NULL (un-normalised) or the normaliser [dk] (in: z_0, out: z_L)
 */
void oracle_recurrent_head(int L, int dk, int dv, const double* q, const double* k,
                           const double* v, int phi, int decay_kind, const double* dh,
                           double* S, double* z, double* out) {
  double* fq = (double*)malloc(sizeof(double) * (size_t)dk);
  double* fk = (double*)malloc(sizeof(double) * (size_t)dk);
  for (int t = 0; t < L; ++t) {
    const double* qt = q + (size_t)t * dk;
    const double* kt = k + (size_t)t * dk;
    const double* vt = v + (size_t)t * dv;
    for (int i = 0; i < dk; ++i) {
      fq[i] = oracle_phi(phi, qt[i]);
      fk[i] = oracle_phi(phi, kt[i]);
    }
    const double a = oracle_decay(decay_kind, dh, t);
    /* write: S = a S + phi(k_t) v_t^T (kind 4: row i decays by exp(log_a[t][i])) */
    for (int i = 0; i < dk; ++i) {
      const double ai = decay_kind == ORACLE_DECAY_CHANNEL ? exp(dh[(size_t)t * dk + i]) : a;
      for (int j = 0; j < dv; ++j)
        S[(size_t)i * dv + j] = ai * S[(size_t)i * dv + j] + fk[i] * vt[j];
    }
    /* normaliser: z = a z + phi(k_t), den = phi(q_t)^T z */
    double den = 1.0;
    if (z) {
      den = 0.0;
      for (int i = 0; i < dk; ++i) {
        const double ai = decay_kind == ORACLE_DECAY_CHANNEL ? exp(dh[(size_t)t * dk + i]) : a;
        z[i] = ai * z[i] + fk[i];
        den += fq[i] * z[i];
      }
    }
    /* read: o_t = phi(q_t)^T S (the state that already holds token t) */
    double* ot = out + (size_t)t * dv;
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += fq[i] * S[(size_t)i * dv + j];
      ot[j] = z ? acc / den : acc;
    }
  }
  free(fq);
  free(fk);
}

typedef struct {
  int B, H, L, dk, dv, phi, kind;
  const double *q, *k, *v, *decay;
  double *S, *Z, *out;
  int first, last; /* head range [first, last) of this thread */
} oracle_job;

static void* oracle_worker(void* p) {
  oracle_job* j = (oracle_job*)p;
  for (int bh = j->first; bh < j->last; ++bh) {
    const int h = bh % j->H;
    const double* dh = NULL;
    if (j->kind == ORACLE_DECAY_HEAD) dh = j->decay + h;
    else if (j->kind == ORACLE_DECAY_LOG || j->kind == ORACLE_DECAY_GATE)
      dh = j->decay + (size_t)bh * j->L;
    else if (j->kind == ORACLE_DECAY_CHANNEL)
      dh = j->decay + (size_t)bh * j->L * j->dk;
    oracle_recurrent_head(j->L, j->dk, j->dv, j->q + (size_t)bh * j->L * j->dk,
                          j->k + (size_t)bh * j->L * j->dk, j->v + (size_t)bh * j->L * j->dv,
                          j->phi, j->kind, dh, j->S + (size_t)bh * j->dk * j->dv,
                          j->Z ? j->Z + (size_t)bh * j->dk : NULL,
                          j->out + (size_t)bh * j->L * j->dv);
  }
  return NULL;
}

/*
 * All heads of a [B, H, L, d] problem, heads spread over `nthreads` threads.
 *   q, k : [B,H,L,dk]  v : [B,H,L,dv]  out : [B,H,L,dv]  S : [B,H,dk,dv] in/out
 *   decay: NULL | gamma[H] | log_a or g [B,H,L] | log_a [B,H,L,dk]
 *   Z    : NULL (un-normalised) or the normaliser state [B,H,dk] in/out
 * Returns the number of threads actually used.
 */
int oracle_recurrent_norm(int B, int H, int L, int dk, int dv, const double* q, const double* k,
                          const double* v, int phi, int decay_kind, const double* decay,
                          double* S, double* Z, double* out, int nthreads) {
  const int heads = B * H;
  if (heads <= 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > heads) nthreads = heads;
  oracle_job* jobs = (oracle_job*)calloc((size_t)nthreads, sizeof(oracle_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    oracle_job* j = &jobs[i];
    j->B = B; j->H = H; j->L = L; j->dk = dk; j->dv = dv; j->phi = phi; j->kind = decay_kind;
    j->q = q; j->k = k; j->v = v; j->decay = decay; j->S = S; j->Z = Z; j->out = out;
    j->first = (int)((long long)heads * i / nthreads);
    j->last = (int)((long long)heads * (i + 1) / nthreads);
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, oracle_worker, &jobs[i]);
  oracle_worker(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(jobs);
  free(th);
  return nthreads;
}

/* The un-normalised recurrence (no z). */
int oracle_recurrent(int B, int H, int L, int dk, int dv, const double* q, const double* k,
                     const double* v, int phi, int decay_kind, const double* decay, double* S,
                     double* out, int nthreads) {
  return oracle_recurrent_norm(B, H, L, dk, dv, q, k, v, phi, decay_kind, decay, S, NULL, out,
                               nthreads);
}

/*
 * The delta rule, one head, L tokens, token by token.
 *   q, k : [L, dk]   v : [L, dv]   beta : [L]   out : [L, dv]
 *   S    : [dk, dv] (in: S_0, out: S_L)
 *   dh   : decay data of this head (kinds 0-3 as above), may be NULL for kind 0
 */
void oracle_delta_head(int L, int dk, int dv, const double* q, const double* k, const double* v,
                       const double* beta, int decay_kind, const double* dh, double* S,
                       double* out) {
  double* r = (double*)malloc(sizeof(double) * (size_t)dv);
  for (int t = 0; t < L; ++t) {
    const double* qt = q + (size_t)t * dk;
    const double* kt = k + (size_t)t * dk;
    const double* vt = v + (size_t)t * dv;
    const double a = oracle_decay(decay_kind, dh, t);
    const double bt = beta[t];
    /* what the previous state returns for k_t: r = k_t^T S_{t-1} */
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += kt[i] * S[(size_t)i * dv + j];
      r[j] = acc;
    }
    /* erase along k_t, decay, then write: S = a (S - beta k r^T) + beta k v^T */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j)
        S[(size_t)i * dv + j] = a * (S[(size_t)i * dv + j] - bt * kt[i] * r[j]) + bt * kt[i] * vt[j];
    /* read: o_t = q_t^T S */
    double* ot = out + (size_t)t * dv;
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += qt[i] * S[(size_t)i * dv + j];
      ot[j] = acc;
    }
  }
  free(r);
}

typedef struct {
  int H, L, dk, dv, kind;
  const double *q, *k, *v, *beta, *decay;
  double *S, *out;
  int first, last;
} oracle_delta_job;

static void* oracle_delta_worker(void* p) {
  oracle_delta_job* j = (oracle_delta_job*)p;
  for (int bh = j->first; bh < j->last; ++bh) {
    const int h = bh % j->H;
    const double* dh = NULL;
    if (j->kind == ORACLE_DECAY_HEAD) dh = j->decay + h;
    else if (j->kind == ORACLE_DECAY_LOG || j->kind == ORACLE_DECAY_GATE)
      dh = j->decay + (size_t)bh * j->L;
    oracle_delta_head(j->L, j->dk, j->dv, j->q + (size_t)bh * j->L * j->dk,
                      j->k + (size_t)bh * j->L * j->dk, j->v + (size_t)bh * j->L * j->dv,
                      j->beta + (size_t)bh * j->L, j->kind, dh,
                      j->S + (size_t)bh * j->dk * j->dv, j->out + (size_t)bh * j->L * j->dv);
  }
  return NULL;
}

/*
 * The delta rule over all heads of a [B, H, L, d] problem.
 *   q, k : [B,H,L,dk]  v : [B,H,L,dv]  beta : [B,H,L]  out : [B,H,L,dv]
 *   S    : [B,H,dk,dv] in/out   decay: NULL | gamma[H] | log_a or g [B,H,L]
 * Returns the number of threads actually used.
 */
int oracle_delta(int B, int H, int L, int dk, int dv, const double* q, const double* k,
                 const double* v, const double* beta, int decay_kind, const double* decay,
                 double* S, double* out, int nthreads) {
  const int heads = B * H;
  if (heads <= 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > heads) nthreads = heads;
  oracle_delta_job* jobs = (oracle_delta_job*)calloc((size_t)nthreads, sizeof(oracle_delta_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    oracle_delta_job* j = &jobs[i];
    j->H = H; j->L = L; j->dk = dk; j->dv = dv; j->kind = decay_kind;
    j->q = q; j->k = k; j->v = v; j->beta = beta; j->decay = decay; j->S = S; j->out = out;
    j->first = (int)((long long)heads * i / nthreads);
    j->last = (int)((long long)heads * (i + 1) / nthreads);
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, oracle_delta_worker, &jobs[i]);
  oracle_delta_worker(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(jobs);
  free(th);
  return nthreads;
}
