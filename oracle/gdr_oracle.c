/*
 * gdr_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct fp64 CPU evaluation of the gated delta
 * rule, token by token.  It exists to check the GPU library against; only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header or constant with the HIP path.
 *
 * What it computes (Systolic Linear Attention paper, section 2.1, Eq. (2),
 * "Gated Delta Recurrence in GDN and KDA"): for every batch b and value head
 * h_v, with key head h_k = h_v / (H_v / H_k), starting from S_0 = h0 (or 0),
 *
 *     F_t  = diag(exp(log_alpha_t))            decay first,
 *     S_t  = F_t S_{t-1} + beta_t k_t (v_t - (F_t S_{t-1})^T k_t)^T
 *          = (I - beta_t k_t k_t^T) F_t S_{t-1} + beta_t k_t v_t^T,
 *     o_t  = S_t^T q_t                          readout after the update.
 *
 * The gate has G decay groups (same paper, section 2.1, the text after
 * Eq. (2); section 2.3 for the four-tile gate): G = 1 is the scalar
 * Gated DeltaNet gate, G = d_k the per-channel KDA gate, and any other G
 * splits the d_k key channels into G contiguous tiles of d_k/G channels that
 * share one decay.  Channel i uses group i / (d_k / G).
 *
 * Value heads that share a key head (grouped value heads, section 2.4.1) are
 * contiguous: h_v in [R*h_k, R*h_k + R).  beta is per value head unless
 * beta_per_key_head is set (then it is indexed by h_k, as in the SLA layer).
 *
 * Inputs arrive as fp32 arrays (bf16 inputs decode to fp32 exactly) and are
 * promoted to fp64; everything after that is fp64.
 *
 * Layouts (row-major, contiguous):
 *   q, k       [B, T, H_k, d_k]
 *   v          [B, T, H_v, d_v]
 *   beta       [B, T, H_v]   (or [B, T, H_k] when beta_per_key_head)
 *   log_alpha  [B, T, H_k, G]
 *   h0, hT     [B, H_v, d_k, d_v]   (h0 may be NULL: zero state; hT may be NULL)
 *   o          [B, T, H_v, d_v]
 *
 * units: optional list of n_units indices u = b * H_v + h_v to evaluate (the
 * others are left untouched); NULL evaluates every (b, h_v).
 * Returns 0 on success, -1 on a malformed problem.
 *
 * oracle_gdr_layer adds the two sequence-level features of the Systolic
 * Linear Attention layer (Table 2, the symbols Z_c, mu and kappa_c; section
 * 2.3, "Why chunk-level momentum"):
 *
 *   Document resets.  reset [B, T] (bytes, NULL = none): reset[b, t] != 0
 *   means token t starts a new document, so the state carried into it is
 *   discarded: S_{t-1} <- 0 before the step above.
 *
 *   Chunk-boundary momentum.  With chunk C > 0 and coefficient mu, the
 *   sequence is cut into chunks of C tokens from its first token (the last
 *   one may be shorter).  Over chunk c the state evolves token by token from
 *   the chunk-entry state S_{c-1} as above (outputs are read from it, token
 *   by token) to S~_c.  At the chunk's end, with F_c the product of the
 *   chunk's decays and kappa_c = 0 when any reset falls inside the chunk
 *   (else 1):
 *     carry = kappa_c F_c S_{c-1}        (cross-document carry discarded)
 *     Z_c   = mu kappa_c Z_{c-1} + (S~_c - carry)
 *     S_c   = carry + Z_c.
 *   Z_0 = z0 (NULL = zero); zT = Z after the last chunk.  mu = 0 skips the
 *   chunk-end step, so the result is the plain recurrence bit for bit.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int B, T, Hk, Hv, dk, dv, G, beta_per_key_head;
  const float *q, *k, *v, *beta, *log_alpha;
  const unsigned char *reset;
  const double *h0, *z0;
  int chunk;
  double momentum;
  double *o, *hT, *zT;
  const int *units;
  int n_units;
  int next; /* work counter, guarded by mu */
  pthread_mutex_t mu;
} job_t;

static void run_unit(const job_t *j, int u) {
  const int Hv = j->Hv, Hk = j->Hk, dk = j->dk, dv = j->dv, G = j->G, T = j->T;
  const int b = u / Hv, hv = u % Hv, R = Hv / Hk, hk = hv / R;
  const int group_width = dk / G;
  double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
  double *f = (double *)malloc(sizeof(double) * (size_t)dk);
  double *kv = (double *)malloc(sizeof(double) * (size_t)dk);
  double *qv = (double *)malloc(sizeof(double) * (size_t)dk);
  double *uu = (double *)malloc(sizeof(double) * (size_t)dv);
  const size_t nS = (size_t)dk * dv;
  const int mom = j->chunk > 0 && j->momentum != 0.0;
  double *S_in = (double *)malloc(sizeof(double) * nS);  /* chunk-entry state S_{c-1} */
  double *Z = (double *)malloc(sizeof(double) * nS);     /* momentum buffer Z_{c-1} */
  double *Fc = (double *)malloc(sizeof(double) * (size_t)dk);  /* product of the chunk's decays */
  int kappa = 1;
  const size_t state_off = ((size_t)b * Hv + hv) * nS;
  if (j->h0) {
    memcpy(S, j->h0 + state_off, sizeof(double) * nS);
  } else {
    memset(S, 0, sizeof(double) * nS);
  }
  if (j->z0) {
    memcpy(Z, j->z0 + state_off, sizeof(double) * nS);
  } else {
    memset(Z, 0, sizeof(double) * nS);
  }
  for (int t = 0; t < T; ++t) {
    const size_t bt = (size_t)b * T + t;
    if (mom && t % j->chunk == 0) { /* chunk entry */
      memcpy(S_in, S, sizeof(double) * nS);
      for (int i = 0; i < dk; ++i) Fc[i] = 1.0;
      kappa = 1;
    }
    if (j->reset && j->reset[bt]) { /* a new document: discard the carried state */
      memset(S, 0, sizeof(double) * nS);
      kappa = 0;
    }
    const float *kt = j->k + (bt * Hk + hk) * (size_t)dk;
    const float *qt = j->q + (bt * Hk + hk) * (size_t)dk;
    const float *vt = j->v + (bt * Hv + hv) * (size_t)dv;
    const float *lat = j->log_alpha + (bt * Hk + hk) * (size_t)G;
    const double beta = (double)(j->beta_per_key_head ? j->beta[bt * Hk + hk] : j->beta[bt * Hv + hv]);
    for (int i = 0; i < dk; ++i) {
      f[i] = exp((double)lat[i / group_width]);
      kv[i] = (double)kt[i];
      qv[i] = (double)qt[i];
      if (mom) Fc[i] *= f[i];
    }
    /* decay: S <- F_t S */
    for (int i = 0; i < dk; ++i) {
      double *row = S + (size_t)i * dv;
      for (int c = 0; c < dv; ++c) row[c] *= f[i];
    }
    /* prediction error u = v_t - S^T k_t (with the decayed S) */
    for (int c = 0; c < dv; ++c) uu[c] = (double)vt[c];
    for (int i = 0; i < dk; ++i) {
      const double *row = S + (size_t)i * dv;
      for (int c = 0; c < dv; ++c) uu[c] -= row[c] * kv[i];
    }
    /* rank-one write S <- S + beta k u^T */
    for (int i = 0; i < dk; ++i) {
      double *row = S + (size_t)i * dv;
      const double bk = beta * kv[i];
      for (int c = 0; c < dv; ++c) row[c] += bk * uu[c];
    }
    /* readout o_t = S_t^T q_t */
    double *ot = j->o + (bt * Hv + hv) * (size_t)dv;
    for (int c = 0; c < dv; ++c) ot[c] = 0.0;
    for (int i = 0; i < dk; ++i) {
      const double *row = S + (size_t)i * dv;
      for (int c = 0; c < dv; ++c) ot[c] += row[c] * qv[i];
    }
    if (mom && (t % j->chunk == j->chunk - 1 || t == T - 1)) { /* chunk end */
      for (int i = 0; i < dk; ++i) {
        const double fk = kappa ? Fc[i] : 0.0;
        for (int c = 0; c < dv; ++c) {
          const size_t e = (size_t)i * dv + c;
          const double carry = fk * S_in[e];
          Z[e] = j->momentum * (kappa ? Z[e] : 0.0) + (S[e] - carry);
          S[e] = carry + Z[e];
        }
      }
    }
  }
  if (j->hT) memcpy(j->hT + state_off, S, sizeof(double) * nS);
  if (j->zT) memcpy(j->zT + state_off, Z, sizeof(double) * nS);
  free(S_in);
  free(Z);
  free(Fc);
  free(S);
  free(f);
  free(kv);
  free(qv);
  free(uu);
}

static void *worker(void *arg) {
  job_t *j = (job_t *)arg;
  for (;;) {
    pthread_mutex_lock(&j->mu);
    const int idx = j->next++;
    pthread_mutex_unlock(&j->mu);
    if (idx >= j->n_units) break;
    run_unit(j, j->units ? j->units[idx] : idx);
  }
  return NULL;
}

int oracle_gdr_layer(int B, int T, int Hk, int Hv, int dk, int dv, int G, int beta_per_key_head,
                     const float *q, const float *k, const float *v, const float *beta,
                     const float *log_alpha, const unsigned char *reset, const double *h0,
                     const double *z0, int chunk, double momentum, double *o, double *hT,
                     double *zT, const int *units, int n_units, int nthreads) {
  if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || G <= 0) return -1;
  if (Hv % Hk != 0 || dk % G != 0 || chunk < 0) return -1;
  job_t j;
  j.B = B; j.T = T; j.Hk = Hk; j.Hv = Hv; j.dk = dk; j.dv = dv; j.G = G;
  j.beta_per_key_head = beta_per_key_head;
  j.q = q; j.k = k; j.v = v; j.beta = beta; j.log_alpha = log_alpha;
  j.reset = reset; j.z0 = z0; j.chunk = chunk; j.momentum = momentum; j.zT = zT;
  j.h0 = h0; j.o = o; j.hT = hT;
  j.units = units;
  j.n_units = units ? n_units : B * Hv;
  j.next = 0;
  if (units) {
    for (int i = 0; i < n_units; ++i)
      if (units[i] < 0 || units[i] >= B * Hv) return -1;
  }
  pthread_mutex_init(&j.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > j.n_units) nthreads = j.n_units > 0 ? j.n_units : 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &j);
  worker(&j);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&j.mu);
  return 0;
}

int oracle_gdr_recurrence(int B, int T, int Hk, int Hv, int dk, int dv, int G,
                          int beta_per_key_head, const float *q, const float *k,
                          const float *v, const float *beta, const float *log_alpha,
                          const double *h0, double *o, double *hT, const int *units,
                          int n_units, int nthreads) {
  return oracle_gdr_layer(B, T, Hk, Hv, dk, dv, G, beta_per_key_head, q, k, v, beta, log_alpha, NULL,
                          h0, NULL, 0, 0.0, o, hT, NULL, units, n_units, nthreads);
}
