/*
 * Double-precision reference ("oracle") for the gated delta-rule scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the library's compute path may link,
 * load or call this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the GPU library.
 *
 * What it computes (one token at a time, in double precision):
 *
 *   The operator is the gated delta-net linear attention with a matrix-valued
 *   recurrent state per head ("[Research] Explore linear attention for the
 *   streaming video models", section "We already ship a hybrid linear-attention
 *   model"), updated one token at a time as standard delta-rule linear attention
 *   does ("Video DeltaNet", "Methodology in Plain English").  With the state
 *   S in R^{dv x dk}, per (batch, head) and token t:
 *
 *     q^_t = q_t / max(|q_t|_2, eps),  k^_t = k_t / max(|k_t|_2, eps),  eps = 1e-6
 *     a_t  = exp(log_alpha_t)
 *     S_t  = a_t S_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T
 *     o_t  = S_t q^_t
 *
 *   evaluated in the algebraically identical delta form
 *     S <- a_t S;  u <- beta_t (v_t - S k^_t);  S <- S + u k^_t^T;  o_t <- S q^_t.
 *
 *   The reverse scan is the same recurrence run from the last token to the
 *   first with its own gates and initial state; the bidirectional output is the
 *   sum of the forward and reverse outputs, each direction keeping its own
 *   final state (the two scans whose readouts are added, "Video DeltaNet",
 *   "Methodology in Plain English").
 *
 *   Exclusive readout (bit 0 of `exclusive` for the forward direction, bit 1
 *   for the reverse one): that direction reads its memory after the decay and
 *   before the token's own write, o_t = a_t S_{t-1} q^_t (reverse:
 *   a_t S_{t+1} q^_t).  With both bits set the two scans of a bidirectional
 *   call cover the disjoint regions s < t and s > t, and with only the reverse
 *   bit the regions s <= t and s > t, which together hold every token once
 *   (the disjoint-region combine of "Video DeltaNet", "Methodology in Plain
 *   English", at token granularity; the reading of where the decay a_t stands
 *   is ours: the excluded part is exactly the token's own write).
 *
 *   With erase == 0 the "- beta k k^T" erase term is dropped (S <- a S +
 *   beta v k^T): the plain gated linear attention that results from removing
 *   the delta-rule update (SANA-Video 2.0 review, "Future work").  It pins the
 *   oracle against brute-force linear attention and is the reference of the
 *   library's erase-free variant.
 *
 * Layouts (all contiguous, row-major):
 *   q, k      [B, T, H, dk]   float (exact values of the inputs; bf16 widened)
 *   v         [B, T, H, dv]   float
 *   log_alpha [dirs, B, T, H] float,  beta [dirs, B, T, H] float
 *   state_in  [dirs, B, H, dv, dk] float or NULL (zero initial state)
 *   state_out [dirs, B, H, dv, dk] double or NULL
 *   out       [B, T, H, dv]   double
 * dirs is 2 for the bidirectional scan, else 1.
 *
 * Parallelism: independent (batch, head) chains run on separate threads; the
 * arithmetic inside a chain is the plain sequential loop above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EPS 1e-6

typedef struct {
  int64_t B, T, H, dk, dv;
  const float *q, *k, *v, *log_alpha, *beta, *state_in;
  double *state_out, *out_fwd, *out_rev;
  int direction; /* 0 forward, 1 reverse, 2 both */
  int erase;
  int exclusive; /* bit 0: forward direction reads before its write, bit 1: reverse */
  int64_t next_chain; /* work counter, protected by lock */
  pthread_mutex_t lock;
} job_t;

static void normalise(const float* x, int64_t d, double* y) {
  double ss = 0.0;
  for (int64_t j = 0; j < d; ++j) ss += (double)x[j] * (double)x[j];
  double n = sqrt(ss);
  if (n < ORACLE_EPS) n = ORACLE_EPS;
  for (int64_t j = 0; j < d; ++j) y[j] = (double)x[j] / n;
}

/* Run one direction of one (b, h) chain; `dir_slot` selects the gate/state
   slice (0 for the first listed direction), `reverse` the token order. */
static void run_chain(job_t* J, int64_t b, int64_t h, int dir_slot, int reverse, double* out,
                      double* S, double* qh, double* kh, double* u) {
  const int64_t B = J->B, T = J->T, H = J->H, dk = J->dk, dv = J->dv;
  const int64_t sidx = ((int64_t)dir_slot * B + b) * H + h;
  if (J->state_in) {
    const float* s0 = J->state_in + sidx * dv * dk;
    for (int64_t i = 0; i < dv * dk; ++i) S[i] = (double)s0[i];
  } else {
    memset(S, 0, sizeof(double) * dv * dk);
  }
  for (int64_t step = 0; step < T; ++step) {
    const int64_t t = reverse ? (T - 1 - step) : step;
    const int64_t row = (b * T + t) * H + h;
    const int64_t g = ((int64_t)dir_slot * B + b) * T * H + t * H + h;
    normalise(J->q + row * dk, dk, qh);
    normalise(J->k + row * dk, dk, kh);
    const double a = exp((double)J->log_alpha[g]);
    const double beta = (double)J->beta[g];
    const float* vt = J->v + row * dv;
    /* S <- a S */
    for (int64_t i = 0; i < dv * dk; ++i) S[i] *= a;
    double* o = out + row * dv;
    const int excl = (J->exclusive >> (reverse ? 1 : 0)) & 1;
    if (excl) {
      /* o = (a S) q^, before the token's own write */
      for (int64_t i = 0; i < dv; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < dk; ++j) s += S[i * dk + j] * qh[j];
        o[i] = s;
      }
    }
    if (J->erase) {
      /* u = beta (v - S k^) */
      for (int64_t i = 0; i < dv; ++i) {
        double sk = 0.0;
        for (int64_t j = 0; j < dk; ++j) sk += S[i * dk + j] * kh[j];
        u[i] = beta * ((double)vt[i] - sk);
      }
    } else {
      for (int64_t i = 0; i < dv; ++i) u[i] = beta * (double)vt[i];
    }
    /* S <- S + u k^T */
    for (int64_t i = 0; i < dv; ++i)
      for (int64_t j = 0; j < dk; ++j) S[i * dk + j] += u[i] * kh[j];
    /* o = S q^ */
    if (!excl) {
      for (int64_t i = 0; i < dv; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < dk; ++j) s += S[i * dk + j] * qh[j];
        o[i] = s;
      }
    }
  }
  if (J->state_out) {
    double* so = J->state_out + sidx * dv * dk;
    memcpy(so, S, sizeof(double) * dv * dk);
  }
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int64_t dk = J->dk, dv = J->dv;
  double* S = (double*)malloc(sizeof(double) * (size_t)(dv * dk + 2 * dk + dv));
  if (!S) return (void*)1;
  double* qh = S + dv * dk;
  double* kh = qh + dk;
  double* u = kh + dk;
  const int ndir = J->direction == 2 ? 2 : 1;
  const int64_t nchains = J->B * J->H * ndir;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    int64_t c = J->next_chain++;
    pthread_mutex_unlock(&J->lock);
    if (c >= nchains) break;
    const int d = (int)(c % ndir);
    const int64_t bh = c / ndir;
    const int64_t b = bh / J->H, h = bh % J->H;
    const int reverse = (J->direction == 1) || (J->direction == 2 && d == 1);
    double* out = (J->direction == 2 && d == 1) ? J->out_rev : J->out_fwd;
    run_chain(J, b, h, d, reverse, out, S, qh, kh, u);
  }
  free(S);
  return NULL;
}

/* Returns 0 on success, 1 on bad arguments, 2 on allocation failure. */
int gdn_oracle_forward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, const float* q,
                       const float* k, const float* v, const float* log_alpha, const float* beta,
                       const float* state_in, double* state_out, double* out, int direction,
                       int erase, int exclusive, int nthreads) {
  if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || direction < 0 || direction > 2) return 1;
  if (exclusive < 0 || exclusive > 3) return 1;
  if (!out || (T > 0 && (!q || !k || !v || !log_alpha || !beta))) return 1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta;
  J.state_in = state_in; J.state_out = state_out;
  J.direction = direction; J.erase = erase; J.exclusive = exclusive;
  J.out_fwd = out;
  double* rev = NULL;
  const size_t n_out = (size_t)(B * T * H * dv);
  if (direction == 2) {
    rev = (double*)malloc(sizeof(double) * (n_out ? n_out : 1));
    if (!rev) return 2;
    J.out_rev = rev;
  } else {
    J.out_rev = out;
  }
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started = 0;
  for (int i = 1; i < nthreads; ++i)
    if (pthread_create(&th[started], NULL, worker, &J) == 0) ++started;
  int fail = worker(&J) != NULL;
  for (int i = 0; i < started; ++i) {
    void* r = NULL;
    pthread_join(th[i], &r);
    fail |= r != NULL;
  }
  pthread_mutex_destroy(&J.lock);
  if (direction == 2) {
    for (size_t i = 0; i < n_out; ++i) out[i] += rev[i];
    free(rev);
  }
  return fail ? 2 : 0;
}
