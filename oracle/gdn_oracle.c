/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  It shares no code
 * with the HIP library.
 *
 * The state is kept K-major, S[i][j] with i over the Dk key dimensions and j
 * over the Dv value dimensions, exactly as in the statement of "Gated DeltaNet
 * State Update".  V-major arrays at the interface (the ONNX card's
 * (batch, Hv, Dv, Dk) layout and the decode pool) are transposed on the way in
 * and out.  Work is split over independent (request, value head) or
 * (batch row, value head) units on plain pthreads; the arithmetic inside a
 * unit is the sequential recurrence, one token at a time, in the order the
 * pages state it.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- gates -- */

/* Softplus with the threshold 20 stated on the FlashInfer decode page
 * ("softplus threshold 20"): the identity above the threshold. */
static double softplus20(double x) { return x > 20.0 ? x : log1p(exp(x)); }

/* Logistic sigmoid, the beta activation of the FlashInfer decode page and of
 * the ONNX card's beta_activation = sigmoid. */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* The qwen gate of the ONNX card / the fused gate of the FlashInfer page:
 * log-decay g = -exp(A_log) * softplus(a + dt_bias); gamma = exp(g). */
static double gate_log_decay(double A_log, double dt_bias, double a) {
  return -exp(A_log) * softplus20(a + dt_bias);
}

void gdno_gate(int64_t n, int32_t hv, const double* A_log, const double* dt_bias,
               const double* a, const double* b,
               double* log_decay, double* gamma, double* beta) {
  for (int64_t i = 0; i < n; ++i) {
    for (int32_t h = 0; h < hv; ++h) {
      const int64_t e = i * hv + h;
      if (a) {
        const double g = gate_log_decay(A_log[h], dt_bias[h], a[e]);
        if (log_decay) log_decay[e] = g;
        if (gamma) gamma[e] = exp(g);
      }
      if (b && beta) beta[e] = sigmoid(b[e]);
    }
  }
}

/* ------------------------------------------------------- recurrence step -- */

/* One step of "Gated DeltaNet State Update":
 *   S <- gamma * (I - beta * k k^T) S + beta * k v^T
 * written out with the rank-one form of (I - beta k k^T) S = S - beta k (k^T S).
 * S is dk x dv (K-major); tmp holds dv doubles. */
static void gd_step(int dk, int dv, double* S, const double* k, const double* v,
                    double gamma, double beta, double* tmp) {
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += k[i] * S[(size_t)i * dv + j];
    tmp[j] = acc; /* (k^T S)_j */
  }
  for (int i = 0; i < dk; ++i) {
    for (int j = 0; j < dv; ++j) {
      double* s = &S[(size_t)i * dv + j];
      *s = gamma * (*s - beta * k[i] * tmp[j]) + beta * k[i] * v[j];
    }
  }
}

/* One step of the ONNX card's recurrence with its update_rule ("Description"
 * and the update_rule attribute):
 *   S_t = exp(g_t) S_{t-1} + k_t (beta_t (v_t - exp(g_t) S_{t-1}^T k_t))^T
 * taken literally: decay the state, retrieve from the decayed state when the
 * rule keeps the delta retrieval (retrieve != 0), then add k u^T.  Rules
 * without the decay pass gamma = 1, rules without beta pass beta = 1. */
static void rule_step(int dk, int dv, double* S, const double* k, const double* v,
                      double gamma, double beta, int retrieve, double* tmp) {
  for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] *= gamma;
  for (int j = 0; j < dv; ++j) {
    double r = 0.0;
    if (retrieve)
      for (int i = 0; i < dk; ++i) r += S[(size_t)i * dv + j] * k[i];
    tmp[j] = beta * (v[j] - r); /* u_j */
  }
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += k[i] * tmp[j];
}

/* Decay of each key row of S by its own factor: the ONNX card's per-key-
 * dimension decay (Inputs, decay (..., num_heads_v, head_size_qk)) read in
 * its recurrence, where exp(g_t) multiplies S_{t-1} elementwise over the
 * key dimension: S <- diag(alpha) S. */
static void decay_rows(int dk, int dv, double* S, const double* alpha) {
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha[i];
}

/* Readout y = scale * q^T S (a dv-vector), taken after the update. */
static void readout(int dk, int dv, const double* S, const double* q, double scale,
                    double* y) {
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];
    y[j] = scale * acc;
  }
}

/* In-kernel L2 normalisation of a query or key head vector, as the FlashInfer
 * decode page states it for use_qk_l2norm: x * rsqrt(sum(x^2) + eps).  The
 * ONNX card's qk_l2_norm names only the epsilon (1e-12); the same form is
 * read there. */
static void l2_normalize(int n, const double* x, double eps, double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  const double r = 1.0 / sqrt(ss + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * r;
}

/* V-major [dv][dk] <-> K-major [dk][dv]. */
static void vmajor_to_kmajor(int dk, int dv, const double* vm, double* km) {
  for (int j = 0; j < dv; ++j)
    for (int i = 0; i < dk; ++i) km[(size_t)i * dv + j] = vm[(size_t)j * dk + i];
}
static void kmajor_to_vmajor(int dk, int dv, const double* km, double* vm) {
  for (int j = 0; j < dv; ++j)
    for (int i = 0; i < dk; ++i) vm[(size_t)j * dk + i] = km[(size_t)i * dv + j];
}

/* ---------------------------------------------------------- thread pool -- */

typedef void (*unit_fn)(void* ctx, int64_t unit);

typedef struct {
  unit_fn fn;
  void* ctx;
  int64_t n_units;
  int64_t next; /* shared work counter */
} pool_job;

static void* pool_worker(void* arg) {
  pool_job* job = (pool_job*)arg;
  for (;;) {
    const int64_t u = __atomic_fetch_add(&job->next, 1, __ATOMIC_RELAXED);
    if (u >= job->n_units) break;
    job->fn(job->ctx, u);
  }
  return NULL;
}

static void run_units(unit_fn fn, void* ctx, int64_t n_units, int nthreads) {
  pool_job job = {fn, ctx, n_units, 0};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads == 1 || n_units <= 1) {
    pool_worker(&job);
    return;
  }
  pthread_t tid[256];
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    if (pthread_create(&tid[t], NULL, pool_worker, &job) != 0) break;
    ++started;
  }
  if (started == 0) pool_worker(&job);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
}

/* -------------------------------------------------------------- prefill -- */

typedef struct {
  int32_t n_seqs, seq_len, hq, hv, dk, dv, decay_is_gamma;
  int64_t T;
  const double *q, *k, *v, *decay, *beta, *init;
  const int64_t* cu;
  double scale;
  double *out, *final_state;
  double qk_eps;                      /* < 0: no in-kernel L2 norm */
  const double *A_log, *dt_bias, *a, *b;  /* fused decay when a != NULL, fused beta when b != NULL */
  int32_t rule;                       /* GDNO_RULE_* */
  int32_t per_key;                    /* decay is [T, hv, dk] */
} prefill_ctx;

static int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

/* One (request r, value head h) unit.  Request bounds follow the ONNX card:
 * offsets clamped to [0, T]; a decreasing pair yields an empty request.
 * Value head h reads query/key head h * hq / hv (integer division). */
static void prefill_unit(void* vctx, int64_t unit) {
  const prefill_ctx* c = (const prefill_ctx*)vctx;
  const int32_t r = (int32_t)(unit / c->hv);
  const int32_t h = (int32_t)(unit % c->hv);
  const int32_t qh = (int32_t)(((int64_t)h * c->hq) / c->hv);
  const int dk = c->dk, dv = c->dv;

  int64_t start, end;
  if (c->cu) {
    start = clamp64(c->cu[r], 0, c->T);
    end = clamp64(c->cu[r + 1], 0, c->T);
  } else {
    start = (int64_t)r * c->seq_len;
    end = start + c->seq_len;
  }
  if (end < start) end = start;

  double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
  double* tmp = (double*)malloc(sizeof(double) * (size_t)dv);
  double* qn = (double*)malloc(sizeof(double) * (size_t)dk);
  double* kn = (double*)malloc(sizeof(double) * (size_t)dk);
  double* alpha = (double*)malloc(sizeof(double) * (size_t)dk);
  const size_t st_off = ((size_t)r * c->hv + h) * (size_t)dv * dk;
  if (c->init) vmajor_to_kmajor(dk, dv, c->init + st_off, S);

  for (int64_t t = start; t < end; ++t) {
    const double* q = c->q + ((size_t)t * c->hq + qh) * dk;
    const double* k = c->k + ((size_t)t * c->hq + qh) * dk;
    const double* v = c->v + ((size_t)t * c->hv + h) * dv;
    if (c->qk_eps >= 0.0) {
      l2_normalize(dk, q, c->qk_eps, qn);
      l2_normalize(dk, k, c->qk_eps, kn);
      q = qn;
      k = kn;
    }
    const size_t e = (size_t)t * c->hv + h;
    const int has_decay = c->rule == GDNO_RULE_GATED_DELTA || c->rule == GDNO_RULE_GATED;
    const int has_beta = c->rule == GDNO_RULE_GATED_DELTA || c->rule == GDNO_RULE_DELTA;
    double gamma = 1.0, beta = 1.0;
    if (has_beta) /* fused: a sigmoid of b */
      beta = c->b ? sigmoid(c->b[e]) : c->beta[e];
    if (c->per_key) {
      /* per-key decay: decay the key rows, then the step without decay */
      const double* d = c->decay + e * (size_t)dk;
      for (int i = 0; i < dk; ++i) alpha[i] = c->decay_is_gamma ? d[i] : exp(d[i]);
      decay_rows(dk, dv, S, alpha);
      rule_step(dk, dv, S, k, v, 1.0, beta, c->rule == GDNO_RULE_GATED_DELTA, tmp);
      readout(dk, dv, S, q, c->scale, c->out + ((size_t)t * c->hv + h) * dv);
      continue;
    }
    if (has_decay) /* fused: the qwen gate on a */
      gamma = c->a ? exp(gate_log_decay(c->A_log[h], c->dt_bias[h], c->a[e]))
                   : (c->decay_is_gamma ? c->decay[e] : exp(c->decay[e]));
    if (c->rule == GDNO_RULE_GATED_DELTA)
      gd_step(dk, dv, S, k, v, gamma, beta, tmp);
    else
      rule_step(dk, dv, S, k, v, gamma, beta, c->rule == GDNO_RULE_DELTA, tmp);
    readout(dk, dv, S, q, c->scale, c->out + ((size_t)t * c->hv + h) * dv);
  }
  free(alpha);
  free(kn);
  free(qn);
  /* final state after the request's last token; an empty request copies its
   * incoming state (zeros when there is none) */
  kmajor_to_vmajor(dk, dv, S, c->final_state + st_off);
  free(tmp);
  free(S);
}

int gdno_prefill(int32_t n_seqs, int64_t total_tokens, int32_t seq_len,
                 int32_t hq, int32_t hv, int32_t dk, int32_t dv,
                 const double* q, const double* k, const double* v,
                 const double* decay, int32_t decay_is_gamma, const double* beta,
                 const int64_t* cu, const double* init, double scale,
                 double* out, double* final_state, int32_t nthreads,
                 double qk_l2norm_eps, const double* A_log, const double* dt_bias,
                 const double* a, const double* b, int32_t update_rule, int32_t decay_per_key) {
  if (n_seqs < 0 || total_tokens < 0 || hq <= 0 || hv <= 0 || dk <= 0 || dv <= 0)
    return -1;
  if (hv % hq != 0) return -1;
  if (!cu && (int64_t)n_seqs * seq_len != total_tokens) return -1;
  if (update_rule < GDNO_RULE_GATED_DELTA || update_rule > GDNO_RULE_LINEAR) return -1;
  const int has_decay = update_rule == GDNO_RULE_GATED_DELTA || update_rule == GDNO_RULE_GATED;
  const int has_beta = update_rule == GDNO_RULE_GATED_DELTA || update_rule == GDNO_RULE_DELTA;
  if (a && (!A_log || !dt_bias)) return -1;
  if (decay_per_key && (a || !has_decay)) return -1; /* per-key decay: given, rules with a decay */
  if (total_tokens > 0 && has_decay && !a && !decay) return -1;
  if (total_tokens > 0 && has_beta && !b && !beta) return -1;
  prefill_ctx c = {n_seqs, seq_len, hq, hv, dk, dv, decay_is_gamma, total_tokens,
                   q, k, v, decay, beta, init, cu, scale, out, final_state,
                   qk_l2norm_eps, A_log, dt_bias, a, b, update_rule, decay_per_key};
  run_units(prefill_unit, &c, (int64_t)n_seqs * hv, nthreads);
  return 0;
}

/* --------------------------------------------------------------- decode -- */

typedef struct {
  int32_t B, T, n_hh, hq, hv, dk, dv, P, disable;
  const double *q, *k, *v, *A_log, *dt_bias, *a, *b;
  const double* pool0; /* snapshot of the pool on entry */
  double* pool;
  const int64_t *read, *write, *scatter;
  double scale;
  double* out;
  double qk_eps; /* < 0: no in-kernel L2 norm */
  const double* pk_decay; /* [B, T, hv, dk] log-decay per key, or NULL (fused gate) */
} decode_ctx;

static int slot_ok(int64_t s, int32_t P) { return s >= 0 && s < P; }

/* One (batch row b, value head h) unit of the FlashInfer decode contract:
 * read the state from slot read[b]; per token decay once by the fused gate,
 * then n_hh delta sub-steps with their own k, v and sigmoid beta; read out
 * after the sub-steps; scatter after each token when a scatter table is
 * given, else write back once after the last token. */
static void decode_unit(void* vctx, int64_t unit) {
  const decode_ctx* c = (const decode_ctx*)vctx;
  const int32_t bi = (int32_t)(unit / c->hv);
  const int32_t h = (int32_t)(unit % c->hv);
  const int32_t qh = (int32_t)(((int64_t)h * c->hq) / c->hv);
  const int dk = c->dk, dv = c->dv;
  const int64_t rd = c->read[bi];
  if (!slot_ok(rd, c->P)) return; /* skipped row: nothing read or written */
  const int64_t wr = c->write ? c->write[bi] : rd;
  const size_t slot_elems = (size_t)c->hv * dv * dk;
  const size_t head_off = (size_t)h * dv * dk;

  double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)dv);
  double* qn = (double*)malloc(sizeof(double) * (size_t)dk);
  double* kn = (double*)malloc(sizeof(double) * (size_t)dk);
  double* alpha = (double*)malloc(sizeof(double) * (size_t)dk);
  vmajor_to_kmajor(dk, dv, c->pool0 + (size_t)rd * slot_elems + head_off, S);

  for (int32_t t = 0; t < c->T; ++t) {
    const size_t bt = (size_t)bi * c->T + t;
    /* decay once per token (gatedDeltaStep: scale the state first) */
    if (c->pk_decay) {
      const double* d = c->pk_decay + (bt * c->hv + h) * (size_t)dk;
      for (int i = 0; i < dk; ++i) alpha[i] = exp(d[i]);
      decay_rows(dk, dv, S, alpha);
    } else {
      const double g = gate_log_decay(c->A_log[h], c->dt_bias[h], c->a[bt * c->hv + h]);
      const double gamma = exp(g);
      for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] *= gamma;
    }
    for (int32_t j = 0; j < c->n_hh; ++j) {
      const size_t btj = bt * c->n_hh + j;
      const double* k = c->k + (btj * c->hq + qh) * dk;
      if (c->qk_eps >= 0.0) {
        l2_normalize(dk, k, c->qk_eps, kn);
        k = kn;
      }
      const double* v = c->v + (btj * c->hv + h) * dv;
      const double beta = sigmoid(c->b[btj * c->hv + h]);
      gd_step(dk, dv, S, k, v, 1.0, beta, tmp); /* delta sub-step, no decay */
    }
    const double* q = c->q + (bt * c->hq + qh) * dk;
    if (c->qk_eps >= 0.0) {
      l2_normalize(dk, q, c->qk_eps, qn);
      q = qn;
    }
    readout(dk, dv, S, q, c->scale, c->out + (bt * c->hv + h) * dv);
    if (c->scatter) {
      const int64_t s = c->scatter[bt];
      if (slot_ok(s, c->P)) kmajor_to_vmajor(dk, dv, S, c->pool + (size_t)s * slot_elems + head_off);
    }
  }
  if (!c->scatter && !c->disable && slot_ok(wr, c->P))
    kmajor_to_vmajor(dk, dv, S, c->pool + (size_t)wr * slot_elems + head_off);
  free(alpha);
  free(kn);
  free(qn);
  free(tmp);
  free(S);
}

int gdno_decode(int32_t B, int32_t T, int32_t n_hh, int32_t hq, int32_t hv,
                int32_t dk, int32_t dv,
                const double* q, const double* k, const double* v,
                const double* A_log, const double* dt_bias,
                const double* a, const double* b,
                double* pool, int32_t P,
                const int64_t* read, const int64_t* write, const int64_t* scatter,
                int32_t disable_state_update, double scale,
                double* out, int32_t nthreads, double qk_l2norm_eps,
                const double* decay_per_key) {
  if (B < 0 || T <= 0 || n_hh <= 0 || hq <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || P < 0)
    return -1;
  if (hv % hq != 0) return -1;
  if (scatter && disable_state_update) return -1;
  const size_t pool_elems = (size_t)P * hv * dv * dk;
  double* pool0 = (double*)malloc(sizeof(double) * (pool_elems ? pool_elems : 1));
  if (!pool0) return -1;
  memcpy(pool0, pool, sizeof(double) * pool_elems);
  decode_ctx c = {B, T, n_hh, hq, hv, dk, dv, P, disable_state_update,
                  q, k, v, A_log, dt_bias, a, b, pool0, pool,
                  read, write, scatter, scale, out, qk_l2norm_eps, decay_per_key};
  run_units(decode_unit, &c, (int64_t)B * hv, nthreads);
  free(pool0);
  return 0;
}

/* ---------------------------------------------------------------- conv1d -- */

/* Causal depthwise conv1d over a ragged batch with a slot-indexed conv-state
 * pool ("gated_delta_conv1d_fwd", parameters and example).  For sequence b
 * (rows [off[b], off[b+1]) of x) and channel c, the window is the slot's
 * K-1 saved inputs (oldest first) followed by the sequence's inputs:
 *   win = state[slot_b, c, 0 .. K-2] ++ x[off[b] .., c]
 *   out[off[b] + t, c] = sum_{j < K} w[c, j] * win[t + j]
 * so w[c, K-1] multiplies the current input.  With write_state the slot then
 * holds the last K-1 entries of win.  A slot outside [0, max_slots) reads
 * zeros and is not written (the page leaves it undefined).  Offsets are
 * clamped to [0, T]; a decreasing pair is an empty sequence. */
int gdno_conv1d(int64_t T, int32_t conv_dim, int32_t K, int32_t n_seqs,
                const double* x, const double* w, double* state, int64_t max_slots,
                const int64_t* slot, const int64_t* off, int32_t write_state, double* out) {
  if (T < 0 || conv_dim <= 0 || K < 1 || n_seqs < 0 || max_slots < 0) return -1;
  const int H = K - 1;
  double* win = (double*)malloc(sizeof(double) * (size_t)(H + (T > 0 ? T : 1)));
  if (!win) return -1;
  for (int32_t b = 0; b < n_seqs; ++b) {
    int64_t s0 = clamp64(off[b], 0, T), s1 = clamp64(off[b + 1], 0, T);
    if (s1 < s0) s1 = s0;
    const int64_t len = s1 - s0;
    const int ok = slot[b] >= 0 && slot[b] < max_slots;
    for (int32_t c = 0; c < conv_dim; ++c) {
      double* st = ok ? state + ((size_t)slot[b] * conv_dim + c) * (size_t)H : NULL;
      for (int i = 0; i < H; ++i) win[i] = st ? st[i] : 0.0;
      for (int64_t t = 0; t < len; ++t) win[H + t] = x[(size_t)(s0 + t) * conv_dim + c];
      for (int64_t t = 0; t < len; ++t) {
        double acc = 0.0;
        for (int j = 0; j < K; ++j) acc += w[(size_t)c * K + j] * win[t + j];
        out[(size_t)(s0 + t) * conv_dim + c] = acc;
      }
      if (write_state && st)
        for (int i = 0; i < H; ++i) st[i] = win[len + i];
    }
  }
  free(win);
  return 0;
}
