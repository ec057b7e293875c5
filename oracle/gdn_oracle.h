/*
 * gdn_oracle.h -- plain fp64 CPU oracle for the gated delta rule (and the
 * causal conv1d that runs before it in a layer).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this library; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * Every input arrives already widened to double (the binding widens fp32 and
 * bf16 exactly).  Index tables arrive as int64.  All arrays are dense,
 * row-major, in the shapes given beside each argument.  Nothing is rounded
 * on output.
 *
 * Sources (cited by page title and section):
 *  - "Gated DeltaNet State Update" (tensortonic problem): the recurrence
 *    S_t = gamma_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T and the
 *    readout y_t = q_t^T S_t, statement and constraints.
 *  - "com.microsoft.GatedDeltaNet" (ONNX Runtime contrib op card): value head
 *    h reads query/key head h*Hq/Hv; cu_seqlens clamped to [0, T]; V-major
 *    (batch, Hv, Dv, Dk) fp32 states; an empty request copies its incoming
 *    state; the "qwen" gate -exp(a_log)*softplus(decay + dt_bias); scale.
 *  - "flashinfer.cake_gdp.cake_gated_delta_product_mtp": decode over a slot
 *    pool, decay once per token then num_householder delta sub-steps, fused
 *    gate with softplus threshold 20 and sigmoid beta, skip / write-slot /
 *    scatter / disable_state_update rules.
 *  - "gated_delta_conv1d_fwd": causal depthwise conv1d with a slot-indexed
 *    conv-state pool, ragged offsets, write_state.
 *  - "Circuit.LLM.Mixer" (Haskell source): gatedDeltaStep -- scale the state
 *    by alpha first, then the delta write.
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

/* update_rule of the ONNX card (Attributes): which terms survive. */
enum {
  GDNO_RULE_GATED_DELTA = 0, /* decay and delta retrieval */
  GDNO_RULE_GATED = 1,       /* decay only: S = gamma S + k v^T */
  GDNO_RULE_DELTA = 2,       /* retrieval only: S = S + k (beta (v - S^T k))^T */
  GDNO_RULE_LINEAR = 3       /* neither: S = S + k v^T */
};

#ifdef __cplusplus
extern "C" {
#endif

/* Fused gates, elementwise over n rows of hv heads.
 *   log_decay[i,h] = -exp(A_log[h]) * softplus20(a[i,h] + dt_bias[h])
 *   gamma[i,h]     = exp(log_decay[i,h])
 *   beta[i,h]      = 1 / (1 + exp(-b[i,h]))
 * softplus20(x) = x for x > 20, else log(1 + exp(x)).
 * a or b may be NULL (then the matching outputs are not written); any output
 * may be NULL. */
void gdno_gate(int64_t n, int32_t hv, const double* A_log, const double* dt_bias,
               const double* a, const double* b,
               double* log_decay, double* gamma, double* beta);

/* Sequential prefill over packed or ragged requests.
 *   q, k     [T, hq, dk]      v [T, hv, dv]
 *   decay    [T, hv]          log-space decay when decay_is_gamma == 0,
 *                             gamma itself when decay_is_gamma != 0
 *   beta     [T, hv]          effective update rate
 *   A_log, dt_bias [hv], a, b [T, hv]: the fused gate (as gdno_gate): a
 *                             != NULL gives the decay (the qwen gate, needs
 *                             A_log and dt_bias; decay is then not read), b
 *                             != NULL gives beta = sigmoid(b) (beta is then
 *                             not read)
 *   decay_per_key             != 0: decay is [T, hv, dk], one decay per key
 *                             dimension (the ONNX card's per-key spelling):
 *                             each step first scales key row i of the state
 *                             by its own factor; rules with a decay only, and
 *                             the decay given (a == NULL)
 *   update_rule               GDNO_RULE_*: which terms of the recurrence
 *                             survive (the ONNX card's update_rule).  Rules
 *                             without the decay read no decay (gamma = 1),
 *                             rules without beta read no beta (beta = 1);
 *                             linear and gated drop the delta retrieval
 *   qk_l2norm_eps             >= 0: every q and k head vector is replaced by
 *                             x / sqrt(sum(x^2) + qk_l2norm_eps) first; < 0: none
 *   cu       [n_seqs + 1]     or NULL: request r covers [r*seq_len, (r+1)*seq_len)
 *   init     [n_seqs, hv, dv, dk] V-major, or NULL (zeros)
 *   out      [T, hv, dv]      rows of tokens that no request covers are left as given
 *   final    [n_seqs, hv, dv, dk] V-major
 * Returns 0, or -1 on an argument error (hv not a multiple of hq, sizes <= 0). */
int gdno_prefill(int32_t n_seqs, int64_t total_tokens, int32_t seq_len,
                 int32_t hq, int32_t hv, int32_t dk, int32_t dv,
                 const double* q, const double* k, const double* v,
                 const double* decay, int32_t decay_is_gamma, const double* beta,
                 const int64_t* cu, const double* init, double scale,
                 double* out, double* final_state, int32_t nthreads,
                 double qk_l2norm_eps, const double* A_log, const double* dt_bias,
                 const double* a, const double* b, int32_t update_rule,
                 int32_t decay_per_key);

/* Slot-pool decode with n_hh Householder sub-steps per token.  With
 * qk_l2norm_eps >= 0 every q and k head vector is first replaced by
 * x / sqrt(sum(x^2) + qk_l2norm_eps) (use_qk_l2norm); < 0: none.
 *   q [B, T, hq, dk]   k [B, T, n_hh, hq, dk]   v [B, T, n_hh, hv, dv]
 *   A_log, dt_bias [hv]   a [B, T, hv]   b [B, T, n_hh, hv]
 *   pool [P, hv, dv, dk]  V-major, updated in place (snapshot semantics: every
 *                         row reads the pool as it was on entry)
 *   read [B]; write [B] or NULL (= read); scatter [B, T] or NULL
 *   out  [B, T, hv, dv]  rows of skipped batch rows are left as given
 *   decay_per_key [B, T, hv, dk] log-decay per key dimension, or NULL: when
 *                         given it replaces the fused gate's decay (each
 *                         token scales key row i of the state by its factor)
 * Returns 0, or -1 on an argument error (includes scatter with disable). */
int gdno_decode(int32_t B, int32_t T, int32_t n_hh, int32_t hq, int32_t hv,
                int32_t dk, int32_t dv,
                const double* q, const double* k, const double* v,
                const double* A_log, const double* dt_bias,
                const double* a, const double* b,
                double* pool, int32_t P,
                const int64_t* read, const int64_t* write, const int64_t* scatter,
                int32_t disable_state_update, double scale,
                double* out, int32_t nthreads, double qk_l2norm_eps,
                const double* decay_per_key);

/* Causal depthwise conv1d over a ragged batch with a slot-indexed conv-state
 * pool ("gated_delta_conv1d_fwd").
 *   x [T, conv_dim]   w [conv_dim, K]   state [max_slots, conv_dim, K-1]
 *   (updated in place when write_state != 0)   slot [n_seqs]
 *   off [n_seqs + 1]   out [T, conv_dim] (rows no sequence covers are left)
 * Sequence b's window is state[slot[b], c, :] (oldest first) followed by its
 * inputs; out = sum_j w[c, j] * window[t + j]; the slot then holds the last
 * K-1 window entries.  A slot outside [0, max_slots) reads zeros and is not
 * written.  Returns 0, or -1 on an argument error. */
int gdno_conv1d(int64_t T, int32_t conv_dim, int32_t K, int32_t n_seqs,
                const double* x, const double* w, double* state, int64_t max_slots,
                const int64_t* slot, const int64_t* off, int32_t write_state, double* out);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ORACLE_H */
