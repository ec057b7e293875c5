/*
 * libgdn.h -- C ABI of the MI355X (gfx950) gated delta rule library.
 *
 * The method (statement of "Gated DeltaNet State Update", first display):
 *     S_t = gamma_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     y_t = scale * q_t^T S_t            (read out after the update)
 * taken independently per value head; value head h reads query/key head
 * h * hq / hv ("com.microsoft.GatedDeltaNet", Description).
 *
 * Conventions shared by every call
 *  - All data pointers are DEVICE pointers (hipMalloc / torch CUDA memory) and
 *    are owned by the caller.  The library never allocates, frees or keeps a
 *    pointer after a call returns.  Inputs are never written.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously; calls read no device memory on the host and
 *    never synchronise, so every call is hipGraph-capturable.
 *  - Recurrent states are fp32 and V-major: one head's state is a [dv][dk]
 *    array, row j holding value index j across all dk keys (the ONNX card's
 *    (batch, Hv, Dv, Dk) state; the FlashInfer pool's "K-last" layout).
 *  - Argument errors visible on the host (NULL required pointer, bad sizes,
 *    unsupported head sizes, misalignment, forbidden combinations) return a
 *    status other than GDN_OK before anything is enqueued; gdn_last_error()
 *    then returns a description (thread-local, valid until the next call on
 *    that thread).  Data-dependent conditions are never errors: out-of-range
 *    cu_seqlens become empty requests, out-of-range or negative slots mean
 *    "skip" (see each call).
 *  - Supported head sizes: dk and dv in {16, 32, 64, 128}.
 *  - Calls that overlap on one device race only where they write the same
 *    memory; two rows of one decode call that name the same pool slot (for
 *    reading by one and writing by another) are undefined behaviour.
 */
#ifndef LIBGDN_H
#define LIBGDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL                          */
  GDN_ERR_SHAPE = 2,       /* a size is <= 0, inconsistent, or hv % hq != 0        */
  GDN_ERR_DTYPE = 3,       /* unknown dtype or decay kind                          */
  GDN_ERR_LAYOUT = 4,      /* misaligned pointer / stride, or a partial overlap    */
  GDN_ERR_UNSUPPORTED = 5, /* valid request the library does not implement           */
  GDN_ERR_HIP = 6          /* a HIP launch failed; gdn_last_error() has the text   */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* update_rule of "com.microsoft.GatedDeltaNet" (Attributes): which terms of
 *   S_t = exp(g_t) S_{t-1} + k_t (beta_t (v_t - exp(g_t) S_{t-1}^T k_t))^T
 * survive.  Rules without the decay use g = 0, rules without beta use 1 in
 * the write, and linear / gated drop the retrieval S^T k. */
typedef enum {
  GDN_RULE_GATED_DELTA = 0, /* decay and delta retrieval (the default)         */
  GDN_RULE_GATED = 1,       /* decay only:     S = exp(g) S + k v^T            */
  GDN_RULE_DELTA = 2,       /* retrieval only: S = S + k (beta (v - S^T k))^T  */
  GDN_RULE_LINEAR = 3       /* neither:        S = S + k v^T                   */
} gdn_update_rule;

/* Meaning of the prefill decay input. */
typedef enum {
  GDN_DECAY_LOG = 0,   /* log-space decay g, gamma = exp(g); -inf means gamma = 0 */
  GDN_DECAY_GAMMA = 1  /* gamma itself, in [0, 1]                                 */
} gdn_decay_kind;

/* Text describing the last non-OK status returned on the calling thread. */
const char* gdn_last_error(void);

/* Library version as "major.minor.patch". */
const char* gdn_version(void);

/* gdn_wait_timeouts -- health check of the in-kernel waits.
 *
 * The bf16 pair prefill kernel (and the scan's passes, which run it) hands
 * each chunk from its preparing waves to its state waves through counters
 * in workgroup memory; every wait on such a counter is bounded (2^22 polls,
 * far beyond any working schedule).  A wait that runs out adds 1 to a
 * per-device word and the kernel finishes normally, with results that are
 * then not to be trusted.  This call stores the current device's word in
 * *count (0 in every correct run) and sets it back to 0 when clear != 0.
 * Synchronous: it waits for all work on the current device.  Returns
 * GDN_ERR_NULL for a NULL count, GDN_ERR_HIP when the copy fails.
 */
gdn_status gdn_wait_timeouts(uint32_t* count, int32_t clear);

/* ----------------------------------------------------------------------------
 * gdn_gate -- fused gates, elementwise over n_tokens rows of hv heads.
 *
 * Follows the "qwen" gate_activation of "com.microsoft.GatedDeltaNet"
 * (Attributes) and the fused gate of "flashinfer.cake_gdp.
 * cake_gated_delta_product_mtp" (description; softplus threshold 20):
 *     log_decay[i,h] = -exp(A_log[h]) * softplus(a[i,h] + dt_bias[h])
 *     gamma[i,h]     = exp(log_decay[i,h])
 *     beta[i,h]      = sigmoid(b[i,h])
 * with softplus(x) = x for x > 20, log1p(exp(x)) otherwise.  Arithmetic fp32.
 *
 *   A_log, dt_bias   [hv] fp32                     (required when a != NULL)
 *   a, b             [n_tokens, hv] dense, ab_dtype; either may be NULL
 *   log_decay_out, gamma_out   [n_tokens, hv] fp32, nullable; need a
 *   beta_out                   [n_tokens, hv] fp32, nullable; needs b
 * n_tokens == 0 is a no-op.  An output requested without its input is
 * GDN_ERR_NULL.
 * ------------------------------------------------------------------------- */
gdn_status gdn_gate(const float* A_log, const float* dt_bias,
                    const void* a, const void* b, int32_t ab_dtype,
                    int64_t n_tokens, int32_t hv,
                    float* log_decay_out, float* gamma_out, float* beta_out,
                    void* stream);

/* ----------------------------------------------------------------------------
 * gdn_prefill -- chunked prefill over packed or ragged requests.
 *
 * Contract of "com.microsoft.GatedDeltaNet" (Inputs, Outputs, Attributes) with
 * the update_rule the update_rule field names (gated_delta when zero), the
 * gates either as given (gate_activation and beta_activation none: they come
 * from gdn_gate or the caller) or fused (gate_activation qwen and
 * beta_activation sigmoid, from the gate_a / gate_b fields), and qk_l2_norm
 * as the qk_l2norm field says (off: keys arrive normalised, as "Gated DeltaNet
 * State Update" Constraints require):
 *  - request r covers tokens [cu_seqlens[r], cu_seqlens[r+1]), both offsets
 *    clamped to [0, total_tokens]; a decreasing pair is an empty request.
 *    cu_seqlens == NULL means uniform packing, request r = [r*seq_len,
 *    (r+1)*seq_len), and then n_seqs * seq_len must equal total_tokens.
 *  - the state of (request r, value head h) starts from initial_state[r,h]
 *    (zeros when initial_state == NULL) and ends in final_state[r,h]; an
 *    empty request copies its incoming state.
 *  - out[t,h,:] = scale * S_t^T q[t, h*hq/hv] for every token t of a request;
 *    rows of tokens no request covers are not written.
 *  - chunk_size is a scheduling hint (0 = 64; accepted 16, 32, 64): it never
 *    changes which result is computed, only the rounding order.
 *
 * Layouts (strides in elements; the last dimension is always dense):
 *   q, k   [total_tokens, hq, dk] io_dtype, strides {token, head}
 *   v      [total_tokens, hv, dv] io_dtype, strides {token, head}
 *   out    [total_tokens, hv, dv] io_dtype, strides {token, head}
 *   decay  [total_tokens, hv] fp32 dense  (decay_kind says log or gamma)
 *   beta   [total_tokens, hv] fp32 dense  (already activated)
 *   cu_seqlens   [n_seqs + 1] int32, or NULL
 *   initial_state, final_state  [n_seqs, hv, dv, dk] fp32 dense, V-major;
 *                final_state may be the same buffer as initial_state (each
 *                state slice is read completely before it is written) but
 *                must not partially overlap it.
 * Gate inputs per update_rule, as the card has them "present exactly" for the
 * rules that use them: the decay source (decay, or gate_a with A_log and
 * dt_bias) is required for gated_delta and gated and must be absent for delta
 * and linear; the beta source (beta, or gate_b) is required for gated_delta
 * and delta and must be absent for gated and linear.  Each source is given
 * or fused on its own, as the card's gate_activation and beta_activation are
 * separate attributes: a fused decay with a given beta, or a given decay with
 * a fused beta, is accepted (it runs on the general kernel, which picks the
 * form per input).
 * Requirements: pointers 16-byte aligned; head and token strides multiples of
 * 8 elements and below 2^23 (in-chunk offsets are 32-bit); total_tokens * hv below 2^31; io_dtype in
 * {GDN_F32, GDN_BF16}.  total_tokens == 0 still writes final_state (copies /
 * zeros).  n_seqs == 0 is a no-op.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t n_seqs;
  int32_t seq_len;         /* used iff cu_seqlens == NULL                     */
  int64_t total_tokens;
  int32_t hq, hv, dk, dv;
  int32_t io_dtype;        /* gdn_dtype of q, k, v and out                     */
  int32_t decay_kind;      /* gdn_decay_kind                                   */
  int32_t chunk_size;      /* 0 = default 64                                   */
  float scale;             /* applied as given                                 */
  const void* q;  int64_t q_stride_token, q_stride_head;
  const void* k;  int64_t k_stride_token, k_stride_head;
  const void* v;  int64_t v_stride_token, v_stride_head;
  void* out;      int64_t out_stride_token, out_stride_head;
  const float* decay;
  const float* beta;
  const int32_t* cu_seqlens;
  const float* initial_state;
  float* final_state;
  /* Optional, zero = off (appended; a zero-filled struct keeps the behaviour
   * above).  qk_l2_norm of the ONNX card: with qk_l2norm != 0 every q and k
   * head vector x is used as x / sqrt(sum(x^2) + qk_l2norm_eps) (the card's
   * epsilon is 1e-12); the inputs are not modified. */
  int32_t qk_l2norm;
  float qk_l2norm_eps;     /* >= 0 and finite                                  */
  /* Fused gate: the gates are computed in the kernel as gdn_gate computes
   * them -- log-decay -exp(A_log[h]) softplus(a + dt_bias[h]) (threshold 20)
   * from gate_a, beta = sigmoid(b) from gate_b; decay and beta must then be
   * NULL and decay_kind is ignored.  A_log, dt_bias [hv] fp32 (with gate_a);
   * gate_a, gate_b [total_tokens, hv] io_dtype, dense. */
  const float* A_log;
  const float* dt_bias;
  const void* gate_a;
  const void* gate_b;
  int32_t update_rule;     /* gdn_update_rule; 0 = gated_delta                 */
  /* State pool (optional; appended).  With state_pool != NULL the states live
   * in a slot-indexed pool laid out as gdn_decode's pool (slot s, head h at
   * state_pool + s*pool_slot_stride + h*pool_head_stride, a dense [dv][dk]
   * fp32 block), and initial_state and final_state must be NULL.  Request r
   * starts from slot read_slot[r] (zeros when read_slot is NULL or the entry
   * is < 0 or >= pool_size) and its final state is stored to slot
   * write_slot[r] (read_slot[r] when write_slot is NULL; nothing when the
   * entry is < 0 or >= pool_size).  A request may read and write one slot; a
   * slot that one request writes and another reads or writes is undefined
   * behaviour.  Same alignment and stride rules as gdn_decode's pool.  With
   * the fused gate and one request per batch row this is a multi-token
   * (chunked) decode over the decode's pool. */
  float* state_pool;
  int32_t pool_size;
  int64_t pool_slot_stride, pool_head_stride;
  const int32_t* read_slot;  /* [n_seqs] or NULL                             */
  const int32_t* write_slot; /* [n_seqs] or NULL                             */
  /* Caller-provided device scratch (appended), 256-byte aligned.  With
   * workspace_bytes >= gdn_prefill_workspace_size(args) > 0 the call runs as
   * a scan over the affine maps of request segments (three launches; see
   * gdn_prefill_workspace_size); otherwise, and whenever that size is 0, the
   * workspace is ignored and every (request, head) is one serial walk over
   * its chunks (for many short bf16 requests one workgroup walks a run of
   * consecutive requests, each from its own initial state).  All compute the
   * same result up to rounding order.  The
   * library neither allocates nor keeps the workspace; calls that share one
   * workspace on overlapping streams race. */
  void* workspace;
  size_t workspace_bytes;
  /* Per-key decay (appended): with decay_per_key != 0, decay is
   * [total_tokens, hv, dk] fp32 dense, one decay per key dimension (the ONNX
   * card's per-key-dimension spelling, in decay_kind's meaning), read in the
   * card's recurrence: each token first scales key column i of the V-major
   * state by its own factor.  Needs a given decay (not gate_a), a given
   * beta or a fused one (gate_b), and an update_rule with a decay (gated_delta or gated; others
   * return GDN_ERR_SHAPE); runs a separate 16-token-chunk MFMA kernel,
   * slower than the scalar-decay kernels. */
  int32_t decay_per_key;
} gdn_prefill_args;

/* Device scratch bytes a gdn_prefill call with these arguments can use; 0
 * when it needs none (args may be NULL: 0).
 *
 * Over any run of tokens the recurrence maps the state entering the run to
 * the state leaving it by an affine map S_out = P S_in + R ("Gated DeltaNet
 * State Update", statement: every step is affine in S), and the chunk is a
 * scheduling choice ("com.microsoft.GatedDeltaNet", Attributes, chunk_size).
 * A call with few (request, value head) units and long requests -- bf16,
 * dk and dv in {64, 128}, the default chunk, scalar decay, gates not mixed,
 * and a serial walk that would fill at most 64 workgroups -- is cut into
 * nseg segments per request (nseg between 4 and 64, chosen from the sizes
 * alone: about 512 workgroups in the first launch, segments of 16 chunks or
 * more on average).  The size is
 *     n_seqs * nseg * hv * dk * (2 dv + dk) * 4 bytes
 * (each segment's map, then each segment's incoming state), at most about
 * 25 MiB for such calls.  Sizes only decide it: the same arguments give the
 * same size on every device. */
size_t gdn_prefill_workspace_size(const gdn_prefill_args* args);

gdn_status gdn_prefill(const gdn_prefill_args* args, void* stream);

/* ----------------------------------------------------------------------------
 * gdn_prefill_noalloc -- gdn_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *
 * Runs exactly what gdn_prefill runs with a workspace of
 * gdn_prefill_workspace_size(args) bytes, taking that workspace from a static
 * device array of GDN_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on
 * every device it runs on until the process ends; args->workspace and
 * args->workspace_bytes are ignored.  It allocates and frees nothing.  A call
 * whose workspace size exceeds the array returns GDN_ERR_UNSUPPORTED (the
 * segment choice keeps every call within about 25 MiB).  Argument errors and
 * results are those of gdn_prefill.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents: calls that overlap on one device (other streams, other
 * threads) race and must be serialised by the caller.  The array needs no
 * clearing -- each call writes every scratch byte it reads.
 * ------------------------------------------------------------------------- */
#define GDN_NOALLOC_SCRATCH_BYTES (32u << 20)
gdn_status gdn_prefill_noalloc(const gdn_prefill_args* args, void* stream);

/* ----------------------------------------------------------------------------
 * gdn_decode -- one fused launch over a slot-indexed fp32 state pool.
 *
 * Contract of "flashinfer.cake_gdp.cake_gated_delta_product_mtp" (parameters
 * and notes), generalised to grouped value heads (hv a multiple of hq) and to
 * dk, dv in {16, 32, 64, 128}; q/k arrive normalised unless qk_l2norm asks
 * for the in-kernel L2 norm (use_qk_l2norm).
 * For every batch row b and value head h:
 *  - rd = read_idx[b]; rd < 0 or rd >= pool_size skips the row entirely: no
 *    pool read, no output store, no write-back, no scatter.
 *  - S = pool[rd, h].  For each token t: gamma_t from the fused gate (as in
 *    gdn_gate, on a[b,t,h]); S <- gamma_t S; then for each sub-step
 *    j < n_householder: beta = sigmoid(b[b,t,j,h]) and
 *    S <- (I - beta k k^T) S + beta k v^T with k = k[b,t,j,h*hq/hv],
 *    v = v[b,t,j,h]; then out[b,t,h] = scale * S^T q[b,t,h*hq/hv].
 *  - scatter_idx != NULL: after every token, S is stored to
 *    pool[scatter_idx[b,t], h] unless that entry is < 0 or >= pool_size; no
 *    end-of-row write-back happens.  Requires disable_state_update == 0.
 *  - otherwise, unless disable_state_update != 0: after the last token S is
 *    stored to pool[wr, h] with wr = write_idx ? write_idx[b] : rd, unless
 *    wr < 0 or wr >= pool_size (the output is still stored).
 *
 * Layouts (dense, row-major):
 *   q [batch, T, hq, dk]; k [batch, T, n_householder, hq, dk];
 *   v [batch, T, n_householder, hv, dv]; a [batch, T, hv];
 *   b [batch, T, n_householder, hv]  -- all io_dtype
 *   A_log, dt_bias [hv] fp32
 *   pool: slot s, head h starts at pool + s*pool_slot_stride +
 *         h*pool_head_stride and holds a dense [dv][dk] fp32 array
 *         (padding between heads or slots is allowed)
 *   read_idx [batch] int32; write_idx [batch] int32 or NULL;
 *   scatter_idx [batch, T] int32 or NULL
 *   out [batch, T, hv, dv] io_dtype; rows of skipped batch rows keep their
 *       previous contents
 * Requirements: pool pointer 16-byte aligned and both pool strides multiples
 * of 4 elements; q, k, v, out 8-byte aligned; 1 <= T <= 64;
 * 1 <= n_householder <= 4; hv <= 65536 (GDN_ERR_UNSUPPORTED above);
 * batch == 0 is a no-op.
 * With T >= 16, n_householder == 1, no scatter_idx and q, k, v, out 16-byte
 * aligned, the call runs the chunked form of the same recurrence (the
 * prefill kernels over the pool, one request per row; the per-key prefill
 * kernel when decay_per_key is given): same results up to rounding order,
 * same skip / write / disable rules.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t batch, T, n_householder;
  int32_t hq, hv, dk, dv;
  int32_t io_dtype;
  int32_t disable_state_update;
  float scale;                     /* applied as given (0.0 included)          */
  const void* q;
  const void* k;
  const void* v;
  const float* A_log;
  const float* dt_bias;
  const void* a;
  const void* b;
  float* pool;
  int32_t pool_size;
  int64_t pool_slot_stride, pool_head_stride;
  const int32_t* read_idx;
  const int32_t* write_idx;
  const int32_t* scatter_idx;
  void* out;
  /* Optional, zero = off (appended).  use_qk_l2norm of the FlashInfer page:
   * with qk_l2norm != 0 every q and k head vector x is used as
   * x / sqrt(sum(x^2) + qk_l2norm_eps) (the page's epsilon is 1e-6). */
  int32_t qk_l2norm;
  float qk_l2norm_eps;     /* >= 0 and finite                                  */
  /* Per-key decay (optional, appended): [batch, T, hv, dk] fp32 log-decay,
   * one per key dimension (the ONNX card's per-key-dimension decay spelling).
   * When given it replaces the fused gate's decay -- each token first scales
   * key column i of the V-major state by exp(decay_per_key[b,t,h,i]) -- and a,
   * A_log, dt_bias are not read (may be NULL); beta still comes from b.
   * 16-byte aligned. */
  const float* decay_per_key;
} gdn_decode_args;

gdn_status gdn_decode(const gdn_decode_args* args, void* stream);

/* ----------------------------------------------------------------------------
 * gdn_conv1d -- causal depthwise conv1d over a ragged batch, reading and
 * updating a slot-indexed conv-state pool in place.
 *
 * Contract of "gated_delta_conv1d_fwd" (parameters and example).  Sequence b
 * covers rows [row_offsets[b], row_offsets[b+1]) of x (offsets clamped to
 * total_tokens; a decreasing pair is an empty sequence).  For every channel c
 * the window is the slot's kernel_size-1 saved inputs, oldest first, followed
 * by the sequence's inputs:
 *     win = conv_state[slot_idx[b], c, :] ++ x[row_offsets[b] .., c]
 *     out[row_offsets[b] + t, c] = sum_{j < K} weight[c, j] * win[t + j]
 * so weight[c, K-1] multiplies the current input; products are summed in
 * fp32 and rounded once to io_dtype.  With write_state != 0 the slot then
 * holds the last K-1 entries of win (an empty sequence leaves it unchanged);
 * with write_state == 0 the pool is only read.  A slot_idx entry >= max_slots
 * reads zeros as its saved inputs and is never written.  Rows of x that no
 * sequence covers leave their out rows untouched.
 *
 * Layouts (row-major):
 *   x    [total_tokens, conv_dim] io_dtype, row stride x_stride_token
 *   out  [total_tokens, conv_dim] io_dtype, row stride out_stride_token
 *   weight     [conv_dim, kernel_size] io_dtype, dense
 *   conv_state [max_slots, conv_dim, kernel_size - 1] io_dtype, dense
 *   slot_idx [n_seqs] uint32; row_offsets [n_seqs + 1] uint32, non-decreasing
 *       (rows that several sequences cover get an unspecified one's output)
 * Requirements: 1 <= kernel_size <= 8; conv_dim a multiple of 16 bytes of
 * io_dtype (8 bf16 / 4 fp32 elements); x, out and conv_state 16-byte aligned;
 * row strides of x and out at least conv_dim and multiples of that same
 * count; out must not overlap x.  conv_state may be NULL only when
 * kernel_size == 1.
 * n_seqs == 0 or total_tokens == 0 is a no-op (every sequence is empty).  Two
 * sequences of one call that name the same valid slot are undefined
 * behaviour.  Two launches: the outputs, then the state write-back, in stream
 * order.
 * ------------------------------------------------------------------------- */
typedef struct {
  int64_t total_tokens;
  int32_t conv_dim;
  int32_t kernel_size;
  int32_t n_seqs;
  int32_t io_dtype;
  int32_t write_state;
  int32_t max_slots;
  const void* x;        int64_t x_stride_token;
  const void* weight;
  void* conv_state;
  const uint32_t* slot_idx;
  const uint32_t* row_offsets;
  void* out;            int64_t out_stride_token;
} gdn_conv1d_args;

gdn_status gdn_conv1d(const gdn_conv1d_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDN_H */
