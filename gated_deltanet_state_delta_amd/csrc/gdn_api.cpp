// gdn_api.cpp -- the C ABI of libgdn: argument validation and dispatch.
//
// Everything checked here is host-visible metadata (pointers, sizes, strides,
// dtypes).  No device memory is read and nothing is synchronised, so every
// entry point can be captured in a HIP graph.  Data-dependent conditions
// (cu_seqlens contents, slot indices) are handled on the device as the pages
// prescribe: clamping and skipping, never faulting.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/libgdn.h"
#include "gdn_kernels.hpp"

namespace {

thread_local char g_err[512] = "";

gdn_status fail(gdn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

gdn_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return GDN_OK;
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Static device scratch of gdn_prefill_noalloc: one copy per device, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: only the address hipGetSymbolAddress returns for the
// current device is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

// The current device's address of `scratch`, looked up once per device (with
// that device current) and kept.
hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = cache[dev].load(std::memory_order_acquire);
  if (!ptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    cache[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

bool head_size_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }
size_t elem_size(int32_t dt) { return dt == GDN_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

const char* gdn_last_error(void) { return g_err; }

const char* gdn_version(void) { return "0.1.0"; }

gdn_status gdn_gate(const float* A_log, const float* dt_bias, const void* a, const void* b,
                    int32_t ab_dtype, int64_t n_tokens, int32_t hv, float* log_decay_out,
                    float* gamma_out, float* beta_out, void* stream) {
  g_err[0] = 0;
  if (ab_dtype != GDN_F32 && ab_dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "gdn_gate: ab_dtype %d", ab_dtype);
  if (n_tokens < 0 || hv <= 0) return fail(GDN_ERR_SHAPE, "gdn_gate: n_tokens=%lld hv=%d", (long long)n_tokens, hv);
  if ((log_decay_out || gamma_out) && !a) return fail(GDN_ERR_NULL, "gdn_gate: decay output requested without a");
  if (beta_out && !b) return fail(GDN_ERR_NULL, "gdn_gate: beta output requested without b");
  if (a && (!A_log || !dt_bias)) return fail(GDN_ERR_NULL, "gdn_gate: a given without A_log / dt_bias");
  if (n_tokens == 0) return GDN_OK;
  // an input whose outputs are all absent is ignored
  const void* ua = (log_decay_out || gamma_out) ? a : nullptr;
  const void* ub = beta_out ? b : nullptr;
  if (!ua && !ub) return GDN_OK;
  return from_hip(gdn::launch_gate(A_log, dt_bias, ua, ub, ab_dtype, n_tokens, hv, log_decay_out,
                                   gamma_out, beta_out, (hipStream_t)stream),
                  "gdn_gate launch");
}

gdn_status gdn_wait_timeouts(uint32_t* count, int32_t clear) {
  g_err[0] = 0;
  if (!count) return fail(GDN_ERR_NULL, "gdn_wait_timeouts: count is NULL");
  return from_hip(gdn::wait_timeouts(count, clear != 0), "gdn_wait_timeouts");
}

size_t gdn_prefill_workspace_size(const gdn_prefill_args* args) {
  return args ? gdn::prefill_workspace_bytes(*args) : 0;
}

// Every host-visible check of a gdn_prefill call, in order; *noop is set
// when the call is valid and has nothing to do (n_seqs == 0).
static gdn_status prefill_check(const gdn_prefill_args& a, bool* noop) {
  *noop = false;
  if (a.io_dtype != GDN_F32 && a.io_dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "gdn_prefill: io_dtype %d", a.io_dtype);
  if (a.decay_kind != GDN_DECAY_LOG && a.decay_kind != GDN_DECAY_GAMMA)
    return fail(GDN_ERR_DTYPE, "gdn_prefill: decay_kind %d", a.decay_kind);
  if (a.n_seqs < 0 || a.total_tokens < 0 || a.hq <= 0 || a.hv <= 0 || a.dk <= 0 || a.dv <= 0)
    return fail(GDN_ERR_SHAPE, "gdn_prefill: bad sizes n_seqs=%d T=%lld hq=%d hv=%d dk=%d dv=%d", a.n_seqs,
                (long long)a.total_tokens, a.hq, a.hv, a.dk, a.dv);
  if (a.hv % a.hq != 0) return fail(GDN_ERR_SHAPE, "gdn_prefill: hv=%d is not a multiple of hq=%d", a.hv, a.hq);
  if (!head_size_ok(a.dk) || !head_size_ok(a.dv))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill: dk=%d dv=%d (supported: 16, 32, 64, 128)", a.dk, a.dv);
  if (a.chunk_size != 0 && a.chunk_size != 16 && a.chunk_size != 32 && a.chunk_size != 64)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill: chunk_size=%d (supported: 0, 16, 32, 64)", a.chunk_size);
  if (!a.cu_seqlens && (a.seq_len < 0 || (int64_t)a.n_seqs * a.seq_len != a.total_tokens))
    return fail(GDN_ERR_SHAPE, "gdn_prefill: without cu_seqlens n_seqs*seq_len (%d*%d) must equal total_tokens %lld",
                a.n_seqs, a.seq_len, (long long)a.total_tokens);
  if (a.qk_l2norm && !(a.qk_l2norm_eps >= 0.f && a.qk_l2norm_eps <= 3.0e38f))
    return fail(GDN_ERR_SHAPE, "gdn_prefill: qk_l2norm_eps must be finite and >= 0");
  if (a.update_rule < GDN_RULE_GATED_DELTA || a.update_rule > GDN_RULE_LINEAR)
    return fail(GDN_ERR_DTYPE, "gdn_prefill: update_rule %d", a.update_rule);
  if ((int64_t)a.total_tokens * a.hv >= (int64_t(1) << 31))
    return fail(GDN_ERR_SHAPE, "gdn_prefill: total_tokens * hv must be below 2^31");
  if (a.total_tokens > 0) {
    // gate sources: present exactly for the rules that use them (not read
    // at all when there are no tokens)
    const bool uses_decay = a.update_rule == GDN_RULE_GATED_DELTA || a.update_rule == GDN_RULE_GATED;
    const bool uses_beta = a.update_rule == GDN_RULE_GATED_DELTA || a.update_rule == GDN_RULE_DELTA;
    const bool has_decay = a.decay || a.gate_a, has_beta = a.beta || a.gate_b;
    if (a.decay && a.gate_a) return fail(GDN_ERR_SHAPE, "gdn_prefill: decay and gate_a are both given");
    if (a.beta && a.gate_b) return fail(GDN_ERR_SHAPE, "gdn_prefill: beta and gate_b are both given");
    if (has_decay != uses_decay)
      return fail(uses_decay ? GDN_ERR_NULL : GDN_ERR_SHAPE, "gdn_prefill: update_rule %d %s a decay input",
                  a.update_rule, uses_decay ? "needs" : "takes no");
    if (has_beta != uses_beta)
      return fail(uses_beta ? GDN_ERR_NULL : GDN_ERR_SHAPE, "gdn_prefill: update_rule %d %s a beta input",
                  a.update_rule, uses_beta ? "needs" : "takes no");
  }
  if (a.gate_a && (!a.A_log || !a.dt_bias)) return fail(GDN_ERR_NULL, "gdn_prefill: gate_a needs A_log and dt_bias");
  if (a.decay_per_key && a.gate_a)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill: decay_per_key takes the decay as a given input (not gate_a)");
  if (a.decay_per_key && a.update_rule != GDN_RULE_GATED_DELTA && a.update_rule != GDN_RULE_GATED)
    return fail(GDN_ERR_SHAPE, "gdn_prefill: decay_per_key needs an update_rule with a decay (gated_delta, gated)");
  if (a.state_pool) {
    if (a.initial_state || a.final_state)
      return fail(GDN_ERR_SHAPE, "gdn_prefill: state_pool replaces initial_state and final_state (pass NULL)");
    if (a.pool_size < 0) return fail(GDN_ERR_SHAPE, "gdn_prefill: pool_size=%d", a.pool_size);
    if (!aligned(a.state_pool, 16) || a.pool_slot_stride % 4 != 0 || a.pool_head_stride % 4 != 0 ||
        a.pool_slot_stride < 0 || a.pool_head_stride < 0)
      return fail(GDN_ERR_LAYOUT, "gdn_prefill: state_pool must be 16-byte aligned with strides multiple of 4 elements");
    if (a.pool_head_stride < (int64_t)a.dv * a.dk ||
        a.pool_slot_stride < (int64_t)(a.hv - 1) * a.pool_head_stride + (int64_t)a.dv * a.dk)
      return fail(GDN_ERR_LAYOUT, "gdn_prefill: pool strides smaller than the dense extents");
  } else if (a.read_slot || a.write_slot) {
    return fail(GDN_ERR_SHAPE, "gdn_prefill: read_slot / write_slot need state_pool");
  }
  if (a.n_seqs == 0) {
    *noop = true;
    return GDN_OK;
  }
  if (!a.final_state && !a.state_pool) return fail(GDN_ERR_NULL, "gdn_prefill: final_state is NULL");
  if (a.total_tokens > 0 && (!a.q || !a.k || !a.v || !a.out))
    return fail(GDN_ERR_NULL, "gdn_prefill: q, k, v and out are required");
  const void* ptrs[] = {a.q, a.k, a.v, a.out, a.decay, a.beta, a.initial_state, a.final_state, a.cu_seqlens,
                        a.state_pool};
  for (const void* q : ptrs)
    if (q && !aligned(q, 16)) return fail(GDN_ERR_LAYOUT, "gdn_prefill: pointers must be 16-byte aligned");
  const int64_t strides[] = {a.q_stride_token, a.q_stride_head, a.k_stride_token, a.k_stride_head,
                             a.v_stride_token, a.v_stride_head, a.out_stride_token, a.out_stride_head};
  // The kernels form in-chunk row offsets (up to 63 rows of a stride, in bytes
  // of fp32 at most) in 32-bit arithmetic: strides below 2^23 elements keep
  // 63 * stride * 4 plus a row's extent below 2^31.
  for (int64_t s : strides)
    if (s < 0 || s % 8 != 0 || s >= (int64_t(1) << 23))
      return fail(GDN_ERR_LAYOUT, "gdn_prefill: strides must be non-negative multiples of 8 elements below 2^23");
  if (a.total_tokens > 0) {
    if (a.q_stride_head < a.dk || a.k_stride_head < a.dk || a.v_stride_head < a.dv || a.out_stride_head < a.dv ||
        a.q_stride_token < (int64_t)a.hq * a.dk || a.k_stride_token < (int64_t)a.hq * a.dk ||
        a.v_stride_token < (int64_t)a.hv * a.dv || a.out_stride_token < (int64_t)a.hv * a.dv)
      return fail(GDN_ERR_LAYOUT, "gdn_prefill: strides smaller than the dense extents");
  }
  if (a.initial_state && a.initial_state != a.final_state) {
    const char* i0 = (const char*)a.initial_state;
    const char* f0 = (const char*)a.final_state;
    const size_t bytes = (size_t)a.n_seqs * a.hv * a.dv * a.dk * sizeof(float);
    if (i0 < f0 + bytes && f0 < i0 + bytes)
      return fail(GDN_ERR_LAYOUT, "gdn_prefill: initial_state and final_state partially overlap");
  }
  return GDN_OK;
}

gdn_status gdn_prefill(const gdn_prefill_args* p, void* stream) {
  g_err[0] = 0;
  if (!p) return fail(GDN_ERR_NULL, "gdn_prefill: args is NULL");
  bool noop = false;
  const gdn_status st = prefill_check(*p, &noop);
  if (st != GDN_OK || noop) return st;
  return from_hip(gdn::launch_prefill(*p, (hipStream_t)stream), "gdn_prefill launch");
}

gdn_status gdn_prefill_noalloc(const gdn_prefill_args* p, void* stream) {
  g_err[0] = 0;
  if (!p) return fail(GDN_ERR_NULL, "gdn_prefill_noalloc: args is NULL");
  bool noop = false;
  const gdn_status st = prefill_check(*p, &noop);
  if (st != GDN_OK || noop) return st;
  const size_t need = gdn::prefill_workspace_bytes(*p);
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
    return fail(GDN_ERR_UNSUPPORTED,
                "gdn_prefill_noalloc: the call needs %zu bytes of scratch, more than the %zu of the static array "
                "(use gdn_prefill with a workspace)",
                need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
  gdn_prefill_args a = *p;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  if (need > 0) {
    void* ptr = nullptr;
    const hipError_t e = noalloc_scratch(&ptr);
    if (e != hipSuccess) return from_hip(e, "gdn_prefill_noalloc: static scratch address");
    a.workspace = ptr;
    a.workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
  }
  return from_hip(gdn::launch_prefill(a, (hipStream_t)stream), "gdn_prefill_noalloc launch");
}

gdn_status gdn_decode(const gdn_decode_args* p, void* stream) {
  g_err[0] = 0;
  if (!p) return fail(GDN_ERR_NULL, "gdn_decode: args is NULL");
  const gdn_decode_args& a = *p;
  if (a.io_dtype != GDN_F32 && a.io_dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "gdn_decode: io_dtype %d", a.io_dtype);
  if (a.batch < 0 || a.T <= 0 || a.hq <= 0 || a.hv <= 0 || a.dk <= 0 || a.dv <= 0 || a.pool_size < 0)
    return fail(GDN_ERR_SHAPE, "gdn_decode: bad sizes batch=%d T=%d hq=%d hv=%d dk=%d dv=%d pool_size=%d", a.batch,
                a.T, a.hq, a.hv, a.dk, a.dv, a.pool_size);
  if (a.T > 64) return fail(GDN_ERR_UNSUPPORTED, "gdn_decode: T=%d (supported 1..64)", a.T);
  if (a.n_householder < 1 || a.n_householder > 4)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_decode: n_householder=%d (supported 1..4)", a.n_householder);
  if (a.hv % a.hq != 0) return fail(GDN_ERR_SHAPE, "gdn_decode: hv=%d is not a multiple of hq=%d", a.hv, a.hq);
  if (a.hv > 65536) return fail(GDN_ERR_UNSUPPORTED, "gdn_decode: hv=%d (supported up to 65536)", a.hv);
  if (a.qk_l2norm && !(a.qk_l2norm_eps >= 0.f && a.qk_l2norm_eps <= 3.0e38f))
    return fail(GDN_ERR_SHAPE, "gdn_decode: qk_l2norm_eps must be finite and >= 0");
  if (!head_size_ok(a.dk) || !head_size_ok(a.dv))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_decode: dk=%d dv=%d (supported: 16, 32, 64, 128)", a.dk, a.dv);
  if (a.scatter_idx && a.disable_state_update)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_decode: scatter_idx requires disable_state_update == 0");
  if (a.batch == 0) return GDN_OK;
  if (!a.q || !a.k || !a.v || !a.b || !a.pool || !a.read_idx || !a.out)
    return fail(GDN_ERR_NULL, "gdn_decode: q, k, v, b, pool, read_idx and out are required");
  if (!a.decay_per_key && (!a.A_log || !a.dt_bias || !a.a))
    return fail(GDN_ERR_NULL, "gdn_decode: A_log, dt_bias and a are required (or decay_per_key)");
  if (a.decay_per_key && !aligned(a.decay_per_key, 16))
    return fail(GDN_ERR_LAYOUT, "gdn_decode: decay_per_key must be 16-byte aligned");
  if (!aligned(a.pool, 16) || a.pool_slot_stride % 4 != 0 || a.pool_head_stride % 4 != 0 ||
      a.pool_slot_stride < 0 || a.pool_head_stride < 0)
    return fail(GDN_ERR_LAYOUT, "gdn_decode: pool must be 16-byte aligned with strides multiple of 4 elements");
  if (a.pool_head_stride < (int64_t)a.dv * a.dk || a.pool_slot_stride < (int64_t)(a.hv - 1) * a.pool_head_stride + (int64_t)a.dv * a.dk)
    return fail(GDN_ERR_LAYOUT, "gdn_decode: pool strides smaller than the dense extents");
  const size_t es = elem_size(a.io_dtype);
  const void* act[] = {a.q, a.k, a.v, a.out};
  for (const void* q : act)
    if (!aligned(q, es == 2 ? 8 : 16)) return fail(GDN_ERR_LAYOUT, "gdn_decode: q, k, v, out must be aligned to 4 elements");
  return from_hip(gdn::launch_decode(a, (hipStream_t)stream), "gdn_decode launch");
}

gdn_status gdn_conv1d(const gdn_conv1d_args* p, void* stream) {
  g_err[0] = 0;
  if (!p) return fail(GDN_ERR_NULL, "gdn_conv1d: args is NULL");
  const gdn_conv1d_args& a = *p;
  if (a.io_dtype != GDN_F32 && a.io_dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "gdn_conv1d: io_dtype %d", a.io_dtype);
  if (a.total_tokens < 0 || a.conv_dim <= 0 || a.n_seqs < 0 || a.max_slots < 0)
    return fail(GDN_ERR_SHAPE, "gdn_conv1d: bad sizes T=%lld conv_dim=%d n_seqs=%d max_slots=%d",
                (long long)a.total_tokens, a.conv_dim, a.n_seqs, a.max_slots);
  if (a.kernel_size < 1 || a.kernel_size > 8)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_conv1d: kernel_size=%d (supported 1..8)", a.kernel_size);
  const int64_t ve = a.io_dtype == GDN_BF16 ? 8 : 4;
  if (a.conv_dim % ve != 0)
    return fail(GDN_ERR_LAYOUT, "gdn_conv1d: conv_dim=%d is not a multiple of %lld elements", a.conv_dim, (long long)ve);
  if (a.n_seqs == 0 || a.total_tokens == 0) return GDN_OK;
  if (!a.x || !a.weight || !a.slot_idx || !a.row_offsets || !a.out || (a.kernel_size > 1 && !a.conv_state))
    return fail(GDN_ERR_NULL, "gdn_conv1d: x, weight, slot_idx, row_offsets, out (and conv_state for kernel_size > 1) are required");
  if (a.x_stride_token < a.conv_dim || a.out_stride_token < a.conv_dim || a.x_stride_token % ve != 0 ||
      a.out_stride_token % ve != 0)
    return fail(GDN_ERR_LAYOUT, "gdn_conv1d: row strides must be >= conv_dim and multiples of %lld elements", (long long)ve);
  if (!aligned(a.x, 16) || !aligned(a.out, 16) || !aligned(a.conv_state, 16))
    return fail(GDN_ERR_LAYOUT, "gdn_conv1d: x, out and conv_state must be 16-byte aligned");
  {
    const size_t es = elem_size(a.io_dtype);
    const uintptr_t x0 = (uintptr_t)a.x, o0 = (uintptr_t)a.out;
    const uintptr_t x1 = x0 + ((size_t)(a.total_tokens - 1) * a.x_stride_token + a.conv_dim) * es;
    const uintptr_t o1 = o0 + ((size_t)(a.total_tokens - 1) * a.out_stride_token + a.conv_dim) * es;
    if (x0 < o1 && o0 < x1) return fail(GDN_ERR_LAYOUT, "gdn_conv1d: out overlaps x");
  }
  return from_hip(gdn::launch_conv1d(a, (hipStream_t)stream), "gdn_conv1d launch");
}

}  // extern "C"
