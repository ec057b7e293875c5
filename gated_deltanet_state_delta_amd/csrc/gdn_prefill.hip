// gdn_prefill.hip -- host dispatch of the chunked prefill.
//
// bf16 problems with dk, dv in {64, 128} and the default chunk go to the
// pair-role kernel (gdn_prefill_pair.hpp).  Everything else goes to
// prefill_kernel (gdn_prefill.hpp), which picks the chunk -- the ONNX card's
// chunk_size is a scheduling hint that never changes the result: 0 means 64,
// and a hint is lowered to the largest chunk whose double-buffered working
// set fits one workgroup's LDS (for fp32 operands with dk = 128 that is 32)
// -- and the (dk, dv) instantiation.
#include <atomic>

#include "gdn_prefill.hpp"
#include "gdn_prefill_pair.hpp"

namespace gdn {

// What an absent gate input reads: log-decay 0 (or a raw gate input 0) at
// [0], beta 1 at [1].  Each device holds its own copy; its address comes
// from hipGetSymbolAddress on that device.
__device__ float kGateConst[2] = {0.f, 1.f};

static hipError_t gate_consts(float** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<float*> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* c = cache[dev].load(std::memory_order_acquire);
  if (!c) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(kGateConst));
    if (e != hipSuccess) return e;
    c = static_cast<float*>(addr);
    cache[dev].store(c, std::memory_order_release);
  }
  *out = c;
  return hipSuccess;
}

hipError_t launch_prefill(const gdn_prefill_args& a, hipStream_t stream, int pool_flags) {
  PrefillParams p;
  p.pool_flags = pool_flags;
  p.q = a.q; p.k = a.k; p.v = a.v; p.out = a.out;
  p.q_st = a.q_stride_token; p.q_sh = a.q_stride_head;
  p.k_st = a.k_stride_token; p.k_sh = a.k_stride_head;
  p.v_st = a.v_stride_token; p.v_sh = a.v_stride_head;
  p.o_st = a.out_stride_token; p.o_sh = a.out_stride_head;
  p.decay = a.decay; p.beta = a.beta; p.cu = a.cu_seqlens;
  p.init = a.initial_state; p.fin = a.final_state;
  p.pool = a.state_pool; p.rslot = a.read_slot; p.wslot = a.write_slot;
  p.pss = a.pool_slot_stride; p.phs = a.pool_head_stride; p.pool_size = a.pool_size;
  if (a.state_pool) { p.init = a.state_pool; p.fin = a.state_pool; }
  p.T = a.total_tokens; p.n_seqs = a.n_seqs; p.seq_len = a.seq_len;
  p.hq = a.hq; p.hv = a.hv; p.dv = a.dv; p.nsplit = 1;
  p.decay_is_gamma = a.decay_kind == GDN_DECAY_GAMMA;
  p.scale = a.scale;
  p.qk_norm = a.qk_l2norm != 0;
  p.qk_eps = a.qk_l2norm_eps;
  p.A_log = a.A_log; p.dt_bias = a.dt_bias; p.ga = a.gate_a; p.gb = a.gate_b;
  // update_rule: the delta retrieval is kept by gated_delta and delta
  p.rho = (a.update_rule == GDN_RULE_GATED_DELTA || a.update_rule == GDN_RULE_DELTA) ? 1.f : 0.f;
  p.dmask = p.bmask = ~int64_t(0);
  // Each gate input is given or fused on its own ("com.microsoft.GatedDeltaNet",
  // Attributes: gate_activation and beta_activation).  One fused and one given
  // input ("mixed") runs on the general kernel, which chooses per input.
  const bool fused = a.gate_a || a.gate_b;
  const bool mixed = (a.gate_a && a.beta) || (a.gate_b && a.decay);
  if (a.gate_a) p.decay_is_gamma = 0;  // the fused gate yields log-space decay
  const bool absent = fused ? (!a.gate_a || !a.gate_b) : (!a.decay || !a.beta);
  if (absent && !mixed) {
    // a rule without decay or beta: the missing source reads the constants
    float* c = nullptr;
    const hipError_t e = gate_consts(&c);
    if (e != hipSuccess) return e;
    if (fused) {
      if (!a.gate_a) { p.ga = c; p.A_log = c; p.dt_bias = c; p.dmask = 0; }
      if (!a.gate_b) { p.gb = c; p.bmask = 0; }
    } else {
      if (!a.decay) { p.decay = c; p.dmask = 0; p.decay_is_gamma = 0; }
      if (!a.beta) { p.beta = c + 1; p.bmask = 0; }
    }
  }
  const bool bf = a.io_dtype == GDN_BF16;
  if (a.decay_per_key) return launch_prefill_pk(p, a.dk, a.dv, bf, stream);
  if (bf && !mixed && prefill_pair_supported(a.dk, a.dv, a.chunk_size)) return prefill_pair_bf16(p, a.dk, stream);
  const int hint = a.chunk_size != 0 ? a.chunk_size : 64;
  const int c = bf ? prefill_chunk_for<__bf16>(a.dk, a.dv, hint)
                   : prefill_chunk_for<float>(a.dk, a.dv, hint);
  switch (c) {
    case 16: return bf ? prefill_bf16_c16(p, a.dk, a.dv, stream) : prefill_f32_c16(p, a.dk, a.dv, stream);
    case 32: return bf ? prefill_bf16_c32(p, a.dk, a.dv, stream) : prefill_f32_c32(p, a.dk, a.dv, stream);
    case 64: return bf ? prefill_bf16_c64(p, a.dk, a.dv, stream) : prefill_f32_c64(p, a.dk, a.dv, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
