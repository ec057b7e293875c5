// gdn_prefill.hip -- host dispatch of the chunked prefill.
//
// bf16 problems with dk, dv in {64, 128} and the default chunk go to the
// pair-role kernel (gdn_prefill_pair.hpp).  Everything else goes to
// prefill_kernel (gdn_prefill.hpp), which picks the chunk -- the ONNX card's
// chunk_size is a scheduling hint that never changes the result: 0 means 64,
// and a hint is lowered to the largest chunk whose double-buffered working
// set fits one workgroup's LDS (for fp32 operands with dk = 128 that is 32)
// -- and the (dk, dv) instantiation.
#include <algorithm>
#include <atomic>

#include "gdn_prefill.hpp"
#include "gdn_prefill_pair.hpp"

namespace gdn {

// Device globals.  kGateConst (read-only): what an absent gate input reads,
// log-decay 0 (or a raw gate input 0) at [0], beta 1 at [1].  kZeroRow
// (read-only): the zero V rows of the scan's transition slices.
// kWaitExpired: the number of in-kernel waits that ran out of polls since
// the last clear (0 unless a schedule is broken).  Each device holds its own
// copies; their addresses come from hipGetSymbolAddress on that device.
__device__ float kGateConst[2] = {0.f, 1.f};
__device__ __align__(16) float kZeroRow[32] = {};
__device__ unsigned int kWaitExpired = 0;

struct DeviceSyms {
  float* gate;
  const void* zero;
  unsigned int* wait_err;
};

static hipError_t device_syms(DeviceSyms* out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<float*> cache_g[kMaxDevices];
  static std::atomic<float*> cache_z[kMaxDevices];
  static std::atomic<unsigned int*> cache_w[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* c = cache_g[dev].load(std::memory_order_acquire);
  float* z = cache_z[dev].load(std::memory_order_acquire);
  unsigned int* w = cache_w[dev].load(std::memory_order_acquire);
  if (!c || !z || !w) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(kGateConst));
    if (e != hipSuccess) return e;
    c = static_cast<float*>(addr);
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(kZeroRow));
    if (e != hipSuccess) return e;
    z = static_cast<float*>(addr);
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(kWaitExpired));
    if (e != hipSuccess) return e;
    w = static_cast<unsigned int*>(addr);
    cache_g[dev].store(c, std::memory_order_release);
    cache_z[dev].store(z, std::memory_order_release);
    cache_w[dev].store(w, std::memory_order_release);
  }
  out->gate = c;
  out->zero = z;
  out->wait_err = w;
  return hipSuccess;
}

hipError_t wait_timeouts(uint32_t* count, bool clear) {
  DeviceSyms d;
  hipError_t e = device_syms(&d);
  if (e != hipSuccess) return e;
  unsigned int v = 0;
  e = hipMemcpy(&v, d.wait_err, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  if (count) *count = v;
  if (clear) {
    const unsigned int zero = 0;
    e = hipMemcpy(d.wait_err, &zero, sizeof(zero), hipMemcpyHostToDevice);
  }
  return e;
}

// Whether one fused and one given gate input are combined.
static bool gates_mixed(const gdn_prefill_args& a) {
  return (a.gate_a && a.beta) || (a.gate_b && a.decay);
}

// Segments per request for the scan over segment maps (gdn_prefill_scan.hip),
// or 1 when the call runs as one serial walk per (request, head, slice).
// The scan takes the pair kernel's problems (bf16, dk and dv in {64, 128},
// the default chunk, scalar decay, not called from the decode) when the
// serial walk would fill at most a quarter of a 256-CU chip (64 units):
// enough segments that the local pass has about 512 workgroups, each
// segment on average at least 16 chunks long, at most 64 segments, and at
// least 4 (fewer cannot repay the three passes).  Only sizes decide, so a
// call's result does not depend on the device.
// Requests per workgroup of the pair kernel's multi-request walk: a call
// with more (request, value head, slice) units than one round of the chip
// takes (256 workgroups, one per CU) and short requests (four chunks or
// fewer on average) runs each workgroup over a run of consecutive requests,
// so that the kernel's start (the first chunks' loads and preparation) is
// paid once per workgroup, not once per request.  Sizes only, so a call's
// result never depends on the device.  0: one request per workgroup.
static int pair_request_group(const gdn_prefill_args& a, int lpt) {
  if (lpt || a.n_seqs < 2) return 0;
  const int64_t per_req = (int64_t)a.hv * (a.dv / 64);
  if ((int64_t)a.n_seqs * per_req <= 256) return 0;
  if (a.total_tokens > (int64_t)a.n_seqs * 4 * 64) return 0;
  const int64_t groups = std::max<int64_t>(1, 256 / per_req);
  const int64_t g = std::min<int64_t>((a.n_seqs + groups - 1) / groups, kMultiMax);
  return g >= 2 ? (int)g : 0;
}

int prefill_scan_segments(const gdn_prefill_args& a, int pool_flags) {
  if (pool_flags || a.decay_per_key || a.io_dtype != GDN_BF16 || gates_mixed(a) ||
      !prefill_pair_supported(a.dk, a.dv, a.chunk_size) || a.n_seqs <= 0 || a.total_tokens <= 0)
    return 1;
  const int64_t seg_wgs = (int64_t)a.n_seqs * a.hv * ((a.dv + a.dk) / 64);
  int64_t nseg = 512 / seg_wgs;
  nseg = std::min<int64_t>(nseg, (a.total_tokens / a.n_seqs) / 64 / 16);
  nseg = std::min<int64_t>(nseg, 64);
  return nseg >= 4 ? (int)nseg : 1;
}

size_t prefill_workspace_bytes(const gdn_prefill_args& a) {
  const int nseg = prefill_scan_segments(a, 0);
  if (nseg <= 1) return 0;
  return (size_t)a.n_seqs * nseg * a.hv * a.dk * (2 * (size_t)a.dv + a.dk) * sizeof(float);
}

// The three launches of the scan (see gdn_prefill_scan.hip); the workspace
// holds the segment maps, then every segment's incoming state.
static hipError_t launch_prefill_scan(const PrefillParams& p, const gdn_prefill_args& a, int nseg,
                                      hipStream_t stream) {
  DeviceSyms d;
  hipError_t e = device_syms(&d);
  if (e != hipSuccess) return e;
  const void* zero = d.zero;
  float* ws_map = static_cast<float*>(a.workspace);
  float* ws_in = ws_map + (size_t)a.n_seqs * nseg * a.hv * (a.dv + a.dk) * a.dk;
  PrefillParams pa = p;
  pa.nseg = nseg;
  pa.seg_mode = 1;
  pa.vzero = zero;
  pa.init = nullptr;
  pa.fin = ws_map;
  pa.pool = nullptr;
  pa.rslot = pa.wslot = nullptr;
  e = prefill_pair_bf16(pa, a.dk, stream);
  if (e != hipSuccess) return e;
  e = launch_scan_combine(p, nseg, a.dk, ws_map, ws_in, stream);
  if (e != hipSuccess) return e;
  PrefillParams pb = p;
  pb.nseg = nseg;
  pb.seg_mode = 2;
  pb.init = ws_in;
  pb.fin = nullptr;
  pb.pool = nullptr;
  pb.rslot = pb.wslot = nullptr;
  return prefill_pair_bf16(pb, a.dk, stream);
}

hipError_t launch_prefill(const gdn_prefill_args& a, hipStream_t stream, int pool_flags) {
  DeviceSyms syms;
  const hipError_t se = device_syms(&syms);
  if (se != hipSuccess) return se;
  PrefillParams p;
  p.wait_err = syms.wait_err;
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
  p.nseg = 1; p.nsv = 1; p.seg_mode = 0; p.vzero = nullptr;
  p.lpt = a.cu_seqlens && a.n_seqs >= 2 && a.n_seqs <= kLptMax &&
          a.total_tokens >= (int64_t)kLptMinTokens * a.n_seqs;
  p.rgroup = 0;
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
  const bool mixed = gates_mixed(a);
  if (a.gate_a) p.decay_is_gamma = 0;  // the fused gate yields log-space decay
  const bool absent = fused ? (!a.gate_a || !a.gate_b) : (!a.decay || !a.beta);
  if (absent && !mixed) {
    // a rule without decay or beta: the missing source reads the constants
    float* c = syms.gate;
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
  const int nseg = prefill_scan_segments(a, pool_flags);
  if (nseg > 1 && a.workspace && a.workspace_bytes >= prefill_workspace_bytes(a))
    return launch_prefill_scan(p, a, nseg, stream);
  if (bf && !mixed && prefill_pair_supported(a.dk, a.dv, a.chunk_size)) {
    p.rgroup = pair_request_group(a, p.lpt);
    return prefill_pair_bf16(p, a.dk, stream);
  }
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
