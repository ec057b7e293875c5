// gdn_decode.hip -- decode dispatch and the chunked multi-token route (the
// kernel is in gdn_decode.hpp; value width 128 is instantiated in
// gdn_decode_dv128.hip).
#include "gdn_decode.hpp"

namespace gdn {

template <typename IO, int DK>
static hipError_t dispatch_dv(const DecodeParams& p, int dv, hipStream_t s) {
  switch (dv) {
    case 16: return launch_decode_t<IO, DK, 16>(p, s);
    case 32: return launch_decode_t<IO, DK, 32>(p, s);
    case 64: return launch_decode_t<IO, DK, 64>(p, s);
    case 128: return launch_decode_dv128(p, DK, sizeof(IO) == 2, s);
  }
  return hipErrorInvalidValue;
}

template <typename IO>
static hipError_t dispatch_dk(const DecodeParams& p, int dk, int dv, hipStream_t s) {
  switch (dk) {
    case 16: return dispatch_dv<IO, 16>(p, dv, s);
    case 32: return dispatch_dv<IO, 32>(p, dv, s);
    case 64: return dispatch_dv<IO, 64>(p, dv, s);
    case 128: return dispatch_dv<IO, 128>(p, dv, s);
  }
  return hipErrorInvalidValue;
}

// Many tokens per row, one delta step per token, no per-token scatter: the
// chunked prefill over the pool computes the same recurrence with MFMA
// instead of one state pass per token.  Measured on B64 x Hv32 x 128x128 bf16
// (token loop -> chunked): T = 16: 146 -> 112 us, T = 32: 256 -> 127 us,
// T = 64: 470 -> 174 us (the token loop stays ahead below 16 tokens: 74 vs
// 144 us at T = 4).  The chunk follows T (see launch_decode_chunked).  Every
// activation must be 16-byte aligned, as the prefill kernels require.
static bool decode_as_prefill(const gdn_decode_args& a) {
  if (a.T < 16 || a.n_householder != 1 || a.scatter_idx) return false;
  if ((int64_t)a.batch * a.T * a.hv >= (int64_t(1) << 31)) return false;
  const void* ptrs[] = {a.q, a.k, a.v, a.out};
  for (const void* q : ptrs)
    if ((uintptr_t)q % 16 != 0) return false;
  return true;
}

static hipError_t launch_decode_chunked(const gdn_decode_args& a, hipStream_t stream) {
  gdn_prefill_args pa = {};
  pa.n_seqs = a.batch;
  pa.seq_len = a.T;  // request r = batch row r: tokens [r*T, (r+1)*T)
  pa.total_tokens = (int64_t)a.batch * a.T;
  pa.hq = a.hq; pa.hv = a.hv; pa.dk = a.dk; pa.dv = a.dv;
  pa.io_dtype = a.io_dtype;
  pa.decay_kind = GDN_DECAY_LOG;
  // bf16 with the pair kernel's head sizes and T >= 32: its 64-token chunks
  // with the multi-request walk (each workgroup runs a run of rows); B64 x
  // Hv32 x 128x128: T = 32 125 -> 123 us, T = 64 177 -> 133 us against the
  // general kernel at 32 tokens, which stays ahead at T = 16 (109 vs 123
  // us).  Otherwise the general kernel at 16 or 32 tokens.
  const bool pair = a.T >= 16 && a.io_dtype == GDN_BF16 && !a.decay_per_key && (a.dk == 64 || a.dk == 128) &&
                    (a.dv == 64 || a.dv == 128);
  pa.chunk_size = pair ? 0 : (a.T < 32 ? 16 : 32);
  pa.scale = a.scale;
  pa.q = a.q; pa.q_stride_token = (int64_t)a.hq * a.dk; pa.q_stride_head = a.dk;
  pa.k = a.k; pa.k_stride_token = (int64_t)a.hq * a.dk; pa.k_stride_head = a.dk;  // n = 1
  pa.v = a.v; pa.v_stride_token = (int64_t)a.hv * a.dv; pa.v_stride_head = a.dv;
  pa.out = a.out; pa.out_stride_token = (int64_t)a.hv * a.dv; pa.out_stride_head = a.dv;
  pa.qk_l2norm = a.qk_l2norm; pa.qk_l2norm_eps = a.qk_l2norm_eps;
  if (a.decay_per_key) {
    // per-key decay: given (log space, [batch * T, hv, dk]), beta fused from b
    pa.decay = a.decay_per_key;
    pa.decay_per_key = 1;
    pa.gate_b = a.b;
  } else {
    pa.A_log = a.A_log; pa.dt_bias = a.dt_bias; pa.gate_a = a.a; pa.gate_b = a.b;
  }
  pa.update_rule = GDN_RULE_GATED_DELTA;
  pa.state_pool = a.pool; pa.pool_size = a.pool_size;
  pa.pool_slot_stride = a.pool_slot_stride; pa.pool_head_stride = a.pool_head_stride;
  pa.read_slot = a.read_idx;
  pa.write_slot = a.write_idx;  // NULL: the read slot, as in the token loop
  const int flags = kPoolSkipUnread | (a.disable_state_update ? kPoolNoWrite : 0);
  return launch_prefill(pa, stream, flags);
}

hipError_t launch_decode(const gdn_decode_args& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (decode_as_prefill(a)) return launch_decode_chunked(a, stream);
  DecodeParams p;
  p.q = a.q; p.k = a.k; p.v = a.v;
  p.A_log = a.A_log; p.dt_bias = a.dt_bias;
  p.a = a.a; p.b = a.b;
  p.pool = a.pool;
  p.slot_stride = a.pool_slot_stride; p.head_stride = a.pool_head_stride;
  p.read_idx = a.read_idx; p.write_idx = a.write_idx; p.scatter_idx = a.scatter_idx;
  p.out = a.out;
  p.batch = a.batch; p.T = a.T; p.nhh = a.n_householder; p.hq = a.hq; p.hv = a.hv;
  p.pool_size = a.pool_size; p.disable = a.disable_state_update; p.scale = a.scale;
  p.qk_norm = a.qk_l2norm != 0; p.qk_eps = a.qk_l2norm_eps;
  p.decay_pk = a.decay_per_key;
  if (a.io_dtype == GDN_BF16) return dispatch_dk<__bf16>(p, a.dk, a.dv, stream);
  return dispatch_dk<float>(p, a.dk, a.dv, stream);
}

}  // namespace gdn
