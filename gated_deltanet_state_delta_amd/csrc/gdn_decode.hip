// gdn_decode.hip -- streaming decode / multi-token verification over a slot pool.
//
// Contract: "flashinfer.cake_gdp.cake_gated_delta_product_mtp" (parameters and
// notes) -- per batch row and value head: read the state from the row's read
// slot, per token decay it once by the fused gate, apply num_householder
// delta sub-steps (own k, v, sigmoid beta), read out after the sub-steps,
// scatter after each token or write back once after the last.
//
// Design (HBM-bound): the state of one head is a V-major [DV][DK] fp32 array;
// every V-row evolves independently (the recurrence only couples a row with
// itself through k).  A row is held by L = DK/16 lanes, 16 floats per lane
// in four 16-byte segments, so each wave instruction touches whole 128-byte
// lines.  The row is read once into VGPRs with non-temporal 16-byte loads,
// updated in registers for every token and sub-step (dot products reduced
// across the L lanes with DPP), and written once per required slot with
// non-temporal 16-byte stores.  One workgroup covers ROWS rows of one
// (batch row, head); skipped rows exit before touching memory.  The per-token
// inputs of the workgroup (k and q rows, its slice of v, and the gates, which
// one thread per token computes) are staged in LDS up to TT tokens at a time,
// so the per-token chain reads LDS instead of waiting on global loads.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const float* A_log;
  const float* dt_bias;
  const void* a;
  const void* b;
  float* pool;
  int64_t slot_stride, head_stride;
  const int32_t* read_idx;
  const int32_t* write_idx;
  const int32_t* scatter_idx;
  void* out;
  int batch, T, nhh, hq, hv, pool_size, disable;
  float scale;
  int qk_norm;    // q, k used as x * rsqrt(sum x^2 + qk_eps) (use_qk_l2norm)
  float qk_eps;
  const float* decay_pk;  // [B, T, hv, DK] log-decay per key, or nullptr (fused gate)
};

// Four io elements moved as one word group (8 bytes for bf16, 16 for fp32).
template <typename IO> struct Quad4 { typedef u32x4 type; };
template <> struct Quad4<__bf16> { typedef uint32_t type __attribute__((ext_vector_type(2))); };

template <typename IO, int DK, int DV, int ROWS>
__global__ void __launch_bounds__(ROWS * (DK / 16))
decode_kernel(const DecodeParams p) {
  constexpr int L = DK / 16;          // lanes per V-row
  constexpr int NRB = DV / ROWS;      // row blocks per head
  constexpr int NT = ROWS * L;        // threads
  constexpr int TT = 8;               // tokens staged per pass
  constexpr int NJ = 4;               // most sub-steps per token
  typedef typename Quad4<IO>::type Q4;
  __shared__ __attribute__((aligned(16))) IO sk[TT * NJ * DK];    // [t][j][DK]
  __shared__ __attribute__((aligned(16))) IO sq[TT * DK];         // [t][DK]
  __shared__ __attribute__((aligned(16))) IO sv[TT * NJ * ROWS];  // [t][j][rows of this block]
  __shared__ float sgam[TT], sbet[TT * NJ];
  __shared__ __attribute__((aligned(16))) float spk[TT * DK];       // per-key log-decay [t][DK]
  const int blk = blockIdx.x;
  const int rb = blk % NRB;
  const int h = (blk / NRB) % p.hv;
  const int b = blk / (NRB * p.hv);
  const int tid = threadIdx.x;
  const int row = rb * ROWS + tid / L;
  const int o = tid % L;

  const int rd = p.read_idx[b];
  if (rd < 0 || rd >= p.pool_size) return;  // skipped row: touch nothing
  const int wr = p.write_idx ? p.write_idx[b] : rd;
  const int qh = (int)(((int64_t)h * p.hq) / p.hv);

  const IO* __restrict__ q = (const IO*)p.q;
  const IO* __restrict__ k = (const IO*)p.k;
  const IO* __restrict__ v = (const IO*)p.v;
  const IO* __restrict__ ga = (const IO*)p.a;
  const IO* __restrict__ gb = (const IO*)p.b;
  IO* __restrict__ out = (IO*)p.out;

  // column of element e of segment i held by this lane: i*4L + 4o + e
  const int64_t head_off = (int64_t)h * p.head_stride + (int64_t)row * DK + 4 * o;
  f4 x[4];
  {
    const float* src = p.pool + (int64_t)rd * p.slot_stride + head_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = ld_nt(src + i * 4 * L);
  }
  const bool per_key = p.decay_pk != nullptr;  // uniform: the per-key decay replaces the gate's
  const float A_log = per_key ? 0.f : p.A_log[h];
  const float dt_bias = per_key ? 0.f : p.dt_bias[h];

  // One token: decay, the sub-steps, the readout and the optional scatter.
  // kp(j): this lane's k of sub-step j; vj(j), beta(j): the row's v and beta;
  // qp: this lane's q.
  // in-kernel L2 norm of a vector spread over the row's L lanes (16 elements
  // each); an all-zero vector stays zero
  auto l2n = [&](f4* v4) {
    if (!p.qk_norm) return;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) ss += v4[i][0] * v4[i][0] + v4[i][1] * v4[i][1] + v4[i][2] * v4[i][2] + v4[i][3] * v4[i][3];
    ss = group_sum<L>(ss) + p.qk_eps;
    const float r = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] *= r;
  };
  // gp: this lane's per-key log-decays (used when per_key)
  auto token = [&](int t, float gamma, const float* gp, auto kp, auto vj, auto beta, const IO* qp) {
    const int64_t bt = (int64_t)b * p.T + t;
    if (per_key) {
      // key column i*4L + 4o + e of this lane decays by its own factor
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f4 gi = *reinterpret_cast<const f4*>(gp + i * 4 * L);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[i][e] *= __builtin_amdgcn_exp2f(gi[e] * 1.4426950408889634f);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] *= gamma;
    }
    for (int j = 0; j < p.nhh; ++j) {
      const IO* kj = kp(j);
      f4 kf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[i] = load4(kj + i * 4 * L);
      l2n(kf);
      float r = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r += x[i][0] * kf[i][0] + x[i][1] * kf[i][1] + x[i][2] * kf[i][2] + x[i][3] * kf[i][3];
      r = group_sum<L>(r);
      const float u = beta(j) * (vj(j) - r);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] += u * kf[i];
    }
    f4 qf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qf[i] = load4(qp + i * 4 * L);
    l2n(qf);
    float y = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) y += x[i][0] * qf[i][0] + x[i][1] * qf[i][1] + x[i][2] * qf[i][2] + x[i][3] * qf[i][3];
    y = group_sum<L>(y);
    if (o == 0) out[(bt * p.hv + h) * DV + row] = from_f32<IO>(p.scale * y);
    if (p.scatter_idx) {
      const int s = p.scatter_idx[bt];
      if (s >= 0 && s < p.pool_size) {
        float* dst = p.pool + (int64_t)s * p.slot_stride + head_off;
#pragma unroll
        for (int i = 0; i < 4; ++i) st_nt(dst + i * 4 * L, x[i]);
      }
    }
  };

  if (p.T == 1 && p.nhh == 1) {
    // a single step: its inputs straight from global memory, issued beside
    // the state loads (staging would only add a round trip)
    const int64_t bt = (int64_t)b;
    const float gamma = per_key ? 1.f : expf(gate_log_decay(A_log, dt_bias, to_f32(ga[bt * p.hv + h])));
    const float* gp = per_key ? p.decay_pk + (bt * p.hv + h) * DK + 4 * o : nullptr;
    token(0, gamma, gp, [&](int) { return k + (bt * p.hq + qh) * DK + 4 * o; },
          [&](int) { return to_f32(v[(bt * p.hv + h) * DV + row]); },
          [&](int) { return sigmoidf(to_f32(gb[bt * p.hv + h])); }, q + (bt * p.hq + qh) * DK + 4 * o);
  } else {
    for (int t0 = 0; t0 < p.T; t0 += TT) {
      const int nt = min(TT, p.T - t0);
      const int ntj = nt * p.nhh;
      if (t0 > 0) __syncthreads();  // the previous pass has read the staging area
      // stage k rows [t][j], q rows [t], v slices [t][j] (4-element groups)
      // and the gates of this pass
      const int64_t bt0 = (int64_t)b * p.T + t0;
      for (int idx = tid; idx < ntj * (DK / 4); idx += NT) {
        const int tj = idx / (DK / 4), c = idx % (DK / 4);
        const int t = tj / p.nhh, j = tj % p.nhh;
        reinterpret_cast<Q4*>(sk)[(t * NJ + j) * (DK / 4) + c] =
            reinterpret_cast<const Q4*>(k + ((bt0 * p.nhh + tj) * p.hq + qh) * DK)[c];
      }
      for (int idx = tid; idx < nt * (DK / 4); idx += NT) {
        const int t = idx / (DK / 4), c = idx % (DK / 4);
        reinterpret_cast<Q4*>(sq)[t * (DK / 4) + c] =
            reinterpret_cast<const Q4*>(q + ((bt0 + t) * p.hq + qh) * DK)[c];
      }
      for (int idx = tid; idx < ntj * (ROWS / 4); idx += NT) {
        const int tj = idx / (ROWS / 4), c = idx % (ROWS / 4);
        const int t = tj / p.nhh, j = tj % p.nhh;
        reinterpret_cast<Q4*>(sv)[(t * NJ + j) * (ROWS / 4) + c] =
            reinterpret_cast<const Q4*>(v + ((bt0 * p.nhh + tj) * p.hv + h) * DV + rb * ROWS)[c];
      }
      if (per_key) {
        for (int idx = tid; idx < nt * (DK / 4); idx += NT) {
          const int t = idx / (DK / 4), c = idx % (DK / 4);
          reinterpret_cast<f4*>(spk)[t * (DK / 4) + c] =
              reinterpret_cast<const f4*>(p.decay_pk + ((bt0 + t) * p.hv + h) * DK)[c];
        }
      } else {
        for (int idx = tid; idx < nt; idx += NT)
          sgam[idx] = expf(gate_log_decay(A_log, dt_bias, to_f32(ga[(bt0 + idx) * p.hv + h])));
      }
      for (int idx = tid; idx < ntj; idx += NT) {
        const int t = idx / p.nhh, j = idx % p.nhh;
        sbet[t * NJ + j] = sigmoidf(to_f32(gb[(bt0 * p.nhh + idx) * p.hv + h]));
      }
      __syncthreads();
      for (int tl = 0; tl < nt; ++tl)
        token(t0 + tl, per_key ? 1.f : sgam[tl], spk + tl * DK + 4 * o,
              [&](int j) -> const IO* { return sk + (tl * NJ + j) * DK + 4 * o; },
              [&](int j) { return to_f32(sv[(tl * NJ + j) * ROWS + (row - rb * ROWS)]); },
              [&](int j) { return sbet[tl * NJ + j]; }, sq + tl * DK + 4 * o);
    }
  }
  if (!p.scatter_idx && !p.disable && wr >= 0 && wr < p.pool_size) {
    float* dst = p.pool + (int64_t)wr * p.slot_stride + head_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) st_nt(dst + i * 4 * L, x[i]);
  }
}

template <typename IO, int DK, int DV>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  constexpr int L = DK / 16;
  constexpr int ROWS = (DV * L <= 256) ? DV : 256 / L;  // rows per workgroup
  constexpr int NRB = DV / ROWS;
  const int64_t nblk = (int64_t)p.batch * p.hv * NRB;
  hipLaunchKernelGGL((decode_kernel<IO, DK, DV, ROWS>), dim3((unsigned)nblk), dim3(ROWS * L), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename IO, int DK>
static hipError_t dispatch_dv(const DecodeParams& p, int dv, hipStream_t s) {
  switch (dv) {
    case 16: return launch_decode_t<IO, DK, 16>(p, s);
    case 32: return launch_decode_t<IO, DK, 32>(p, s);
    case 64: return launch_decode_t<IO, DK, 64>(p, s);
    case 128: return launch_decode_t<IO, DK, 128>(p, s);
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
// instead of one state pass per token.  Measured on B64 x Hv32 x 128x128 bf16:
// T = 16: 146 -> 132 us, T = 32: 256 -> 155 us, T = 64: 470 -> 181 us (the
// token loop stays ahead below 16 tokens: 74 vs 144 us at T = 4).  The chunk
// hint follows T (16, 32, 64).  Every activation must be 16-byte aligned,
// as the prefill kernels require.
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
  pa.chunk_size = a.T < 32 ? 16 : (a.T < 64 ? 32 : 64);
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
