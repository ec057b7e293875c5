// gdn_decode.hpp -- streaming decode / multi-token verification over a slot pool.
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
#pragma once

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
  __shared__ int ssc[TT];  // scatter slots of the pass's tokens
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
  // kp(j, kf): this lane's k of sub-step j into kf[4]; vj(j), beta(j): the
  // row's v and beta; qp(qf): this lane's q into qf[4].
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
  // gp: this lane's per-key log-decays (used when per_key); scatter_slot(t):
  // token t's scatter slot (read before the token loop: a load inside it
  // would wait for the previous tokens' stores)
  auto token = [&](int t, float gamma, const float* gp, auto kp, auto vj, auto beta, auto qp,
                   auto scatter_slot) {
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
      f4 kf[4];
      kp(j, kf);
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
    qp(qf);
    l2n(qf);
    float y = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) y += x[i][0] * qf[i][0] + x[i][1] * qf[i][1] + x[i][2] * qf[i][2] + x[i][3] * qf[i][3];
    y = group_sum<L>(y);
    if (o == 0) out[(bt * p.hv + h) * DV + row] = from_f32<IO>(p.scale * y);
    if (p.scatter_idx) {
      const int s = scatter_slot(t);
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
    const int sc0 = p.scatter_idx ? p.scatter_idx[bt] : -1;
    const IO* kq = k + (bt * p.hq + qh) * DK + 4 * o;
    const IO* qq = q + (bt * p.hq + qh) * DK + 4 * o;
    token(0, gamma, gp,
          [&](int, f4* kf) {
#pragma unroll
            for (int i = 0; i < 4; ++i) kf[i] = load4(kq + i * 4 * L);
          },
          [&](int) { return to_f32(v[(bt * p.hv + h) * DV + row]); },
          [&](int) { return sigmoidf(to_f32(gb[bt * p.hv + h])); },
          [&](f4* qf) {
#pragma unroll
            for (int i = 0; i < 4; ++i) qf[i] = load4(qq + i * 4 * L);
          },
          [&](int) { return sc0; });
  } else {
    for (int t0 = 0; t0 < p.T; t0 += TT) {
      const int nt = min(TT, p.T - t0);
      const int ntj = nt * p.nhh;
      // stage k rows [t][j], q rows [t], v slices [t][j] (4-element groups),
      // the gates and the scatter slots of this pass: every thread issues
      // all of its loads before it writes any of them to LDS, so the pass
      // waits for its loads once (a load-then-store loop waits per element)
      constexpr int MK = (TT * NJ * (DK / 4) + NT - 1) / NT;
      constexpr int MQ = (TT * (DK / 4) + NT - 1) / NT;
      constexpr int MV = (TT * NJ * (ROWS / 4) + NT - 1) / NT;
      constexpr int MP = (TT * (DK / 4) + NT - 1) / NT;
      const int64_t bt0 = (int64_t)b * p.T + t0;
      // the loads run unconditionally (indices clamped into the pass, values
      // past it are not stored): guarded loads compile to branches whose
      // register reuse makes every load wait for the previous one
      Q4 rk[MK], rq[MQ], rv[MV];
      f4 rp[MP];
      // uniform bases of the pass; lane offsets stay 32-bit (a pass spans at
      // most TT tokens of one batch row)
      const Q4* kb = reinterpret_cast<const Q4*>(k + (bt0 * p.nhh * p.hq + qh) * DK);
      const Q4* qb = reinterpret_cast<const Q4*>(q + (bt0 * p.hq + qh) * DK);
      const Q4* vb = reinterpret_cast<const Q4*>(v + (bt0 * p.nhh * p.hv + h) * DV + rb * ROWS);
      const int ks = p.hq * (DK / 4), vs = p.hv * (DV / 4);  // token(-step) strides in Q4
#pragma unroll
      for (int u = 0; u < MK; ++u) {
        const int idx = min(tid + u * NT, ntj * (DK / 4) - 1), tj = idx / (DK / 4), c = idx % (DK / 4);
        rk[u] = kb[tj * ks + c];
      }
#pragma unroll
      for (int u = 0; u < MQ; ++u) {
        const int idx = min(tid + u * NT, nt * (DK / 4) - 1), t = idx / (DK / 4), c = idx % (DK / 4);
        rq[u] = qb[t * ks + c];
      }
#pragma unroll
      for (int u = 0; u < MV; ++u) {
        const int idx = min(tid + u * NT, ntj * (ROWS / 4) - 1), tj = idx / (ROWS / 4), c = idx % (ROWS / 4);
        rv[u] = vb[tj * vs + c];
      }
      if (per_key) {
        const f4* pb = reinterpret_cast<const f4*>(p.decay_pk + (bt0 * p.hv + h) * DK);
#pragma unroll
        for (int u = 0; u < MP; ++u) {
          const int idx = min(tid + u * NT, nt * (DK / 4) - 1), t = idx / (DK / 4), c = idx % (DK / 4);
          rp[u] = pb[t * (p.hv * (DK / 4)) + c];
        }
      }
      // one thread per token (gate, scatter slot) and per (token, sub-step) (beta)
      // (with a per-key decay the raw gate a is absent: b, which holds at
      // least as many entries, stands in and its value is not used)
      const IO raw_a = (per_key ? gb : ga)[(bt0 + min(tid, nt - 1)) * p.hv + h];
      const float rbv = to_f32(gb[(bt0 * p.nhh + min(tid, ntj - 1)) * p.hv + h]);
      const int rsc = p.scatter_idx ? p.scatter_idx[bt0 + min(tid, nt - 1)] : -1;
      if (t0 > 0) __syncthreads();  // the previous pass has read the staging area
#pragma unroll
      for (int u = 0; u < MK; ++u) {
        const int idx = tid + u * NT, tj = idx / (DK / 4), c = idx % (DK / 4);
        const int t = tj / p.nhh, j = tj % p.nhh;
        if (idx < ntj * (DK / 4)) reinterpret_cast<Q4*>(sk)[(t * NJ + j) * (DK / 4) + c] = rk[u];
      }
#pragma unroll
      for (int u = 0; u < MQ; ++u) {
        const int idx = tid + u * NT, t = idx / (DK / 4), c = idx % (DK / 4);
        if (idx < nt * (DK / 4)) reinterpret_cast<Q4*>(sq)[t * (DK / 4) + c] = rq[u];
      }
#pragma unroll
      for (int u = 0; u < MV; ++u) {
        const int idx = tid + u * NT, tj = idx / (ROWS / 4), c = idx % (ROWS / 4);
        const int t = tj / p.nhh, j = tj % p.nhh;
        if (idx < ntj * (ROWS / 4)) reinterpret_cast<Q4*>(sv)[(t * NJ + j) * (ROWS / 4) + c] = rv[u];
      }
      if (per_key) {
#pragma unroll
        for (int u = 0; u < MP; ++u) {
          const int idx = tid + u * NT, t = idx / (DK / 4), c = idx % (DK / 4);
          if (idx < nt * (DK / 4)) reinterpret_cast<f4*>(spk)[t * (DK / 4) + c] = rp[u];
        }
      } else if (tid < nt) {
        sgam[tid] = expf(gate_log_decay(A_log, dt_bias, to_f32(raw_a)));
      }
      if (tid < ntj) sbet[(tid / p.nhh) * NJ + tid % p.nhh] = sigmoidf(rbv);
      if (tid < nt) ssc[tid] = rsc;
      __syncthreads();
      for (int tl = 0; tl < nt; ++tl)
        token(t0 + tl, per_key ? 1.f : sgam[tl], spk + tl * DK + 4 * o,
              [&](int j, f4* kf) {
                const IO* kj = sk + (tl * NJ + j) * DK + 4 * o;
#pragma unroll
                for (int i = 0; i < 4; ++i) kf[i] = load4(kj + i * 4 * L);
              },
              [&](int j) { return to_f32(sv[(tl * NJ + j) * ROWS + (row - rb * ROWS)]); },
              [&](int j) { return sbet[tl * NJ + j]; },
              [&](f4* qf) {
                const IO* qj = sq + tl * DK + 4 * o;
#pragma unroll
                for (int i = 0; i < 4; ++i) qf[i] = load4(qj + i * 4 * L);
              },
              [&](int) { return ssc[tl]; });
    }
  }
  if (!p.scatter_idx && !p.disable && wr >= 0 && wr < p.pool_size) {
    float* dst = p.pool + (int64_t)wr * p.slot_stride + head_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) st_nt(dst + i * 4 * L, x[i]);
  }
}

template <typename IO, int DK, int DV>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  constexpr int L = DK / 16;
  constexpr int ROWS = (DV * L <= 256) ? DV : 256 / L;  // rows per workgroup
  constexpr int NRB = DV / ROWS;
  const int64_t nblk = (int64_t)p.batch * p.hv * NRB;
  hipLaunchKernelGGL((decode_kernel<IO, DK, DV, ROWS>), dim3((unsigned)nblk), dim3(ROWS * L), 0,
                     stream, p);
  return hipGetLastError();
}

// The value-width-128 launches, built in gdn_decode_dv128.hip with their own
// scheduler flags (see the build script).
hipError_t launch_decode_dv128(const DecodeParams& p, int dk, bool bf16, hipStream_t stream);

}  // namespace gdn
