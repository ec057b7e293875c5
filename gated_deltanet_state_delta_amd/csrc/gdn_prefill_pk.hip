// gdn_prefill_pk.hip -- chunked prefill with a per-key decay (gfx950).
//
// The decay of "com.microsoft.GatedDeltaNet" in its per-key-dimension
// spelling (Inputs: decay (..., num_heads_v, head_size_qk)), read in the
// card's recurrence (Description): exp(g_t) scales S_{t-1} elementwise over
// the key dimension,
//   S_t = D_t S_{t-1} + k_t u_t^T,   u_t = beta_t (v_t - rho (D_t S_{t-1})^T k_t),
// D_t = diag(exp(g_t)), rho = 1 when the update_rule keeps the retrieval.
//
// Chunked form over C = 16 tokens (state S0 before the chunk; per key i:
// Gam_t = prod_{r<=t} alpha_r, Gam_{t/s} = prod_{s<r<=t} alpha_r):
//   (I + A) U = X,  A_ts = rho beta_t sum_i k_ti k_si Gam_{t/s,i}   (s < t)
//                   X_t  = beta_t (v_t - rho S0^T (Gam_t o k_t))
//   Y_t = scale (S0^T (Gam_t o q_t) + sum_{s<=t} (sum_i q_ti k_si Gam_{t/s,i}) u_s)
//   S_C = diag(Gam_{C-1}) S0 + sum_s (Gam_{C-1/s} o k_s) u_s^T
// So the state pass is the scalar-decay one with decayed operands:
// Qd = Gam o Q and Kd = Gam o K in [Q; K] S0, K~ = Gam_{C-1/.} o K in the
// state update, and a per-key row scale Gam_{C-1} of S0.
//
// The Gram sums are not plain dot products (each key has its own decay), but
// Gam_{t/s,i} = Gam_{t,i} / Gam_{s,i} when no decay of key i in (s, t] is 0,
// so  sum_i k_ti k_si Gam_{t/s,i} = Kd_t . Kc_s  with Kc_s = k_s / Gam_s:
// one MFMA tile per chunk.  1 / Gam_s grows with the decay inside the chunk,
// so a key takes this form only when none of its chunk's decays is 0 and
// Gam_{C-1,i} >= 2^-96 (then every operand and product stays below 2^103).
// Any other key (an exceptional key) is left out of the tile (Kc = 0) and
// added to the sums exactly, term by term, in segment form: with n_{t,i} the
// number of zero decays of key i up to t and P_{t,i} the log2 decay summed
// since the last one, Gam_{t/s,i} = [n_t == n_s] 2^(P_t - P_s).  The same
// (P, n) give every factor above as exp2 of a difference <= 0, so no
// -inf - (-inf) is ever formed.
//
// Mapping.  One workgroup of 8 waves per (request, value head, slice of DVS
// <= 64 value columns) walks the request's chunks in order, one workgroup
// barrier per chunk; in iteration j:
//  * prep waves 4..7 prepare chunk j+2.  Prep wave w holds keys 32w .. 32w+31
//    of all 16 tokens in MFMA fragment layout (lane (x, g): token x, keys
//    32w + 8g .. +7), so the per-key scan over tokens is a DPP scan inside
//    16-lane rows.  It writes the decayed operands (Qd, Kd, K~^T, Gam_{C-1})
//    to one of three LDS buffers and its partial Gram tiles Kc Kd^T and
//    Kc Qd^T (one MFMA each: rows s, columns t), row norms and the raw values
//    of exceptional keys for the finishing step;
//  * state wave 3 finishes chunk j+1: the partial tiles summed, the
//    exceptional keys' terms added, -A and M formed, (I + A) inverted;
//  * state waves 0..3 each own one 16-column tile of the slice, keep the
//    state in MFMA accumulators and run the state pass of chunk j:
//    R = [Qd; Kd] S0, X, Y, the per-key row scale, U = (I + A)^-1 X,
//    Y += M U, S += K~^T U, the outputs.
// A chunk with exceptional keys adds one barrier, so that the next chunk's
// raw values (one LDS buffer) are written only after it has been finished.
// The same kernel runs the multi-token decode's chunked form over its state
// pool, with beta formed here as sigmoid(b) from the raw b.
// Operand precision: bf16 inputs use bf16 MFMA operands (the decayed q and k
// are rounded once to bf16); the state, accumulators, decays and the inverse
// are fp32.  fp32 inputs use fp32 MFMA.
#include "gdn_device.hpp"
#include "gdn_prefill.hpp"

namespace gdn {

// Exceptional-key bound: Gam_{C-1} below 2^-96 (log2 below -96).
constexpr float kPkLog2Floor = -96.f;

typedef float pk_f2 __attribute__((ext_vector_type(2)));

template <typename E, int DK>
struct PkSmem {
  static constexpr int C = 16;
  static constexpr int PAD = 16 / sizeof(E);  // 16-byte row skew
  static constexpr int LDK = DK + PAD;        // Qd, Kd rows
  static constexpr int LDC = C + PAD;         // K~^T, M and inverse rows
  struct Raw {       // one chunk's decayed operands (prepared two chunks ahead)
    E q[C][LDK];     // Qd
    E k[C][LDK];     // Kd
    E kt[DK][LDC];   // K~^T
    alignas(16) float lam[DK];  // Gam_{C-1} per key
    alignas(16) float bet[C];   // beta_t (0 on padded tokens)
  };
  struct Der {       // one chunk's finished Gram results (one chunk ahead)
    E m[C][LDC];     // M (scale and norms folded in), lower triangle
    E tinv[C][LDC];  // (I + A)^-1
    alignas(16) float gb[C];    // rho beta_t / |k_t|
    alignas(16) float gs[C];    // scale / |q_t|
    alignas(16) float dc[C];    // 1 / |k_t|
  };
  struct Part {      // one chunk's per-prep-wave results, for its finishing
    alignas(16) float gp[4][2][C][C];  // partial tiles [wave][KK | QK][t][s]
    alignas(16) float np[4][2][C];     // partial |q_t|^2, |k_t|^2
    uint32_t xmask[4];                 // exceptional keys: bit 8g + e of wave w's word
  };
  Raw raw[3];
  Der der[2];
  Part part[2];
  // the finishing wave's rows of A, split by column parity:
  // ad[20 r + 8 h + jj] = A[r][2 jj + h]
  alignas(16) float ad[C * 20];
  // exceptional keys' q, k, P, n of the chunk being finished (one buffer:
  // a chunk that has any is finished before the next is prepared)
  alignas(16) float xq[C][DK];
  alignas(16) float xk[C][DK];
  alignas(16) float xP[C][DK];
  alignas(16) float xn[C][DK];
  int fin_cnt;  // chunks whose -A and M rows state wave 2 has formed (normal path)
};

// DPP move inside 16-lane rows; lanes without a source lane receive `fill`.
template <int CTRL>
__device__ __forceinline__ float pk_dpp(float fill, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Eight consecutive io elements: 16 bytes of bf16 or 32 bytes of fp32, kept
// as loaded (NV 16-byte vectors) and widened to fp32 when used.
template <typename E> struct Raw8 { static constexpr int NV = sizeof(E) / 2; u32x4 v[NV]; };
template <typename E>
__device__ __forceinline__ void load8(const E* p, Raw8<E>& r) {
#pragma unroll
  for (int i = 0; i < Raw8<E>::NV; ++i) r.v[i] = reinterpret_cast<const u32x4*>(p)[i];
}
__device__ __forceinline__ float elem8(const Raw8<__bf16>& r, int e) {
  return bf16_bits_to_float((uint16_t)((e & 1) ? (r.v[0][e >> 1] >> 16) : (r.v[0][e >> 1] & 0xffffu)));
}
__device__ __forceinline__ float elem8(const Raw8<float>& r, int e) { return __uint_as_float(r.v[e >> 2][e & 3]); }

// Eight fp32 values -> io elements, stored as one row piece (16 or 32 bytes).
__device__ __forceinline__ void store8(__bf16* p, const float* v) {
  bf8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (__bf16)v[e];
  *reinterpret_cast<bf8*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<f4*>(p) = f4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f4*>(p + 4) = f4{v[4], v[5], v[6], v[7]};
}

// acc += A B^T over this lane's 8 contraction values (32 per wave), row x of
// A and of B held by the lanes with that x; operands rounded to the io type.
__device__ __forceinline__ f4 mma_k32v(f4 acc, const float* a, const float* b, __bf16) {
  bf8 av, bv;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    av[e] = (__bf16)a[e];
    bv[e] = (__bf16)b[e];
  }
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ f4 mma_k32v(f4 acc, const float* a, const float* b, float) {
  return mma_k32(acc, f4{a[0], a[1], a[2], a[3]}, f4{a[4], a[5], a[6], a[7]}, f4{b[0], b[1], b[2], b[3]},
                 f4{b[4], b[5], b[6], b[7]});
}

// (I + A)^-1 of a unit-lower 16x16 block (A strictly lower, in `ad` as laid
// out above), right-looking: the lane pair (2r, 2r+1) owns row r, lane parity
// h keeps T[r][j] for j = h mod 2, and T[r][j] = [j == r] - sum_{k > j}
// T[r][k] A[k][j].  Once T[r][k] is final (its owner passes it to the
// partner) it updates every j < k; A is strictly lower, so updates of entries
// j >= k add zero.  Lanes 32..63 repeat lanes 0..31 and store nothing.
template <typename E, int LDC>
__device__ __forceinline__ void pk_tri_inverse(const float* ad, E (*tout)[LDC], int lane) {
  const int r = (lane >> 1) & 15, h = lane & 1;
  const float* arow = ad + 8 * h;
  float acc[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = 2 * jj + h == r ? 1.f : 0.f;
  // row k of A: entries 2 jj + h for jj < (k + 1) / 2 can be nonzero
  f4 a[16][2];
#pragma unroll
  for (int k = 1; k < 16; ++k) {
    a[k][0] = *reinterpret_cast<const f4*>(arow + 20 * k);
    if (k > 8) a[k][1] = *reinterpret_cast<const f4*>(arow + 20 * k + 4);
  }
#pragma unroll
  for (int k = 15; k >= 1; --k) {
    const float mine = acc[k >> 1];
    const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mine), 0xB1, 0xF, 0xF, false));
    const float tk = (k & 1) == h ? mine : other;
    auto ak = [&](int jj) -> float { return jj < 4 ? a[k][0][jj] : a[k][1][jj - 4]; };
    acc[(k - 1) >> 1] -= tk * ak((k - 1) >> 1);  // the entry the next step reads first
#pragma unroll
    for (int jj = 0; jj < ((k - 1) >> 1); ++jj) acc[jj] -= tk * ak(jj);
  }
  // row r, columns 8h .. 8h+7: even columns from parity 0, odd from parity 1
  float o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = acc[q], hi = acc[4 + q];
    const float sw_lo = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(lo), 0xB1, 0xF, 0xF, false));
    const float sw_hi = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(hi), 0xB1, 0xF, 0xF, false));
    o[2 * q] = h == 0 ? lo : sw_hi;
    o[2 * q + 1] = h == 0 ? sw_lo : hi;
  }
  if (lane < 32) {
    *reinterpret_cast<typename pack4<E>::type*>(&tout[r][8 * h]) = to_pack4<E>(f4{o[0], o[1], o[2], o[3]});
    *reinterpret_cast<typename pack4<E>::type*>(&tout[r][8 * h + 4]) = to_pack4<E>(f4{o[4], o[5], o[6], o[7]});
  }
}

// FB: beta fused as sigmoid(b) from the raw b (p.gb), else given (p.beta).
template <typename E, int DK, int DVS, bool FB>
__global__ void __launch_bounds__(512)
prefill_pk_kernel(const PrefillParams p) {
  typedef typename frag_of<E>::type Fr;
  typedef PkSmem<E, DK> Sm;
  constexpr int C = 16;
  constexpr int NKT = DK / 16;        // key tiles of the state
  constexpr int NVT = DVS / 16;       // value tiles (state waves) per workgroup
  constexpr int NW = (DK + 31) / 32;  // prep waves holding keys
  static_assert(NVT >= 1 && NVT <= 4, "one value tile per state wave");
  __shared__ Sm sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int x = lane & 15;
  const int g = lane >> 4;

  const int blk = prefill_block_unit(blockIdx.x, gridDim.x, p.nsplit * max(p.hv / p.hq, 1), p.lpt);
  const int split = blk % p.nsplit;
  const int h = (blk / p.nsplit) % p.hv;
  const int r = prefill_request_of_rank(p, blk / (p.nsplit * p.hv), reinterpret_cast<int*>(&sm.xq[0][0]));
  const int qh = (int)(((int64_t)h * p.hq) / p.hv);
  const int v0 = split * DVS;

  int64_t start, end;
  if (p.cu) {
    start = min(max((int64_t)p.cu[r], (int64_t)0), p.T);
    end = min(max((int64_t)p.cu[r + 1], (int64_t)0), p.T);
  } else {
    start = (int64_t)r * p.seq_len;
    end = start + p.seq_len;
  }
  if (end < start) end = start;
  const int nch = (int)((end - start + C - 1) / C);
  int64_t ibase, fbase;
  prefill_state_offsets(p, r, h, v0, DK, ibase, fbase);
  if ((p.pool_flags & kPoolSkipUnread) && ibase < 0) return;  // uniform over the workgroup

  const E* __restrict__ gq = (const E*)p.q + (int64_t)qh * p.q_sh;
  const E* __restrict__ gk = (const E*)p.k + (int64_t)qh * p.k_sh;
  const E* __restrict__ gv = (const E*)p.v + (int64_t)h * p.v_sh + v0;
  E* __restrict__ gout = (E*)p.out + (int64_t)h * p.o_sh + v0;
  const float* __restrict__ gdec = p.decay + (int64_t)h * DK;  // [T, hv, DK]
  // beta given, or fused as sigmoid(b) from the raw b (the multi-token
  // decode's gate, which runs this kernel over its state pool)
  const float* __restrict__ gbet = FB ? nullptr : p.beta + (h & p.bmask);
  const E* __restrict__ ggb = FB ? (const E*)p.gb + (h & p.bmask) : nullptr;
  const bool nrm = p.qk_norm != 0;

  // Whether chunk jc holds exceptional keys (read after the barrier that
  // follows its preparation; the same in every wave).
  auto has_exc = [&](int jc) -> bool {
    if (jc < 0 || jc >= nch) return false;
    uint32_t any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= sm.part[jc & 1].xmask[w];
    return any != 0;
  };

  if (tid == 0) sm.fin_cnt = 0;  // first read after the loops' first barrier

  // ------------------------------------------------------------ state waves
  // Iteration j: the state pass of chunk j (state waves below NVT) and the
  // finishing of chunk j+1 in two parts: state wave 2 sums its partial
  // tiles, adds the exceptional keys' terms and forms -A and M before its
  // state pass; state wave 3 inverts (I + A) after its own (an LDS counter
  // says when the rows are there), so neither wave carries a state pass and
  // a whole finishing.  A chunk with exceptional keys is finished whole by
  // wave 3 before the state pass (see below).
  if (wave < 4) {
    const bool active = wave < NVT;  // waves beyond the slice only finish and keep the barriers
    const int vc = 16 * wave + x;    // value column inside the slice
    const int vst = (int)p.v_st, ost = (int)p.o_st;
    const int v_lane = 4 * g * vst + x, o_lane = 4 * g * ost + x;
    f4 S[NKT];
    E vreg[4];
#pragma unroll
    for (int j = 0; j < NKT; ++j) S[j] = f4{0.f, 0.f, 0.f, 0.f};
    // V(c) in accumulator layout: rows t = 4g + e, column vc
    auto load_v = [&](int c) {
      const int64_t t0 = start + (int64_t)c * C;
      const int rem = (int)min((int64_t)C, end - t0);  // >= 1
      const E* vb = gv + t0 * p.v_st + 16 * wave;
      if (rem == C) {
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(vb);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vreg[e] = buf_load<E>(rs, v_lane * (uint32_t)sizeof(E), e * vst * (uint32_t)sizeof(E));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g + e;
          const E v = vb[min(t, rem - 1) * vst + x];  // clamped: inside the request
          vreg[e] = t < rem ? v : from_f32<E>(0.f);
        }
      }
    };
    // The state pass of chunk c.
    auto state_pass = [&](int c) {
      const typename Sm::Raw& R = sm.raw[c % 3];
      const typename Sm::Der& Dd = sm.der[c & 1];
      // R = [Qd; Kd] S0; X = beta V - rho beta R_K / |k|; Y = scale R_Q / |q|
      Fr Sb[NKT];
#pragma unroll
      for (int j = 0; j < NKT; ++j) cvt_frag(S[j], Sb[j]);
      f4 rq = f4{0.f, 0.f, 0.f, 0.f}, rk = rq;
      if constexpr (NKT % 2 == 0) {
#pragma unroll
        for (int pp = 0; pp < NKT / 2; ++pp) {
          Fr aq0, aq1, ak0, ak1;
          lds_frag8(&R.q[x][32 * pp + 8 * g], aq0, aq1);
          lds_frag8(&R.k[x][32 * pp + 8 * g], ak0, ak1);
          rq = mma_k32(rq, aq0, aq1, Sb[2 * pp], Sb[2 * pp + 1]);
          rk = mma_k32(rk, ak0, ak1, Sb[2 * pp], Sb[2 * pp + 1]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NKT; ++j) {
          Fr aq, ak;
          lds_frag(&R.q[x][16 * j + 4 * g], aq);
          lds_frag(&R.k[x][16 * j + 4 * g], ak);
          rq = mma_k16(rq, aq, Sb[j]);
          rk = mma_k16(rk, ak, Sb[j]);
        }
      }
      const f4 bt = *reinterpret_cast<const f4*>(&R.bet[4 * g]);
      const f4 gb = *reinterpret_cast<const f4*>(&Dd.gb[4 * g]);
      const f4 gs = *reinterpret_cast<const f4*>(&Dd.gs[4 * g]);
      f4 X, Y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        X[e] = bt[e] * to_f32(vreg[e]) - gb[e] * rk[e];
        Y[e] = gs[e] * rq[e];
      }
      if (c + 1 < nch) load_v(c + 1);
      // S <- Gam_{C-1} S; U = (I + A)^-1 X; Y += M U; S += K~^T U / |k|
#pragma unroll
      for (int j = 0; j < NKT; ++j) S[j] = S[j] * *reinterpret_cast<const f4*>(&R.lam[dk_of<NKT>(j, 4 * g)]);
      Fr Pb, ti, Ub, DU, a;
      cvt_frag(X, Pb);
      lds_frag(&Dd.tinv[x][4 * g], ti);
      const f4 U = mma_k16(f4{0.f, 0.f, 0.f, 0.f}, ti, Pb);
      cvt_frag(U, Ub);
      cvt_frag(*reinterpret_cast<const f4*>(&Dd.dc[4 * g]) * U, DU);
      lds_frag(&Dd.m[x][4 * g], a);
      Y = mma_k16(Y, a, Ub);
#pragma unroll
      for (int j = 0; j < NKT; ++j) {
        lds_frag(&R.kt[dk_of<NKT>(j, x)][4 * g], a);
        S[j] = mma_k16(S[j], a, DU);
      }
      const int64_t tok0 = start + (int64_t)c * C;
      const int nvalid = (int)min((int64_t)C, end - tok0);
      E* ob = gout + tok0 * p.o_st + 16 * wave;
      if (nvalid == C) {
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(ob);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buf_store(rs, o_lane * (uint32_t)sizeof(E), e * ost * (uint32_t)sizeof(E), from_f32<E>(Y[e]));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * g + e < nvalid) ob[(4 * g + e) * ost + x] = from_f32<E>(Y[e]);
      }
    };
    // Finishing of chunk c, first part (all 64 lanes of one wave): -A and M.
    auto finish_rows = [&](int c) {
      const typename Sm::Part& Pa = sm.part[c & 1];
      const typename Sm::Raw& R = sm.raw[c % 3];
      typename Sm::Der& Dd = sm.der[c & 1];
      const int t = x;
      f4 kk = *reinterpret_cast<const f4*>(&Pa.gp[0][0][t][4 * g]);
      f4 qk = *reinterpret_cast<const f4*>(&Pa.gp[0][1][t][4 * g]);
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        kk += *reinterpret_cast<const f4*>(&Pa.gp[w][0][t][4 * g]);
        qk += *reinterpret_cast<const f4*>(&Pa.gp[w][1][t][4 * g]);
      }
      // exceptional keys, term by term (s <= t only)
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        uint32_t mk = Pa.xmask[w];  // uniform over the wave
        while (mk) {
          const int b = __builtin_ctz(mk);
          mk &= mk - 1;
          const int i = 32 * w + b;
          const float kti = sm.xk[t][i], qti = sm.xq[t][i], Pt = sm.xP[t][i], nt = sm.xn[t][i];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = 4 * g + e;
            if (s <= t && sm.xn[s][i] == nt) {
              const float ks = sm.xk[s][i] * __builtin_amdgcn_exp2f(Pt - sm.xP[s][i]);
              kk[e] += kti * ks;
              qk[e] += qti * ks;
            }
          }
        }
      }
      float rqt = 1.f, rkt = 1.f;
      f4 rks = f4{1.f, 1.f, 1.f, 1.f};
      if (nrm) {
        // an all-zero row (a padded token, or eps 0) keeps the factor 0
        auto inv_norm = [&](int which, int tt) {
          float s2 = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) s2 += Pa.np[w][which][tt];
          s2 += p.qk_eps;
          return s2 > 0.f ? 1.f / sqrtf(s2) : 0.f;
        };
        rqt = inv_norm(0, t);
        rkt = inv_norm(1, t);
#pragma unroll
        for (int e = 0; e < 4; ++e) rks[e] = inv_norm(1, 4 * g + e);
      }
      const float bt = R.bet[t];
      f4 arow, mrow;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 4 * g + e;
        arow[e] = s < t ? p.rho * bt * rkt * rks[e] * kk[e] : 0.f;
        mrow[e] = s <= t ? p.scale * rqt * rks[e] * qk[e] : 0.f;
      }
      // columns 4g, 4g+2 (parity 0) and 4g+1, 4g+3 (parity 1) of row t
      *reinterpret_cast<pk_f2*>(&sm.ad[20 * t + 2 * g]) = pk_f2{arow[0], arow[2]};
      *reinterpret_cast<pk_f2*>(&sm.ad[20 * t + 8 + 2 * g]) = pk_f2{arow[1], arow[3]};
      *reinterpret_cast<typename pack4<E>::type*>(&Dd.m[t][4 * g]) = to_pack4<E>(mrow);
      if (g == 0) {
        Dd.gb[t] = p.rho * bt * rkt;
        Dd.gs[t] = p.scale * rqt;
        Dd.dc[t] = rkt;
      }
    };
    // Second part: (I + A)^-1 from the rows the first part left in sm.ad.
    auto finish_inverse = [&](int c) { pk_tri_inverse<E, Sm::LDC>(sm.ad, sm.der[c & 1].tinv, lane); };

    if (active) {
      if (ibase >= 0) {
#pragma unroll
        for (int j = 0; j < NKT; ++j)
          S[j] = *reinterpret_cast<const f4*>(p.init + ibase + (int64_t)vc * DK + dk_of<NKT>(j, 4 * g));
      }
      if (nch > 0) load_v(0);
    }
    int nsplit_fin = 0;  // chunks finished in two parts so far (the same in every wave)
    for (int j = -2; j < nch; ++j) {
      const bool fj = j + 1 >= 0 && j + 1 < nch;  // a chunk to finish
      if (has_exc(j + 1)) {
        // the prep waves overwrite the exceptional keys' values only after
        // chunk j+1 has been finished
        if (fj && wave == 3) {
          finish_rows(j + 1);
          finish_inverse(j + 1);
        }
        lds_barrier();
        if (active && j >= 0) state_pass(j);
      } else {
        if (fj) ++nsplit_fin;
        if (fj && wave == 2) {
          finish_rows(j + 1);
          if (lane == 0) __hip_atomic_fetch_add(&sm.fin_cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (active && j >= 0) state_pass(j);
        if (fj && wave == 3) {
          wait_lds_count(&sm.fin_cnt, nsplit_fin, p.wait_err);
          finish_inverse(j + 1);
        }
      }
      lds_barrier();
    }
    if (active && fbase >= 0) {
#pragma unroll
      for (int j = 0; j < NKT; ++j)
        *reinterpret_cast<f4*>(p.fin + fbase + (int64_t)vc * DK + dk_of<NKT>(j, 4 * g)) = S[j];
    }
    return;
  }

  // ------------------------------------------------------------- prep waves
  // Iteration j prepares chunk j+2.
  const int pw = wave - 4;
  const int kb = 32 * pw + 8 * g;  // first of this lane's 8 keys
  const bool keys = kb < DK;       // lanes past the head size hold zeros
  // the next chunk exactly as loaded: nothing here may wait on these loads
  // (they are converted when the chunk is prepared, an iteration later)
  Raw8<E> pq, pk;
  Raw8<float> pd;
  float pbt = 0.f;
  E pbr = from_f32<E>(0.f);
#pragma unroll
  for (int i = 0; i < Raw8<E>::NV; ++i) pq.v[i] = pk.v[i] = u32x4{0u, 0u, 0u, 0u};
  pd.v[0] = pd.v[1] = u32x4{0u, 0u, 0u, 0u};
  int prem = 0;
  auto prefetch = [&](int c) {
    const int64_t t0 = start + (int64_t)c * C;
    prem = (int)min((int64_t)C, end - t0);      // >= 1
    const int64_t tok = t0 + min(x, prem - 1);  // clamped: inside the request
    // beta first: a wait the compiler places for its register must not also
    // wait for the row loads (the wait counter is in order)
    if (pw == 0) {
      if constexpr (FB) pbr = ggb[(tok * p.hv) & p.bmask];
      else pbt = gbet[(tok * p.hv) & p.bmask];
    }
    // lanes past the head size read the last keys (in bounds) and are masked
    // when used, so the loads take no branch
    const int kl = min(kb, DK - 8);
    load8(gq + tok * p.q_st + kl, pq);
    load8(gk + tok * p.k_st + kl, pk);
    load8(gdec + tok * (int64_t)p.hv * DK + kl, pd);
  };
  // Preparation of chunk c from the prefetched registers.
  auto prepare = [&](int c) {
    typename Sm::Raw& R = sm.raw[c % 3];
    typename Sm::Part& Pa = sm.part[c & 1];
    const bool live = x < prem && keys;
    if (pw == 0 && g == 0) R.bet[x] = x < prem ? (FB ? sigmoid_fast(to_f32(pbr)) : pbt) : 0.f;
    float P[8], n[8], qf[8], kf[8];
    if (p.decay_is_gamma) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = elem8(pd, e);
        const bool zero = !(d > 0.f);
        P[e] = live && !zero ? __log2f(d) : 0.f;  // padded tokens: no decay
        n[e] = live && zero ? 1.f : 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = elem8(pd, e);
        const bool zero = !(d > -INFINITY);
        P[e] = live && !zero ? d * 1.4426950408889634f : 0.f;
        n[e] = live && zero ? 1.f : 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qf[e] = live ? elem8(pq, e) : 0.f;
      kf[e] = live ? elem8(pk, e) : 0.f;
    }
    if (c + 1 < nch) prefetch(c + 1);
    // inclusive scan over the 16 tokens (the lanes x of a row).  With a zero
    // decay in the wave it is segmented: (P, n) of an earlier span and
    // (P', n') of the later one combine to (n' > 0 ? P' : P + P', n + n').
    bool lz = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) lz = lz || n[e] > 0.f;
    if (__builtin_amdgcn_ballot_w64(lz) != 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pv = P[e], nv = n[e], pl, nl;
        pl = pk_dpp<0x111>(0.f, pv);  // row_shr:1
        nl = pk_dpp<0x111>(0.f, nv);
        pv = nv > 0.f ? pv : pv + pl;
        nv += nl;
        pl = pk_dpp<0x112>(0.f, pv);  // row_shr:2
        nl = pk_dpp<0x112>(0.f, nv);
        pv = nv > 0.f ? pv : pv + pl;
        nv += nl;
        pl = pk_dpp<0x114>(0.f, pv);  // row_shr:4
        nl = pk_dpp<0x114>(0.f, nv);
        pv = nv > 0.f ? pv : pv + pl;
        nv += nl;
        pl = pk_dpp<0x118>(0.f, pv);  // row_shr:8
        nl = pk_dpp<0x118>(0.f, nv);
        pv = nv > 0.f ? pv : pv + pl;
        nv += nl;
        P[e] = pv;
        n[e] = nv;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pv = P[e];
        pv += pk_dpp<0x111>(0.f, pv);
        pv += pk_dpp<0x112>(0.f, pv);
        pv += pk_dpp<0x114>(0.f, pv);
        pv += pk_dpp<0x118>(0.f, pv);
        P[e] = pv;
      }
    }
    // factors (token 15's values broadcast along the row, row_newbcast)
    float qd[8], kd[8], kt[8], kc[8], PL[8], nL[8];
    bool exc_l = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      PL[e] = pk_dpp<0x15F>(0.f, P[e]);
      nL[e] = pk_dpp<0x15F>(0.f, n[e]);
      const float gam = n[e] == 0.f ? __builtin_amdgcn_exp2f(P[e]) : 0.f;  // Gam_t
      qd[e] = qf[e] * gam;
      kd[e] = kf[e] * gam;
      if (keys && x == C - 1) R.lam[kb + e] = gam;  // Gam_{C-1}
      kt[e] = gam;
      exc_l = exc_l || nL[e] > 0.f || PL[e] < kPkLog2Floor;  // the same for all tokens
    }
    uint32_t xbits = 0;
    if (__builtin_amdgcn_ballot_w64(exc_l) == 0) {
      // no exceptional key: Gam_{C-1/t} = Gam_{C-1} / Gam_t
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float inv = __builtin_amdgcn_exp2f(-P[e]);  // 1 / Gam_t
        kc[e] = kf[e] * inv;
        kt[e] = kf[e] * (pk_dpp<0x15F>(0.f, kt[e]) * inv);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool exc = nL[e] > 0.f || PL[e] < kPkLog2Floor;
        const float gct = n[e] == nL[e] ? __builtin_amdgcn_exp2f(PL[e] - P[e]) : 0.f;  // Gam_{C-1/t}
        kc[e] = exc ? 0.f : kf[e] * __builtin_amdgcn_exp2f(-P[e]);
        kt[e] = kf[e] * gct;
        if (exc) {
          xbits |= 1u << e;
          sm.xq[x][kb + e] = qf[e];
          sm.xk[x][kb + e] = kf[e];
          sm.xP[x][kb + e] = P[e];
          sm.xn[x][kb + e] = n[e];
        }
      }
    }
    if (keys) {
      store8(&R.q[x][kb], qd);
      store8(&R.k[x][kb], kd);
#pragma unroll
      for (int e = 0; e < 8; ++e) R.kt[kb + e][x] = from_f32<E>(kt[e]);
    }
    // exceptional keys of this wave: byte g of the word (the same in every
    // lane of a row)
    const uint32_t word = (uint32_t)__builtin_amdgcn_readlane((int)xbits, 0) |
                          ((uint32_t)__builtin_amdgcn_readlane((int)xbits, 16) << 8) |
                          ((uint32_t)__builtin_amdgcn_readlane((int)xbits, 32) << 16) |
                          ((uint32_t)__builtin_amdgcn_readlane((int)xbits, 48) << 24);
    if (lane == 0) Pa.xmask[pw] = word;
    // partial Gram tiles: lane (x, g) gets rows s = 4g .. 4g+3 of column t = x
    const f4 zero4 = f4{0.f, 0.f, 0.f, 0.f};
    const f4 kk = mma_k32v(zero4, kc, kd, E{});
    const f4 qk = mma_k32v(zero4, kc, qd, E{});
    *reinterpret_cast<f4*>(&Pa.gp[pw][0][x][4 * g]) = kk;
    *reinterpret_cast<f4*>(&Pa.gp[pw][1][x][4 * g]) = qk;
    if (nrm) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq += qf[e] * qf[e];
        sk += kf[e] * kf[e];
      }
      sq += __shfl_xor(sq, 16);
      sk += __shfl_xor(sk, 16);
      sq += __shfl_xor(sq, 32);
      sk += __shfl_xor(sk, 32);
      if (g == 0) {
        Pa.np[pw][0][x] = sq;
        Pa.np[pw][1][x] = sk;
      }
    }
  };

  if (nch > 0 && pw < NW) prefetch(0);
  for (int j = -2; j < nch; ++j) {
    if (has_exc(j + 1)) lds_barrier();  // see the state waves' loop
    if (j + 2 < nch && pw < NW) prepare(j + 2);
    lds_barrier();
  }
}

template <typename E, int DK, int DVS>
static hipError_t launch_pk_t(PrefillParams p, hipStream_t stream) {
  p.nsplit = p.dv / DVS;
  const int64_t nblk = (int64_t)p.n_seqs * p.hv * p.nsplit;
  if (p.gb) hipLaunchKernelGGL((prefill_pk_kernel<E, DK, DVS, true>), dim3((unsigned)nblk), dim3(512), 0, stream, p);
  else hipLaunchKernelGGL((prefill_pk_kernel<E, DK, DVS, false>), dim3((unsigned)nblk), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <typename E, int DK>
static hipError_t launch_pk_dv(const PrefillParams& p, int dv, hipStream_t s) {
  switch (dv) {
    case 16: return launch_pk_t<E, DK, 16>(p, s);
    case 32: return launch_pk_t<E, DK, 32>(p, s);
    case 64: case 128: return launch_pk_t<E, DK, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename E>
static hipError_t launch_pk_dk(const PrefillParams& p, int dk, int dv, hipStream_t s) {
  switch (dk) {
    case 16: return launch_pk_dv<E, 16>(p, dv, s);
    case 32: return launch_pk_dv<E, 32>(p, dv, s);
    case 64: return launch_pk_dv<E, 64>(p, dv, s);
    case 128: return launch_pk_dv<E, 128>(p, dv, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_pk(const PrefillParams& p, int dk, int dv, bool bf16, hipStream_t s) {
  return bf16 ? launch_pk_dk<__bf16>(p, dk, dv, s) : launch_pk_dk<float>(p, dk, dv, s);
}

}  // namespace gdn
