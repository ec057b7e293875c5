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
// <= 64 value columns), walking the request's chunks in order with two
// workgroup barriers per chunk:
//  * state waves 0..3 each own one 16-column tile of the slice and keep the
//    state in MFMA accumulators.  Part 1: R = [Qd; Kd] S0, X, Y.  Part 2: the
//    per-key row scale, U = (I + A)^-1 X, Y += M U, S += K~^T U, the outputs;
//  * prep waves 4..7 prepare the next chunk.  Prep wave w holds keys
//    32w .. 32w+31 of all 16 tokens in MFMA fragment layout (lane (x, g):
//    token x, keys 32w + 8g .. +7), so the per-key scan over tokens is a DPP
//    scan inside 16-lane rows.  Part 1: the scan, the decayed operands (Qd,
//    Kd and K~^T to LDS), the wave's partial Gram tiles Kc Kd^T and Kc Qd^T
//    (one MFMA each: rows s, columns t), the raw values of exceptional keys
//    and partial row norms.  Part 2 (prep wave 4): the partial tiles summed,
//    the exceptional keys' terms added, -A and M formed, (I + A) inverted.
// Operand precision: bf16 inputs use bf16 MFMA operands (the decayed q and k
// are rounded once to bf16); the state, accumulators, decays and the inverse
// are fp32.  fp32 inputs use fp32 MFMA.
#include "gdn_device.hpp"
#include "gdn_prefill.hpp"

namespace gdn {

// Exceptional-key bound: Gam_{C-1} below 2^-96 (log2 below -96).
constexpr float kPkLog2Floor = -96.f;

template <typename E, int DK>
struct PkSmem {
  static constexpr int C = 16;
  static constexpr int PAD = 16 / sizeof(E);  // 16-byte row skew
  static constexpr int LDK = DK + PAD;        // Qd, Kd rows
  static constexpr int LDC = C + PAD;         // K~^T, M and inverse rows
  struct Raw {       // one chunk's decayed operands
    E q[C][LDK];     // Qd
    E k[C][LDK];     // Kd
    E kt[DK][LDC];   // K~^T
  };
  struct Der {       // one chunk's prep results
    E m[C][LDC];     // M (scale and norms folded in), lower triangle
    E tinv[C][LDC];  // (I + A)^-1
    alignas(16) float bet[C];   // beta_t (0 on padded tokens)
    alignas(16) float gb[C];    // rho beta_t / |k_t|
    alignas(16) float gs[C];    // scale / |q_t|
    alignas(16) float dc[C];    // 1 / |k_t|
    alignas(16) float lam[DK];  // Gam_{C-1} per key
  };
  Raw raw[2];
  Der der[2];
  // single-buffered: written in part 1, read in part 2 of the same chunk
  alignas(16) float gp[4][2][C][C];  // partial tiles [wave][KK | QK][t][s]
  alignas(16) float np[4][2][C];     // partial |q_t|^2, |k_t|^2
  alignas(16) float adT[C][20];      // A transposed: adT[s][t] = A[t][s]
  alignas(16) float xq[C][DK];       // exceptional keys: q, k, P, n
  alignas(16) float xk[C][DK];
  alignas(16) float xP[C][DK];
  alignas(16) float xn[C][DK];
  uint32_t xmask[4];                 // exceptional keys: bit 8g + e of wave w's word
};

// DPP move inside 16-lane rows; lanes without a source lane receive `fill`.
template <int CTRL>
__device__ __forceinline__ float pk_dpp(float fill, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Eight consecutive io elements (16 or 32 bytes) from global memory, as fp32.
__device__ __forceinline__ void load8(const __bf16* p, float* o) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    o[e] = bf16_bits_to_float((uint16_t)((e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu)));
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  const f4 a = *reinterpret_cast<const f4*>(p), b = *reinterpret_cast<const f4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = a[e];
    o[4 + e] = b[e];
  }
}

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

template <typename E, int DK, int DVS>
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

  // Workgroups sharing a query/key head are consecutive; keep them on one XCD.
  int blk = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 31) == 0) blk = (blk & 7) * (nblk >> 3) + (blk >> 3);
  const int split = blk % p.nsplit;
  const int h = (blk / p.nsplit) % p.hv;
  const int r = blk / (p.nsplit * p.hv);
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
  const float* __restrict__ gbet = p.beta + (h & p.bmask);

  // ------------------------------------------------------------ state waves
  if (wave < 4) {
    const bool active = wave < NVT;  // waves beyond the slice only keep the barriers
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
    if (active) {
      if (ibase >= 0) {
#pragma unroll
        for (int j = 0; j < NKT; ++j)
          S[j] = *reinterpret_cast<const f4*>(p.init + ibase + (int64_t)vc * DK + dk_of<NKT>(j, 4 * g));
      }
      if (nch > 0) load_v(0);
    }
    f4 X, Y;
    for (int c = -1; c < nch; ++c) {
      const int cur = c & 1;
      const bool work = active && c >= 0;
      // ---- part 1: R = [Qd; Kd] S0, X = beta V - rho beta R_K / |k|, Y = scale R_Q / |q|
      if (work) {
        const typename Sm::Raw& R = sm.raw[cur];
        const typename Sm::Der& Dd = sm.der[cur];
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
        const f4 bt = *reinterpret_cast<const f4*>(&Dd.bet[4 * g]);
        const f4 gb = *reinterpret_cast<const f4*>(&Dd.gb[4 * g]);
        const f4 gs = *reinterpret_cast<const f4*>(&Dd.gs[4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          X[e] = bt[e] * to_f32(vreg[e]) - gb[e] * rk[e];
          Y[e] = gs[e] * rq[e];
        }
        if (c + 1 < nch) load_v(c + 1);
      }
      lds_barrier();
      // ---- part 2: S <- Gam_{C-1} S; U = (I + A)^-1 X; Y += M U; S += K~^T U / |k|
      if (work) {
        const typename Sm::Raw& R = sm.raw[cur];
        const typename Sm::Der& Dd = sm.der[cur];
#pragma unroll
        for (int j = 0; j < NKT; ++j) S[j] = S[j] * *reinterpret_cast<const f4*>(&Dd.lam[dk_of<NKT>(j, 4 * g)]);
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
  const int pw = wave - 4;
  const int kb = 32 * pw + 8 * g;  // first of this lane's 8 keys
  const bool keys = kb < DK;       // lanes past the head size hold zeros
  const bool nrm = p.qk_norm != 0;
  // the next chunk as loaded (converted when it is used)
  float pq[8], pk[8], pd[8], pbt = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) pq[e] = pk[e] = pd[e] = 0.f;
  int prem = 0;
  auto prefetch = [&](int c) {
    const int64_t t0 = start + (int64_t)c * C;
    prem = (int)min((int64_t)C, end - t0);      // >= 1
    const int64_t tok = t0 + min(x, prem - 1);  // clamped: inside the request
    if (keys) {
      load8(gq + tok * p.q_st + kb, pq);
      load8(gk + tok * p.k_st + kb, pk);
      const float* dp = gdec + tok * (int64_t)p.hv * DK + kb;
      const f4 d0 = *reinterpret_cast<const f4*>(dp), d1 = *reinterpret_cast<const f4*>(dp + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pd[e] = d0[e];
        pd[4 + e] = d1[e];
      }
    }
    if (pw == 0) pbt = gbet[(tok * p.hv) & p.bmask];
  };

  if (nch > 0 && pw < NW) prefetch(0);
  for (int c = -1; c < nch; ++c) {
    const int nxt = (c + 1) & 1;
    const bool work = c + 1 < nch;
    float bt = 0.f;  // beta of token x of chunk c+1 (prep wave 4)
    // ---- part 1: scan, decayed operands, partial Gram tiles and norms
    if (work && pw < NW) {
      typename Sm::Raw& R = sm.raw[nxt];
      typename Sm::Der& Dd = sm.der[nxt];
      const bool live = x < prem && keys;
      bt = x < prem ? pbt : 0.f;
      float P[8], n[8], qf[8], kf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = pd[e];
        bool zero;
        float l;
        if (p.decay_is_gamma) {
          zero = !(d > 0.f);
          l = zero ? 0.f : __log2f(d);
        } else {
          zero = !(d > -INFINITY);
          l = zero ? 0.f : d * 1.4426950408889634f;
        }
        P[e] = live ? l : 0.f;  // padded tokens: no decay
        n[e] = zero && live ? 1.f : 0.f;
        qf[e] = live ? pq[e] : 0.f;
        kf[e] = live ? pk[e] : 0.f;
      }
      if (c + 2 < nch) prefetch(c + 2);
      // segmented inclusive scan over the 16 tokens (the lanes x of a row):
      // (P, n) of an earlier span and (P', n') of the later one combine to
      // (n' > 0 ? P' : P + P', n + n')
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
      float qd[8], kd[8], kt[8], kc[8];
      uint32_t xbits = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float PL = pk_dpp<0x15F>(0.f, P[e]), nL = pk_dpp<0x15F>(0.f, n[e]);  // token 15 (row_newbcast)
        const float gam = n[e] == 0.f ? __builtin_amdgcn_exp2f(P[e]) : 0.f;        // Gam_t
        const float gct = n[e] == nL ? __builtin_amdgcn_exp2f(PL - P[e]) : 0.f;    // Gam_{C-1/t}
        const bool exc = nL > 0.f || PL < kPkLog2Floor;                            // same for all tokens
        const float inv = exc ? 0.f : __builtin_amdgcn_exp2f(-P[e]);               // 1 / Gam_t
        qd[e] = qf[e] * gam;
        kd[e] = kf[e] * gam;
        kt[e] = kf[e] * gct;
        kc[e] = kf[e] * inv;
        if (exc) {
          xbits |= 1u << e;
          sm.xq[x][kb + e] = qf[e];
          sm.xk[x][kb + e] = kf[e];
          sm.xP[x][kb + e] = P[e];
          sm.xn[x][kb + e] = n[e];
        }
        if (keys && x == 0) Dd.lam[kb + e] = nL == 0.f ? __builtin_amdgcn_exp2f(PL) : 0.f;
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
      if (lane == 0) sm.xmask[pw] = word;
      // partial Gram tiles: lane (x, g) gets rows s = 4g .. 4g+3 of column t = x
      const f4 zero4 = f4{0.f, 0.f, 0.f, 0.f};
      const f4 kk = mma_k32v(zero4, kc, kd, E{});
      const f4 qk = mma_k32v(zero4, kc, qd, E{});
      *reinterpret_cast<f4*>(&sm.gp[pw][0][x][4 * g]) = kk;
      *reinterpret_cast<f4*>(&sm.gp[pw][1][x][4 * g]) = qk;
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
          sm.np[pw][0][x] = sq;
          sm.np[pw][1][x] = sk;
        }
      }
    }
    lds_barrier();
    // ---- part 2 (prep wave 4): -A, M, the exceptional terms and the inverse
    if (work && pw == 0) {
      typename Sm::Der& Dd = sm.der[nxt];
      const int t = x;
      f4 kk = *reinterpret_cast<const f4*>(&sm.gp[0][0][t][4 * g]);
      f4 qk = *reinterpret_cast<const f4*>(&sm.gp[0][1][t][4 * g]);
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        kk += *reinterpret_cast<const f4*>(&sm.gp[w][0][t][4 * g]);
        qk += *reinterpret_cast<const f4*>(&sm.gp[w][1][t][4 * g]);
      }
      // exceptional keys, term by term (s <= t only)
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        uint32_t mk = sm.xmask[w];  // uniform over the wave
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
          for (int w = 0; w < NW; ++w) s2 += sm.np[w][which][tt];
          s2 += p.qk_eps;
          return s2 > 0.f ? 1.f / sqrtf(s2) : 0.f;
        };
        rqt = inv_norm(0, t);
        rkt = inv_norm(1, t);
#pragma unroll
        for (int e = 0; e < 4; ++e) rks[e] = inv_norm(1, 4 * g + e);
      }
      f4 mrow;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 4 * g + e;
        sm.adT[s][t] = s < t ? p.rho * bt * rkt * rks[e] * kk[e] : 0.f;
        mrow[e] = s <= t ? p.scale * rqt * rks[e] * qk[e] : 0.f;
      }
      *reinterpret_cast<typename pack4<E>::type*>(&Dd.m[t][4 * g]) = to_pack4<E>(mrow);
      if (g == 0) {
        Dd.bet[t] = bt;
        Dd.gb[t] = p.rho * bt * rkt;
        Dd.gs[t] = p.scale * rqt;
        Dd.dc[t] = rkt;
        // row t of (I + A)^-1 by back substitution on the transposed block:
        // T[t][j] = [j == t] - sum_{k > j} A[k][j] T[t][k], j = 15 .. 0
        float row[16];
#pragma unroll
        for (int j = 15; j >= 0; --j) {
          float acc = j == t ? 1.f : 0.f;
#pragma unroll
          for (int k = j + 1; k < 16; ++k) acc -= sm.adT[j][k] * row[k];
          row[j] = acc;
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<typename pack4<E>::type*>(&Dd.tinv[t][4 * q4]) =
              to_pack4<E>(f4{row[4 * q4], row[4 * q4 + 1], row[4 * q4 + 2], row[4 * q4 + 3]});
      }
    }
    lds_barrier();
  }
}

template <typename E, int DK, int DVS>
static hipError_t launch_pk_t(PrefillParams p, hipStream_t stream) {
  p.nsplit = p.dv / DVS;
  const int64_t nblk = (int64_t)p.n_seqs * p.hv * p.nsplit;
  hipLaunchKernelGGL((prefill_pk_kernel<E, DK, DVS>), dim3((unsigned)nblk), dim3(512), 0, stream, p);
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
