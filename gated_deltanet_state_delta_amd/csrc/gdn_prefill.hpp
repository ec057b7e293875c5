// gdn_prefill.hpp -- chunked prefill kernel for the gated delta rule (gfx950).
//
// What is computed: the recurrence of "Gated DeltaNet State Update" (first
// display; readout after the update) for every (request, value head) of a
// packed or ragged batch, with the request, head-map, state-layout and
// empty-request rules of "com.microsoft.GatedDeltaNet" (Inputs / Outputs).
// chunk_size (same card, Attributes) only changes the rounding order.
//
// Chunked form.  Inside a chunk of C tokens t = 0..C-1 entering with state S0
// (K-major dk x dv), write D(t,s) = gamma_{s+1} ... gamma_t for s <= t
// (D(t,t) = 1) and Gam_t = D(t,-1).  Unrolling S_t = gamma_t S_{t-1} + k_t u_t^T
// with u_t = beta_t (v_t - gamma_t S_{t-1}^T k_t) gives the lower-triangular
// system
//     (I + A) U = X,   A_ts = beta_t D(t,s) k_t.k_s (s < t),
//                      X_t  = beta_t (v_t - Gam_t S0^T k_t),
// and then
//     y_t  = scale (Gam_t S0^T q_t + sum_{s<=t} D(t,s) (q_t.k_s) u_s)
//     S_C  = Gam_{C-1} S0 + sum_s D(C-1,s) k_s u_s^T .
// All decays are formed from differences of an in-chunk prefix sum of
// log2(gamma) (never ratios of products), and a gamma of exactly 0 is handled
// exactly by tracking the last zero index z_t inside the chunk:
// D(t,s) = 0 when z_t > s.
//
// Mapping onto gfx950.  One workgroup (4 waves) owns one (request, value
// head, slice of DVS value columns); it walks the request's chunks in order
// and keeps its state slice in MFMA accumulators for the whole request.  Per
// chunk:
//   1. load   Q, K (and a transposed copy of K), the V slice, decay, beta
//             into LDS; padded tokens get gamma = 1, beta = 0, k = q = v = 0;
//   2. scan   (wave 0) prefix sums of log2 gamma, last-zero index, and the
//             factors Gam_t, D(C-1,t);
//   3. gram   lower-triangular 16x16 tiles of K K^T and Q K^T on MFMA, masked
//             and decayed into -A (off-diagonal blocks), the fp32 diagonal
//             blocks of A, and M = D o (Q K^T) (s <= t);
//   4. inv    (wave 0) inverses of the 16x16 unit-lower diagonal blocks of
//             I + A by forward substitution in fp32 (one column per lane);
//   5. state  every wave owns 16-column tiles of the slice and, entirely in
//             registers: R = [Q; K] S0 (MFMA, S0 rounded to the operand
//             type), X, block forward substitution for U using the inverted
//             diagonal blocks and the off-diagonal -A blocks, Y = Gam R_Q +
//             M U, the output store, and S <- Gam_{C-1} S + K^T (D(C-1,.) U).
// The state's accumulator tiles are laid out so that they are directly the B
// operand of the next product (see the fragment notes in gdn_device.hpp):
// the state chain needs no LDS round trip and no barrier among waves.
//
// Operand precision: bf16 inputs use bf16 MFMA operands (the state, U, X, M
// and the inverse blocks are rounded to bf16 as operands; every accumulation,
// the state itself and all decay/gate arithmetic are fp32).  fp32 inputs use
// fp32 MFMA (v_mfma_f32_16x16x4_f32) throughout.
#pragma once

#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
  const float* decay;
  const float* beta;
  const int32_t* cu;
  const float* init;
  float* fin;
  int64_t T;
  int n_seqs, seq_len, hq, hv, dv, nsplit, decay_is_gamma;
  float scale;
};

// LDS layout of one workgroup.
template <typename E, int DK, int DVS, int C>
struct PrefillSmem {
  static constexpr int PAD = 16 / sizeof(E);  // 16-byte row skew
  static constexpr int NT = C / 16;
  static constexpr int LDK = DK + PAD;        // Q, K rows
  static constexpr int LDC = C + PAD;         // K^T, -A, M rows
  static constexpr int LDV = DVS + PAD;       // V rows
  static constexpr int LDT = 16 + PAD;        // inverse blocks
  E q[C][LDK];
  E k[C][LDK];
  E kt[DK][LDC];
  E v[C][LDV];
  E negA[C][LDC];
  E m[C][LDC];
  E tinv[NT][16][LDT];
  float adiag[NT][16][17];
  float F[C];     // prefix sum of log2 gamma over non-zero gammas
  int zr[C];      // last index <= t with gamma == 0, or -1
  float gam[C];   // Gam_t
  float bet[C];   // beta_t (0 on padded tokens)
  float dc[C];    // D(C-1, t)
};

template <typename E, int DK, int DVS, int C>
__global__ void __launch_bounds__(256)
prefill_kernel(const PrefillParams p) {
  typedef typename frag_of<E>::type Fr;
  constexpr int NT = C / 16;      // token tiles per chunk
  constexpr int NKT = DK / 16;    // key tiles
  constexpr int NVT = DVS / 16;   // value tiles per workgroup
  constexpr int VTW = (NVT + 3) / 4;  // value tiles per wave
  constexpr int VE = 16 / sizeof(E);  // elements per 16-byte vector
  typedef PrefillSmem<E, DK, DVS, C> Sm;
  __shared__ Sm sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int x = lane & 15;   // row/column inside a 16x16 tile
  const int g = lane >> 4;   // lane group: contraction indices 4g..4g+3

  // workgroup -> (request, value head, value slice)
  const int blk = blockIdx.x;
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

  const E* __restrict__ gq = (const E*)p.q + (int64_t)qh * p.q_sh;
  const E* __restrict__ gk = (const E*)p.k + (int64_t)qh * p.k_sh;
  const E* __restrict__ gv = (const E*)p.v + (int64_t)h * p.v_sh + v0;
  E* __restrict__ gout = (E*)p.out + (int64_t)h * p.o_sh + v0;

  // ---- state slice: accumulator tiles S[vv][kt], rows = key index, cols = value index
  f4 S[VTW][NKT];
  const int64_t st_base = (((int64_t)r * p.hv + h) * p.dv + v0) * DK;
#pragma unroll
  for (int vv = 0; vv < VTW; ++vv) {
    const int vt = wave + 4 * vv;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      S[vv][kt] = f4{0.f, 0.f, 0.f, 0.f};
      if (p.init && vt < NVT)
        S[vv][kt] = *reinterpret_cast<const f4*>(p.init + st_base + (int64_t)(16 * vt + x) * DK + 16 * kt + 4 * g);
    }
  }

  for (int64_t tok0 = start; tok0 < end; tok0 += C) {
    const int nvalid = (int)min((int64_t)C, end - tok0);

    // ---------------------------------------------------------------- 1. load
    for (int idx = tid; idx < C * (DK / VE); idx += 256) {
      const int t = idx / (DK / VE);
      const int cv = (idx % (DK / VE)) * VE;
      uint4 vq = {0u, 0u, 0u, 0u}, vk = {0u, 0u, 0u, 0u};
      if (t < nvalid) {
        vq = *reinterpret_cast<const uint4*>(gq + (tok0 + t) * p.q_st + cv);
        vk = *reinterpret_cast<const uint4*>(gk + (tok0 + t) * p.k_st + cv);
      }
      *reinterpret_cast<uint4*>(&sm.q[t][cv]) = vq;
      *reinterpret_cast<uint4*>(&sm.k[t][cv]) = vk;
      const E* ke = reinterpret_cast<const E*>(&vk);
#pragma unroll
      for (int e = 0; e < VE; ++e) sm.kt[cv + e][t] = ke[e];
    }
    for (int idx = tid; idx < C * (DVS / VE); idx += 256) {
      const int t = idx / (DVS / VE);
      const int cv = (idx % (DVS / VE)) * VE;
      uint4 vv = {0u, 0u, 0u, 0u};
      if (t < nvalid) vv = *reinterpret_cast<const uint4*>(gv + (tok0 + t) * p.v_st + cv);
      *reinterpret_cast<uint4*>(&sm.v[t][cv]) = vv;
    }
    __syncthreads();

    // ---------------------------------------------------------------- 2. scan
    if (wave == 0) {
      const int t = lane;
      float lg = 0.f, bt = 0.f;
      bool reset = false;
      if (t < nvalid) {
        const float d = p.decay[(tok0 + t) * p.hv + h];
        bt = p.beta[(tok0 + t) * p.hv + h];
        if (p.decay_is_gamma) {
          reset = !(d > 0.f);
          lg = reset ? 0.f : __log2f(d);
        } else {
          reset = !(d > -INFINITY);
          lg = reset ? 0.f : d * 1.4426950408889634f;
        }
      }
      float F = lg;
      int z = reset ? t : -1;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float Fo = __shfl_up(F, off);
        const int zo = __shfl_up(z, off);
        if (lane >= off) {
          F += Fo;
          z = max(z, zo);
        }
      }
      const float Flast = __shfl(F, C - 1);
      const int zlast = __shfl(z, C - 1);
      if (t < C) {
        sm.F[t] = F;
        sm.zr[t] = z;
        sm.gam[t] = z < 0 ? exp2f(F) : 0.f;
        sm.bet[t] = bt;
        sm.dc[t] = zlast <= t ? exp2f(Flast - F) : 0.f;
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- 3. gram
    {
      constexpr int NTILES = NT * (NT + 1) / 2;
      for (int tile = wave; tile < NTILES; tile += 4) {
        int i = 0, rem = tile;
        while (rem > i) { rem -= i + 1; ++i; }
        const int m = rem;  // m <= i
        f4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
        if constexpr (NKT % 2 == 0) {
#pragma unroll
          for (int kb = 0; kb < NKT; kb += 2) {
            Fr ak0, ak1, aq0, aq1, b0, b1;
            lds_frag(&sm.k[16 * i + x][16 * kb + 4 * g], ak0);
            lds_frag(&sm.k[16 * i + x][16 * kb + 16 + 4 * g], ak1);
            lds_frag(&sm.q[16 * i + x][16 * kb + 4 * g], aq0);
            lds_frag(&sm.q[16 * i + x][16 * kb + 16 + 4 * g], aq1);
            lds_frag(&sm.k[16 * m + x][16 * kb + 4 * g], b0);
            lds_frag(&sm.k[16 * m + x][16 * kb + 16 + 4 * g], b1);
            kk = mma_k32(kk, ak0, ak1, b0, b1);
            qk = mma_k32(qk, aq0, aq1, b0, b1);
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < NKT; ++kb) {
            Fr ak, aq, b;
            lds_frag(&sm.k[16 * i + x][16 * kb + 4 * g], ak);
            lds_frag(&sm.q[16 * i + x][16 * kb + 4 * g], aq);
            lds_frag(&sm.k[16 * m + x][16 * kb + 4 * g], b);
            kk = mma_k16(kk, ak, b);
            qk = mma_k16(qk, aq, b);
          }
        }
        const int s = 16 * m + x;
        const float Fs = sm.F[s];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * i + 4 * g + e;
          const float d = (s <= t && sm.zr[t] <= s) ? exp2f(sm.F[t] - Fs) : 0.f;
          sm.m[t][s] = from_f32<E>(d * qk[e]);
          const float av = (s < t) ? sm.bet[t] * d * kk[e] : 0.f;
          if (i == m) sm.adiag[i][4 * g + e][x] = av;
          else sm.negA[t][s] = from_f32<E>(-av);
        }
      }
    }
    __syncthreads();

    // ----------------------------------------------------------------- 4. inv
    if (wave == 0 && g < NT) {
      // column x of (I + A_gg)^-1 by forward substitution
      float col[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float acc = (rr == x) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < rr; ++j) acc -= sm.adiag[g][rr][j] * col[j];
        col[rr] = acc;
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sm.tinv[g][rr][x] = from_f32<E>(col[rr]);
    }
    __syncthreads();

    // --------------------------------------------------------------- 5. state
#pragma unroll
    for (int vv = 0; vv < VTW; ++vv) {
      const int vt = wave + 4 * vv;
      if (vt >= NVT) break;
      const int vc = 16 * vt + x;  // this lane's value column inside the slice

      Fr Sb[NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) cvt_frag(S[vv][kt], Sb[kt]);

      // R = [Q; K] S0 ;  X = beta (V - Gam R_K) ;  Y = Gam R_Q
      f4 X[NT], Y[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        f4 rq = {0.f, 0.f, 0.f, 0.f}, rk = {0.f, 0.f, 0.f, 0.f};
        if constexpr (NKT % 2 == 0) {
#pragma unroll
          for (int kt = 0; kt < NKT; kt += 2) {
            Fr aq0, aq1, ak0, ak1;
            lds_frag(&sm.q[16 * i + x][16 * kt + 4 * g], aq0);
            lds_frag(&sm.q[16 * i + x][16 * kt + 16 + 4 * g], aq1);
            lds_frag(&sm.k[16 * i + x][16 * kt + 4 * g], ak0);
            lds_frag(&sm.k[16 * i + x][16 * kt + 16 + 4 * g], ak1);
            rq = mma_k32(rq, aq0, aq1, Sb[kt], Sb[kt + 1]);
            rk = mma_k32(rk, ak0, ak1, Sb[kt], Sb[kt + 1]);
          }
        } else {
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt) {
            Fr aq, ak;
            lds_frag(&sm.q[16 * i + x][16 * kt + 4 * g], aq);
            lds_frag(&sm.k[16 * i + x][16 * kt + 4 * g], ak);
            rq = mma_k16(rq, aq, Sb[kt]);
            rk = mma_k16(rk, ak, Sb[kt]);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * i + 4 * g + e;
          const float gm = sm.gam[t];
          X[i][e] = sm.bet[t] * (to_f32(sm.v[t][vc]) - gm * rk[e]);
          Y[i][e] = gm * rq[e];
        }
      }

      // (I + A) U = X by 16-row blocks: U_i = Tinv_i (X_i - sum_{m<i} A_im U_m)
      f4 U[NT];
      Fr Ub[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        f4 P = X[i];
#pragma unroll
        for (int m = 0; m < i; ++m) {
          Fr a;
          lds_frag(&sm.negA[16 * i + x][16 * m + 4 * g], a);
          P = mma_k16(P, a, Ub[m]);
        }
        Fr Pb, ti;
        cvt_frag(P, Pb);
        lds_frag(&sm.tinv[i][x][4 * g], ti);
        U[i] = mma_k16(f4{0.f, 0.f, 0.f, 0.f}, ti, Pb);
        cvt_frag(U[i], Ub[i]);
      }

      // Y += M U ; store
#pragma unroll
      for (int i = 0; i < NT; ++i) {
#pragma unroll
        for (int m = 0; m <= i; ++m) {
          Fr a;
          lds_frag(&sm.m[16 * i + x][16 * m + 4 * g], a);
          Y[i] = mma_k16(Y[i], a, Ub[m]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * i + 4 * g + e;
          if (t < nvalid) gout[(tok0 + t) * p.o_st + vc] = from_f32<E>(p.scale * Y[i][e]);
        }
      }

      // S <- Gam_{C-1} S + K^T (D(C-1, .) U)
      Fr DU[NT];
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        f4 du;
#pragma unroll
        for (int e = 0; e < 4; ++e) du[e] = sm.dc[16 * m + 4 * g + e] * U[m][e];
        cvt_frag(du, DU[m]);
      }
      const float gC = sm.gam[C - 1];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        f4 acc = gC * S[vv][kt];
        if constexpr (NT % 2 == 0) {
#pragma unroll
          for (int m = 0; m < NT; m += 2) {
            Fr a0, a1;
            lds_frag(&sm.kt[16 * kt + x][16 * m + 4 * g], a0);
            lds_frag(&sm.kt[16 * kt + x][16 * m + 16 + 4 * g], a1);
            acc = mma_k32(acc, a0, a1, DU[m], DU[m + 1]);
          }
        } else {
#pragma unroll
          for (int m = 0; m < NT; ++m) {
            Fr a;
            lds_frag(&sm.kt[16 * kt + x][16 * m + 4 * g], a);
            acc = mma_k16(acc, a, DU[m]);
          }
        }
        S[vv][kt] = acc;
      }
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ final state
#pragma unroll
  for (int vv = 0; vv < VTW; ++vv) {
    const int vt = wave + 4 * vv;
    if (vt < NVT) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
        *reinterpret_cast<f4*>(p.fin + st_base + (int64_t)(16 * vt + x) * DK + 16 * kt + 4 * g) = S[vv][kt];
    }
  }
}

// Value columns per workgroup for an operand type and chunk (LDS budget).
template <typename E, int DV, int C>
constexpr int prefill_dvs() {
  if constexpr (sizeof(E) == 2) return DV < 64 ? DV : 64;
  else return (C == 64) ? (DV < 32 ? DV : 32) : (DV < 64 ? DV : 64);
}

template <typename E, int DK, int DV, int C>
hipError_t launch_prefill_t(PrefillParams p, hipStream_t stream) {
  constexpr int DVS = prefill_dvs<E, DV, C>();
  static_assert(sizeof(PrefillSmem<E, DK, DVS, C>) <= 160 * 1024, "LDS budget");
  p.nsplit = DV / DVS;
  const int64_t nblk = (int64_t)p.n_seqs * p.hv * p.nsplit;
  hipLaunchKernelGGL((prefill_kernel<E, DK, DVS, C>), dim3((unsigned)nblk), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename E, int C>
hipError_t dispatch_prefill_dk_dv(PrefillParams p, int dk, int dv, hipStream_t s) {
#define GDN_DV_CASES(DK)                                           \
  switch (dv) {                                                    \
    case 16: return launch_prefill_t<E, DK, 16, C>(p, s);          \
    case 32: return launch_prefill_t<E, DK, 32, C>(p, s);          \
    case 64: return launch_prefill_t<E, DK, 64, C>(p, s);          \
    case 128: return launch_prefill_t<E, DK, 128, C>(p, s);        \
  }                                                                \
  break;
  switch (dk) {
    case 16: GDN_DV_CASES(16)
    case 32: GDN_DV_CASES(32)
    case 64: GDN_DV_CASES(64)
    case 128: GDN_DV_CASES(128)
  }
#undef GDN_DV_CASES
  return hipErrorInvalidValue;
}

// One instantiation unit per (operand type, chunk): gdn_prefill_<t>_c<C>.hip
hipError_t prefill_bf16_c16(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_bf16_c32(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_bf16_c64(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_f32_c16(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_f32_c32(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_f32_c64(PrefillParams p, int dk, int dv, hipStream_t s);

}  // namespace gdn
