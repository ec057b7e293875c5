// gdn_prefill_pair.hpp -- chunked prefill for bf16 inputs with dk, dv in
// {64, 128} and 64-token chunks (gfx950).
//
// Same chunked form of the "Gated DeltaNet State Update" recurrence as
// prefill_kernel (gdn_prefill.hpp has the derivation): inside a chunk,
// (I + A) U = X with A_ts = beta_t D(t,s) k_t.k_s and X = beta (V - Gam K S0),
// Y = scale (Gam Q S0 + (D o Q K^T) U), S_C = Gam_{C-1} S0 + K^T (D(C-1,.) U).
// Only the schedule differs; it is built for this case:
//
//  * one workgroup of 4 waves -- one per SIMD, so each may hold up to 512
//    registers -- per (request, value head, 64-column slice of the state);
//  * state waves 0 and 1 each own 32 value columns (two 16-column MFMA
//    tiles), so every Q, K and K^T fragment read from LDS feeds two MFMAs;
//    state wave w inverts the unit-lower diagonal blocks I + A_ii,
//    i = 2w, 2w+1, of chunk c (right-looking, one lane pair per row) and
//    shares them through LDS (a counter tells when both halves are there);
//    both then run [Q; K] S0, the block forward substitution, Y += M U and
//    the state update; they accumulate the outputs transposed (Y^T, the
//    MFMA operands swapped), so each lane holds 4 columns of one token and,
//    after a lane swap between 16-lane rows, stores 16-byte row pieces
//    straight to memory;
//  * prep waves 2 and 3 prepare chunk c+1 meanwhile.  Each loads half of the
//    chunk's Q, K and V rows (two chunks ahead: token-strided loads have a
//    long latency) and stages them in LDS; after an LDS counter shows both
//    halves written, each computes two diagonal and three off-diagonal
//    16x16 Gram tiles, their M and -A blocks (the decay D(t,s) of an
//    off-diagonal tile factored into three per-tile factors <= 1 unless the
//    chunk holds a gamma of exactly 0), and the fp32 rows of its two
//    diagonal blocks A_ii; wave 2 also writes the per-token factors;
//  * one workgroup barrier per chunk: the state waves read buffer c & 1 while
//    the prep waves fill buffer (c+1) & 1;
//  * options, each its own instantiation: the fused gate (the prep waves gate
//    a and b when they stage a chunk) and the in-kernel q/k L2 norm (1/|q_t|
//    and 1/|k_t| from the diagonals of the diagonal Gram tiles, folded into
//    the per-token factors and the -A and M blocks; q and k stay as given).
// K^T fragments for the state update and V in accumulator layout come from
// LDS through the gfx950 transposing LDS read
// (ds_read_b64_tr_b16): lane 4a+b of a 16-lane group receives element b of
// the 8-byte block addressed by lane a+4e as its element e.
//
// LDS rows of Q and K hold 16-byte slots permuted by an XOR of the row
// (slot ^ f(row)), so fragment reads of 8 consecutive rows hit 8 distinct
// bank groups.  All accumulator chains use one MFMA shape (see the note in
// gdn_prefill.hpp).
#pragma once

#include "gdn_prefill.hpp"

namespace gdn {

template <int DK>
struct PairSmem {
  static constexpr int C = 64, NT = 4, DVS = 64;
  static constexpr int LDV = DVS + 16;  // 160-byte V rows
  static constexpr int LDC = C + 4;     // 136-byte -A / M rows
  static constexpr int LDT = 20;        // 40-byte inverse rows
  struct Buf {
    __bf16 q[C][DK];      // slot-swizzled rows
    __bf16 k[C][DK];
    __bf16 v[C][LDV];
    __bf16 negA[C][LDC];  // -A, off-diagonal 16x16 blocks
    __bf16 m[C][LDC];     // scale D o Q K^T, blocks on and below the diagonal
    alignas(16) float bet[C];  // beta_t (0 on padded tokens)
    alignas(16) float gb[C];   // beta_t Gam_t
    alignas(16) float gs[C];   // scale Gam_t
    alignas(16) float dc[C];   // D(C-1, t)
    alignas(16) float rqn[C];  // 1 / |q_t| and 1 / |k_t| (in-kernel L2 norm only)
    alignas(16) float rkn[C];
    float gC;                  // Gam_{C-1}
  };
  struct Scan {                // decay scan of the chunk being prepared (per prep wave)
    alignas(16) float F[C];    // prefix sum of log2 gamma over non-zero gammas
    alignas(16) int z[C];      // last index <= t whose gamma is 0, or -1
    alignas(16) float bt[C];   // beta_t (0 on padded tokens)
    alignas(16) float E[C];    // 2^(F_t - F at the start of t's 16-token tile)
    alignas(16) float Fx[C];   // 2^(F at the end of t's 16-token tile - F_t)
  };
  alignas(16) Buf buf[2];
  Scan scan[2];  // one per prep wave
  // rows of the fp32 diagonal blocks of A, one set per chunk parity: block
  // i, row r at 20 r, split by column parity (adiag[b][i][20 r + 8 h + jj] =
  // A_ii[r][2 jj + h]; padded rows and blocks keep the row reads of the four
  // blocks on distinct banks)
  alignas(16) float adiag[2][NT][16 * 20 + 4];
  // (I + A_ii)^-1 of the current chunk, bf16 (blocks 2w, 2w+1 written by
  // state wave w)
  alignas(16) __bf16 tinv[NT][16][LDT];
  int prep_cnt;  // staging halves written by the prep waves so far
  int nrm_cnt;   // norm halves written by the prep waves so far (L2 norm only)
  int inv_cnt;   // inverse halves written by the state waves so far
};

// 16-byte slot permutation of a Q/K row.
__device__ __forceinline__ int pair_swz(int row, int slot) {
  return slot ^ (((row & 1) << 2) | ((row >> 1) & 3));
}

typedef __attribute__((address_space(3))) s4 lds_s4;

// Transposing LDS read (see the header comment).
__device__ __forceinline__ bf4 lds_tr(const __bf16* p) {
  return __builtin_bit_cast(bf4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p)));
}
__device__ __forceinline__ bf4 lds_b64(const __bf16* p) { return *reinterpret_cast<const bf4*>(p); }
__device__ __forceinline__ bf8 lds_b128(const __bf16* p) { return *reinterpret_cast<const bf8*>(p); }
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, bf2));
}
__device__ __forceinline__ bf4 to_bf4(f4 v) {
  return __builtin_bit_cast(bf4, (u32x2){pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])});
}
__device__ __forceinline__ f4 bf4_to_f4(bf4 v) {
  return f4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f4 mfma32(f4 acc, bf8 a, bf8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ bf8 cat8(bf4 lo, bf4 hi) {
  return bf8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// DPP moves: lanes whose row is not in ROWMASK (or whose source lane lies
// outside the row for the shifts) receive `fill`.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f(float fill, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_i(int fill, int v) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, ROWMASK, 0xF, false);
}
// Inclusive wave-wide scans (sum, max) in lane order: shifts within 16-lane
// rows (row_shr 1, 2, 4, 8), then the row totals carried across rows
// (row_bcast 15 into rows 1 and 3, row_bcast 31 into rows 2 and 3).
__device__ __forceinline__ float wave_scan_add(float v) {
  v += dpp_f<0x111, 0xF>(0.f, v);
  v += dpp_f<0x112, 0xF>(0.f, v);
  v += dpp_f<0x114, 0xF>(0.f, v);
  v += dpp_f<0x118, 0xF>(0.f, v);
  v += dpp_f<0x142, 0xA>(0.f, v);
  v += dpp_f<0x143, 0xC>(0.f, v);
  return v;
}
__device__ __forceinline__ int wave_scan_max(int v) {
  v = max(v, dpp_i<0x111, 0xF>(-1, v));
  v = max(v, dpp_i<0x112, 0xF>(-1, v));
  v = max(v, dpp_i<0x114, 0xF>(-1, v));
  v = max(v, dpp_i<0x118, 0xF>(-1, v));
  v = max(v, dpp_i<0x142, 0xA>(-1, v));
  v = max(v, dpp_i<0x143, 0xC>(-1, v));
  return v;
}

// One prep wave's half of a chunk, as loaded from global memory: Q and K
// tiles 2pw and 2pw+1 (16-byte fragment rows: row 16i + x, keys 32pp + 8g
// .. +7), V rows 32pw .. 32pw+31 (row 32pw + 8u + lane/8, columns 8 (lane % 8)
// .. +7), and the gate of token `lane`.  (Loads of 16 rows x 64 bytes measured
// faster here than loads of 4 rows x 256 bytes.)
template <int DK>
struct PairPrepSet {
  static constexpr int NPP = DK / 32;
  u32x4 q[2][NPP];
  u32x4 k[2][NPP];
  u32x4 v[4];
  float gd, bt;      // decay and beta of token `lane` as loaded (clamped to the chunk)
  __bf16 ga, gbr;    // or the fused gate's raw a and b
};

// Inverse of the unit-lower block I + A_i (A_i strictly lower, fp32 rows in
// `ad` as laid out by the prep waves), right-looking: a lane pair owns row
// r = (lane / 2) % 16 of block i = i0 + lane / 32; lane parity h keeps
// T[r][j] for j = h mod 2.  T[r][j] = [j == r] - sum_{k > j} T[r][k] A[k][j];
// once T[r][k] is final (its owner lane passes it to the partner) it updates
// every j < k.  A is strictly lower, so updates of entries j >= k add zero.
// Writes row r of T_i in bf16 to tout[i][r][0..15].
template <int LDT>
__device__ __forceinline__ void pair_tri_inverse(const float (*ad)[16 * 20 + 4], __bf16 (*tout)[16][LDT], int i0,
                                                 int lane) {
  const int i = i0 + (lane >> 5), r = (lane >> 1) & 15, h = lane & 1;
  const float* arow = &ad[i][8 * h];
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
    // the entry the next step reads first, then the rest
    acc[(k - 1) >> 1] -= tk * ak((k - 1) >> 1);
#pragma unroll
    for (int jj = 0; jj < ((k - 1) >> 1); ++jj) acc[jj] -= tk * ak(jj);
  }
  // row r, columns 8 h .. 8 h + 7: even entries from lane parity 0, odd ones
  // from parity 1
  float o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float even_lo = acc[q], even_hi = acc[4 + q];  // my parity's values
    const float sw_lo = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(even_lo), 0xB1, 0xF, 0xF, false));
    const float sw_hi = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(even_hi), 0xB1, 0xF, 0xF, false));
    // h == 0 assembles columns 0..7: T[r][2q] (mine, jj = q), T[r][2q+1] (partner's jj = q)
    // h == 1 assembles columns 8..15: T[r][8+2q] (partner's jj = 4+q), T[r][9+2q] (mine, jj = 4+q)
    o[2 * q] = h == 0 ? even_lo : sw_hi;
    o[2 * q + 1] = h == 0 ? sw_lo : even_hi;
  }
  *reinterpret_cast<bf4*>(&tout[i][r][8 * h]) = to_bf4(f4{o[0], o[1], o[2], o[3]});
  *reinterpret_cast<bf4*>(&tout[i][r][8 * h + 4]) = to_bf4(f4{o[4], o[5], o[6], o[7]});
}

// Prep wave PW of the pair kernel (see the header comment).  FUSED: the gates
// come from A_log, dt_bias, a, b (computed here); NORM: the in-kernel q/k L2
// norm.  Each combination is its own instantiation, so none carries branches
// for the options it does not use.
template <int DK, int PW, bool FUSED, bool NORM>
__device__ __forceinline__ void pair_prep(const PrefillParams& p, PairSmem<DK>& sm, int64_t start,
                                          int64_t end, int nch, const __bf16* gq, const __bf16* gk,
                                          const __bf16* gv, int h) {
  typedef PairSmem<DK> Sm;
  constexpr int C = 64, NPP = DK / 32;
  const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
  // gates: given (decay, beta) or fused (A_log, dt_bias, a, b: the qwen gate
  // and a sigmoid beta, computed here per token)
  constexpr bool fused = FUSED;
  const float* gdec = p.decay + (h & p.dmask);
  const float* gbet = p.beta + (h & p.bmask);
  const __bf16* gga = (const __bf16*)p.ga + (h & p.dmask);
  const __bf16* ggb = (const __bf16*)p.gb + (h & p.bmask);
  const float ealog = fused ? expf(p.A_log[h & p.dmask]) : 0.f, dtb = fused ? p.dt_bias[h & p.dmask] : 0.f;
  constexpr bool nrm = NORM;

  auto prefetch = [&](int c, PairPrepSet<DK>& s) {
    const int64_t t0 = start + (int64_t)c * C;
    const int rem = (int)min((int64_t)C, end - t0);  // >= 1
    {
      // the values exactly as loaded: nothing here may wait on these loads
      // (padding and the fused gate are applied when the set is staged)
      const int tl = min(lane, rem - 1);
      const int64_t tok = (t0 + tl) * p.hv;
      if constexpr (FUSED) {
        s.ga = gga[tok & p.dmask];
        s.gbr = ggb[tok & p.bmask];
      } else {
        s.gd = gdec[tok & p.dmask];
        s.bt = gbet[tok & p.bmask];
      }
    }
    const __bf16* qb = gq + t0 * p.q_st;
    const __bf16* kb = gk + t0 * p.k_st;
    const __bf16* vb = gv + t0 * p.v_st;
    const int qst = (int)p.q_st, kst = (int)p.k_st, vst = (int)p.v_st;
    if (rem == C) {
      const __amdgpu_buffer_rsrc_t rq = buf_rsrc(qb), rk = buf_rsrc(kb), rv = buf_rsrc(vb);
      const uint32_t lq = (uint32_t)((x * qst + 8 * g) * 2), lk = (uint32_t)((x * kst + 8 * g) * 2);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int pp = 0; pp < NPP; ++pp) {
          s.q[i][pp] = buf_load16(rq, lq, (uint32_t)((16 * (2 * PW + i) * qst + 32 * pp) * 2));
          s.k[i][pp] = buf_load16(rk, lk, (uint32_t)((16 * (2 * PW + i) * kst + 32 * pp) * 2));
        }
      const uint32_t lv = (uint32_t)(((lane >> 3) * vst + 8 * (lane & 7)) * 2);
#pragma unroll
      for (int u = 0; u < 4; ++u) s.v[u] = buf_load16(rv, lv, (uint32_t)((32 * PW + 8 * u) * vst * 2));
    } else {
      auto ld = [&](const __bf16* base, int st, int row, int col) -> u32x4 {
        const u32x4 val = *reinterpret_cast<const u32x4*>(base + (int64_t)min(row, rem - 1) * st + col);
        return val & (row < rem ? 0xffffffffu : 0u);
      };
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int pp = 0; pp < NPP; ++pp) {
          s.q[i][pp] = ld(qb, qst, 16 * (2 * PW + i) + x, 32 * pp + 8 * g);
          s.k[i][pp] = ld(kb, kst, 16 * (2 * PW + i) + x, 32 * pp + 8 * g);
        }
#pragma unroll
      for (int u = 0; u < 4; ++u) s.v[u] = ld(vb, vst, 32 * PW + 8 * u + (lane >> 3), 8 * (lane & 7));
    }
  };

  auto frag_col = [&](int row, int pp) -> int { return 8 * pair_swz(row, 4 * pp + g); };

  int staged = 0;  // chunks staged by this wave so far
  // One iteration: prepare chunk c+1 from `s`, then refill `s` with chunk c+3.
  auto iter = [&](int c, PairPrepSet<DK>& s) {
    if (c + 1 < nch) {
      typename Sm::Buf& B = sm.buf[(c + 1) & 1];
      // ---- stage this wave's half
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int pp = 0; pp < NPP; ++pp) {
          const int r = 16 * (2 * PW + i) + x;
          *reinterpret_cast<u32x4*>(&B.q[r][frag_col(r, pp)]) = s.q[i][pp];
          *reinterpret_cast<u32x4*>(&B.k[r][frag_col(r, pp)]) = s.k[i][pp];
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<u32x4*>(&B.v[32 * PW + 8 * u + (lane >> 3)][8 * (lane & 7)]) = s.v[u];
      // gates of token `lane`; padded tokens: no decay (log-decay 0 / gamma
      // 1) and beta 0
      const bool live = lane < (int)min((int64_t)C, end - (start + (int64_t)(c + 1) * C));
      float gd, btl;
      if constexpr (FUSED) {  // an absent input: no decay, beta 1
        gd = live && p.dmask ? gate_log_decay_fast(ealog, dtb, (float)s.ga) : 0.f;
        btl = live ? (p.bmask ? sigmoid_fast((float)s.gbr) : 1.f) : 0.f;
      } else {
        gd = live ? s.gd : (p.decay_is_gamma ? 1.f : 0.f);
        btl = live ? s.bt : 0.f;
      }
      // ---- signal this half written and refill the registers; the wait for
      // the other prep wave's half comes after the scan.  Both prep waves
      // stage every chunk, so that wait ends; its bound only guards against a
      // wave that never arrives.
      ++staged;
      if (lane == 0) __hip_atomic_fetch_add(&sm.prep_cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (c + 3 < nch) prefetch(c + 3, s);
      // ---- decay scan (lane = token)
      typename Sm::Scan& sc = sm.scan[PW];
      bool reset;
      float lg;
      if (p.decay_is_gamma) {
        reset = !(gd > 0.f);
        lg = reset ? 0.f : __log2f(gd);
      } else {
        reset = !(gd > -INFINITY);
        lg = reset ? 0.f : gd * 1.4426950408889634f;
      }
      const float F = wave_scan_add(lg);
      const int z = wave_scan_max(reset ? lane : -1);
      const float Flast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(F), C - 1));
      const int zlast = __builtin_amdgcn_readlane(z, C - 1);
      sc.F[lane] = F;
      sc.z[lane] = z;
      sc.bt[lane] = p.rho * btl;  // beta as it enters A (the retrieval term)
      {
        // F at the first and last lane of this lane's 16-lane row (row_newbcast)
        const float Fb0 = dpp_f<0x150, 0xF>(0.f, F), Fb1 = dpp_f<0x15F, 0xF>(0.f, F);
        sc.E[lane] = __builtin_amdgcn_exp2f(F - Fb0);
        sc.Fx[lane] = __builtin_amdgcn_exp2f(Fb1 - F);
      }
      for (int spin = 0; spin < (1 << 22); ++spin) {
        if (__hip_atomic_load(&sm.prep_cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= 2 * staged) break;
        __builtin_amdgcn_s_sleep(1);
      }
      const bool any_zero = zlast >= 0;  // wave-uniform

      // ---- per-token factors of the state waves (wave 2), after the norms
      // of all tokens are known when the in-kernel L2 norm is on
      auto factors = [&]() {
        if constexpr (PW == 0) {
          const float gam = z < 0 ? __builtin_amdgcn_exp2f(F) : 0.f;
          const float rq = nrm ? B.rqn[lane] : 1.f, rk = nrm ? B.rkn[lane] : 1.f;
          B.bet[lane] = btl;
          B.gb[lane] = p.rho * btl * gam * rk;
          B.gs[lane] = p.scale * gam * rq;
          B.dc[lane] = zlast <= lane ? __builtin_amdgcn_exp2f(Flast - F) * rk : 0.f;
          if (lane == C - 1) B.gC = gam;
        }
      };
      if constexpr (!NORM) factors();
      // ---- Gram tiles, computed transposed (rows s, columns t): this wave's
      // diagonal tiles (D0, D0), (D0+1, D0+1) and three off-diagonal tiles
      // (TI[n], TM[n]): wave 2 (1,0) (2,0) (3,0), wave 3 (2,1) (3,1) (3,2)
      constexpr int D0 = 2 * PW;
      constexpr int TI[3] = {PW == 0 ? 1 : 2, PW == 0 ? 2 : 3, 3};
      constexpr int TM[3] = {PW == 0 ? 0 : 1, PW == 0 ? 0 : 1, PW == 0 ? 0 : 2};
      constexpr int KLO = PW == 0 ? 0 : 1, QLO = PW == 0 ? 0 : 2;  // tiles read
      f4 kkd[2], qkd[2], qqd[2], kko[3], qko[3];
#pragma unroll
      for (int n = 0; n < 2; ++n) kkd[n] = qkd[n] = qqd[n] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < 3; ++n) kko[n] = qko[n] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < NPP; ++pp) {
        bf8 kf[4], qf[4];
#pragma unroll
        for (int i = KLO; i < 4; ++i) {
          const int r = 16 * i + x;
          kf[i] = lds_b128(&B.k[r][frag_col(r, pp)]);
        }
#pragma unroll
        for (int i = QLO; i < 4; ++i) {
          const int r = 16 * i + x;
          qf[i] = lds_b128(&B.q[r][frag_col(r, pp)]);
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          kkd[n] = mfma32(kkd[n], kf[D0 + n], kf[D0 + n]);
          qkd[n] = mfma32(qkd[n], kf[D0 + n], qf[D0 + n]);
          if constexpr (NORM) qqd[n] = mfma32(qqd[n], qf[D0 + n], qf[D0 + n]);
        }
#pragma unroll
        for (int n = 0; n < 3; ++n) {
          kko[n] = mfma32(kko[n], kf[TM[n]], kf[TI[n]]);
          qko[n] = mfma32(qko[n], kf[TM[n]], qf[TI[n]]);
        }
      }
      if constexpr (NORM) {
        // ---- in-kernel L2 norm: |k_t|^2 and |q_t|^2 are the diagonals of this
        // wave's diagonal tiles K K^T and Q Q^T (token t = 16i + x sits on lane
        // (x, x/4), element x % 4).  The factors 1/|.| go to LDS; the other
        // wave's are waited for (a counter) after the diagonal epilogue, which
        // needs only this wave's.  Both waves write every chunk, so the wait
        // ends.  An all-zero vector (a padded token, or eps == 0) keeps the
        // factor 0.
        if (g == (x >> 2)) {
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const int e = x & 3;
            const float k2 = (e == 0 ? kkd[n][0] : e == 1 ? kkd[n][1] : e == 2 ? kkd[n][2] : kkd[n][3]) + p.qk_eps;
            const float q2 = (e == 0 ? qqd[n][0] : e == 1 ? qqd[n][1] : e == 2 ? qqd[n][2] : qqd[n][3]) + p.qk_eps;
            B.rkn[16 * (D0 + n) + x] = k2 > 0.f ? __builtin_amdgcn_rsqf(k2) : 0.f;
            B.rqn[16 * (D0 + n) + x] = q2 > 0.f ? __builtin_amdgcn_rsqf(q2) : 0.f;
          }
        }
        if (lane == 0) __hip_atomic_fetch_add(&sm.nrm_cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      // ---- diagonal tiles: M blocks, and the rows of A_ii (fp32) split by
      // column parity for the inverses
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int i = D0 + n;
        const int t = 16 * i + x;
        const float Ft = sc.F[t];
        const f4 Fs = *reinterpret_cast<const f4*>(&sc.F[16 * i + 4 * g]);
        const float bt = sc.bt[t];
        const int zt = sc.z[t];
        // in-kernel L2 norm: row factor 1/|q_t| or 1/|k_t|, column 1/|k_s|
        const f4 one4 = f4{1.f, 1.f, 1.f, 1.f};
        const f4 rks = nrm ? *reinterpret_cast<const f4*>(&B.rkn[16 * i + 4 * g]) : one4;
        const f4 fq = rks * (nrm ? B.rqn[t] : 1.f), fk = rks * (nrm ? B.rkn[t] : 1.f);
        f4 d, arow;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sidx = 16 * i + 4 * g + e;
          const bool live = sidx <= t && (!any_zero || zt <= sidx);
          d[e] = live ? __builtin_amdgcn_exp2f(Ft - Fs[e]) : 0.f;
          arow[e] = sidx < t ? bt * d[e] * kkd[n][e] * fk[e] : 0.f;
        }
        *reinterpret_cast<bf4*>(&B.m[t][16 * i + 4 * g]) = to_bf4(p.scale * d * qkd[n] * fq);
        float* ad = sm.adiag[(c + 1) & 1][i];
        *reinterpret_cast<f2*>(&ad[20 * x + 2 * g]) = f2{arow[0], arow[2]};
        *reinterpret_cast<f2*>(&ad[20 * x + 8 + 2 * g]) = f2{arow[1], arow[3]};
      }
      if constexpr (NORM) {
        for (int spin = 0; spin < (1 << 22); ++spin) {
          if (__hip_atomic_load(&sm.nrm_cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= 2 * staged) break;
          __builtin_amdgcn_s_sleep(1);
        }
        factors();
      }
      // ---- off-diagonal tiles: -A and M blocks.  D(t, s) = e_t c_im f_s for
      // s in tile m < i, t in tile i, with e_t = 2^(F_t - F_16i),
      // f_s = 2^(F_16m+15 - F_s), c_im = 2^(F_16i - F_16m+15), each <= 1;
      // the exact form when the chunk holds a gamma of 0
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        const int i = TI[n], m = TM[n];
        const int t = 16 * i + x;
        const float bt = sc.bt[t];
        f4 dm, da;  // decay times scale, decay times -beta_t
        if (!any_zero) {
          const float cim = __builtin_amdgcn_exp2f(sc.F[16 * i] - sc.F[16 * m + 15]);
          const float et = sc.E[t] * cim;
          const f4 fs = *reinterpret_cast<const f4*>(&sc.Fx[16 * m + 4 * g]);
          dm = (p.scale * et) * fs;
          da = (-bt * et) * fs;
        } else {
          const float Ft = sc.F[t];
          const int zt = sc.z[t];
          const f4 Fs = *reinterpret_cast<const f4*>(&sc.F[16 * m + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d = zt <= 16 * m + 4 * g + e ? __builtin_amdgcn_exp2f(Ft - Fs[e]) : 0.f;
            dm[e] = p.scale * d;
            da[e] = -bt * d;
          }
        }
        if constexpr (NORM) {
          const f4 rks = *reinterpret_cast<const f4*>(&B.rkn[16 * m + 4 * g]);
          dm = dm * (rks * B.rqn[t]);
          da = da * (rks * B.rkn[t]);
        }
        *reinterpret_cast<bf4*>(&B.m[t][16 * m + 4 * g]) = to_bf4(dm * qko[n]);
        *reinterpret_cast<bf4*>(&B.negA[t][16 * m + 4 * g]) = to_bf4(da * kko[n]);
      }
    }
    lds_barrier();
  };

  PairPrepSet<DK> sa, sb;
  if (nch > 0) prefetch(0, sa);
  if (nch > 1) prefetch(1, sb);
  for (int c = -1; c < nch; c += 2) {
    iter(c, sa);
    if (c + 1 < nch) iter(c + 1, sb);
  }
}

template <int DK, bool FUSED, bool NORM>
__global__ void __launch_bounds__(256, 1)
prefill_pair_kernel(const PrefillParams p) {
  typedef PairSmem<DK> Sm;
  constexpr int C = 64, NKT = DK / 16, NPP = DK / 32;
  __shared__ Sm sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int x = lane & 15;
  const int g = lane >> 4;

  int blk = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 31) == 0) blk = (blk & 7) * (nblk >> 3) + (blk >> 3);
  const int split = blk % p.nsplit;
  const int h = (blk / p.nsplit) % p.hv;
  const int r = blk / (p.nsplit * p.hv);
  const int qh = (int)(((int64_t)h * p.hq) / p.hv);
  const int v0 = split * 64;

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

  const __bf16* __restrict__ gq = (const __bf16*)p.q + (int64_t)qh * p.q_sh;
  const __bf16* __restrict__ gk = (const __bf16*)p.k + (int64_t)qh * p.k_sh;
  const __bf16* __restrict__ gv = (const __bf16*)p.v + (int64_t)h * p.v_sh + v0;
  __bf16* __restrict__ gout = (__bf16*)p.out + (int64_t)h * p.o_sh + v0;
  int64_t ibase, fbase;
  prefill_state_offsets(p, r, h, v0, DK, ibase, fbase);
  if ((p.pool_flags & kPoolSkipUnread) && ibase < 0) return;  // uniform over the workgroup

  // The readout pairs each diagonal block of M with the block to its right,
  // which the prep waves never write: clear those two blocks once.
  for (int idx = tid; idx < 2 * 2 * 256; idx += 256) {
    const int b = idx >> 9, blk2 = (idx >> 8) & 1, e = idx & 255;
    sm.buf[b].m[32 * blk2 + (e >> 4)][32 * blk2 + 16 + (e & 15)] = (__bf16)0.f;
  }
  if (tid == 0) {
    sm.prep_cnt = 0;
    sm.inv_cnt = 0;
    sm.nrm_cnt = 0;
  }
  lds_barrier();

  if (wave >= 2) {
    if (wave == 2) pair_prep<DK, 0, FUSED, NORM>(p, sm, start, end, nch, gq, gk, gv, h);
    else pair_prep<DK, 1, FUSED, NORM>(p, sm, start, end, nch, gq, gk, gv, h);
    return;
  }

  // ------------------------------------------------------------ state waves
  const int w = wave;  // value columns 32w .. 32w + 31 of the slice
  const int ta = x & 3, te = x >> 2;  // transposing-read block of this lane
  f4 S[NKT][2];
#pragma unroll
  for (int j = 0; j < NKT; ++j) S[j][0] = S[j][1] = f4{0.f, 0.f, 0.f, 0.f};
  if (ibase >= 0) {
#pragma unroll
    for (int j = 0; j < NKT; ++j)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        S[j][ct] = *reinterpret_cast<const f4*>(p.init + ibase + (int64_t)(32 * w + 16 * ct + x) * DK +
                                                dk_of<NKT>(j, 4 * g));
  }
  const int ost = (int)p.o_st;

  for (int c = -1; c < nch; ++c) {
    if (c >= 0) {
      const typename Sm::Buf& B = sm.buf[c & 1];
      // ---- (I + A_ii)^-1 for blocks 2w, 2w+1; the other wave does the rest
      pair_tri_inverse<Sm::LDT>(sm.adiag[c & 1], sm.tinv, 2 * w, lane);
      if (lane == 0) __hip_atomic_fetch_add(&sm.inv_cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      // ---- R_K = K S0 and R_Q^T = S0^T Q^T (the state rounded to bf16; the
      // same fragments serve as B operand for R_K and as A operand for R_Q^T)
      bf8 Sb[NPP][2];
#pragma unroll
      for (int pp = 0; pp < NPP; ++pp)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) Sb[pp][ct] = cat8(to_bf4(S[2 * pp][ct]), to_bf4(S[2 * pp + 1][ct]));
      f4 rq[4][2], rk[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) rq[i][0] = rq[i][1] = rk[i][0] = rk[i][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < NPP; ++pp) {
        bf8 aq[4], ak[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * i + x;
          aq[i] = lds_b128(&B.q[row][8 * pair_swz(row, 4 * pp + g)]);
          ak[i] = lds_b128(&B.k[row][8 * pair_swz(row, 4 * pp + g)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            rq[i][ct] = mfma32(rq[i][ct], Sb[pp][ct], aq[i]);
            rk[i][ct] = mfma32(rk[i][ct], ak[i], Sb[pp][ct]);
          }
      }
      // ---- X = beta V - beta Gam R_K ; Y^T = scale R_Q^T Gam
      f4 X[4][2], Y[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f4 bt = *reinterpret_cast<const f4*>(&B.bet[16 * i + 4 * g]);
        const f4 gb = *reinterpret_cast<const f4*>(&B.gb[16 * i + 4 * g]);
        const float gs = B.gs[16 * i + x];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const f4 vv = bf4_to_f4(lds_tr(&B.v[16 * i + 4 * g + te][32 * w + 16 * ct + 4 * ta]));
          X[i][ct] = bt * vv - gb * rk[i][ct];
          Y[i][ct] = gs * rq[i][ct];
        }
      }
      // ---- (I + A) U = X by block forward substitution; Y += M U; state update
      const float gC = B.gC;
#pragma unroll
      for (int j = 0; j < NKT; ++j) {
        S[j][0] = gC * S[j][0];
        S[j][1] = gC * S[j][1];
      }
      const bf4 zero4 = bf4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
      // operands of the substitution chain, read before it starts (the
      // other state wave inverts every chunk too, so the wait for its
      // blocks ends; its bound only guards against a wave that never arrives)
      for (int spin = 0; spin < (1 << 22); ++spin) {
        if (__hip_atomic_load(&sm.inv_cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= 2 * (c + 1)) break;
        __builtin_amdgcn_s_sleep(1);
      }
      bf4 tiv[4], na[4][4];
      f4 dcs[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        tiv[m] = lds_b64(&sm.tinv[m][x][4 * g]);
        dcs[m] = *reinterpret_cast<const f4*>(&B.dc[16 * m + 4 * g]);
#pragma unroll
        for (int i = m + 1; i < 4; ++i) na[i][m] = lds_b64(&B.negA[16 * i + x][16 * m + 4 * g]);
      }
      // K^T fragments for the state update of token blocks (m0, m0+1): read
      // one pair ahead of its use
      auto load_kt = [&](int m0, bf8* kt) {
#pragma unroll
        for (int j = 0; j < NKT; ++j) {
          const int key = 32 * (j >> 1) + 8 * ta + 4 * (j & 1);
          const int r0 = 16 * m0 + 4 * g + te, r1 = r0 + 16;
          kt[j] = cat8(lds_tr(&B.k[r0][8 * pair_swz(r0, key >> 3) + 4 * (j & 1)]),
                       lds_tr(&B.k[r1][8 * pair_swz(r1, key >> 3) + 4 * (j & 1)]));
        }
      };
      bf8 kt01[NKT], kt23[NKT];
      load_kt(0, kt01);
      bf4 Ub[4][2], DU[4][2];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m == 1) load_kt(2, kt23);
        const bf4 ti = tiv[m];
        const f4 dcv = dcs[m];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const f4 U = mma_k16(f4{0.f, 0.f, 0.f, 0.f}, ti, to_bf4(X[m][ct]));
          Ub[m][ct] = to_bf4(U);
          DU[m][ct] = to_bf4(dcv * U);
        }
        if ((m & 1) == 0) {
          const bf4 a = na[m + 1][m];
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
            X[m + 1][ct] = mfma32(X[m + 1][ct], cat8(a, zero4), cat8(Ub[m][ct], zero4));
        } else {
          const int m0 = m - 1;
#pragma unroll
          for (int i = m + 1; i < 4; ++i) {
            const bf8 a = cat8(na[i][m0], na[i][m]);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) X[i][ct] = mfma32(X[i][ct], a, cat8(Ub[m0][ct], Ub[m][ct]));
          }
#pragma unroll
          for (int i = m0; i < 4; ++i) {
            const bf8 a = cat8(lds_b64(&B.m[16 * i + x][16 * m0 + 4 * g]),
                               lds_b64(&B.m[16 * i + x][16 * m + 4 * g]));
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) Y[i][ct] = mfma32(Y[i][ct], cat8(Ub[m0][ct], Ub[m][ct]), a);
          }
#pragma unroll
          for (int j = 0; j < NKT; ++j) {
            const bf8 a = m0 == 0 ? kt01[j] : kt23[j];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) S[j][ct] = mfma32(S[j][ct], a, cat8(DU[m0][ct], DU[m][ct]));
          }
        }
      }
      // ---- outputs (scale is folded into Gam and M)
      const int64_t tok0 = start + (int64_t)c * C;
      const int nvalid = (int)min((int64_t)C, end - tok0);
      __bf16* ob = gout + tok0 * p.o_st + 32 * w;
      if (nvalid == C) {
        // Y^T tiles: lane (x, g) holds columns 16 ct + 4 g .. +3 of token
        // 16 i + x.  Swapping rows 1, 3 of the ct = 0 tile with rows 0, 2 of
        // the ct = 1 tile (v_permlane16_swap) leaves each lane 8 consecutive
        // columns, 16 ct' + 8 g' .. +7 with ct' = g & 1, g' = g >> 1.
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(ob);
        const uint32_t o_lane = (uint32_t)((x * ost + 16 * (g & 1) + 8 * (g >> 1)) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x2 p0 = __builtin_bit_cast(u32x2, to_bf4(Y[i][0]));
          const u32x2 p1 = __builtin_bit_cast(u32x2, to_bf4(Y[i][1]));
          const auto s0 = __builtin_amdgcn_permlane16_swap(p0[0], p1[0], false, false);
          const auto s1 = __builtin_amdgcn_permlane16_swap(p0[1], p1[1], false, false);
          __builtin_amdgcn_raw_buffer_store_b128((u32x4){s0[0], s1[0], s0[1], s1[1]}, rs, o_lane,
                                                 (uint32_t)(16 * i * ost * 2), 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const int t = 16 * i + x;
            if (t < nvalid) *reinterpret_cast<bf4*>(ob + (int64_t)t * ost + 16 * ct + 4 * g) = to_bf4(Y[i][ct]);
          }
      }
    }
    lds_barrier();
  }
  if (fbase >= 0) {
#pragma unroll
    for (int j = 0; j < NKT; ++j)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        *reinterpret_cast<f4*>(p.fin + fbase + (int64_t)(32 * w + 16 * ct + x) * DK + dk_of<NKT>(j, 4 * g)) =
            S[j][ct];
  }
}

// Whether the pair kernel covers a bf16 problem of this shape and chunk hint.
inline bool prefill_pair_supported(int dk, int dv, int chunk_hint) {
  return (dk == 64 || dk == 128) && (dv == 64 || dv == 128) && (chunk_hint == 0 || chunk_hint == 64);
}

template <int DK>
hipError_t launch_prefill_pair_t(PrefillParams p, hipStream_t stream) {
  p.nsplit = p.dv / 64;
  const int64_t nblk = (int64_t)p.n_seqs * p.hv * p.nsplit;
  const dim3 grid((unsigned)nblk), block(256);
  const bool fused = p.ga || p.gb;
  if (fused && p.qk_norm) hipLaunchKernelGGL((prefill_pair_kernel<DK, true, true>), grid, block, 0, stream, p);
  else if (fused) hipLaunchKernelGGL((prefill_pair_kernel<DK, true, false>), grid, block, 0, stream, p);
  else if (p.qk_norm) hipLaunchKernelGGL((prefill_pair_kernel<DK, false, true>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((prefill_pair_kernel<DK, false, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t prefill_pair_bf16(PrefillParams p, int dk, hipStream_t s);

}  // namespace gdn
