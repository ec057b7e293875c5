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
//    each state wave inverts all four unit-lower diagonal blocks I + A_ii
//    of chunk c itself (right-looking, one lane per row, row k of A_ii
//    broadcast from its owner lane by DPP), so the two waves never wait
//    for each other; both then run [Q; K] S0, the block forward
//    substitution, Y += M U and
//    the state update; they accumulate the outputs transposed (Y^T, the
//    MFMA operands swapped), so each lane holds 4 columns of one token and,
//    after a lane swap between 16-lane rows, stores 16-byte row pieces
//    straight to memory;
//  * prep waves 2 and 3 prepare chunk c+1 meanwhile.  Each loads half of the
//    chunk's Q, K and V rows (two chunks ahead: token-strided loads have a
//    long latency; whole 16-byte row pieces, unconditionally, through buffer
//    loads whose range check zeroes rows past the request, in three batches
//    -- gates and V, Q, K -- placed between the wave's compute phases so the
//    waits for one batch never stall the next) and stages them in LDS;
//    after an LDS counter shows both
//    halves written, each computes two diagonal and three off-diagonal
//    16x16 Gram tiles, their M and -A blocks (the decay D(t,s) of an
//    off-diagonal tile factored into three per-tile factors <= 1 unless the
//    chunk holds a gamma of exactly 0), and the fp32 rows of its two
//    diagonal blocks A_ii; wave 2 also writes the per-token factors;
//  * one workgroup barrier per chunk: the state waves read buffer c & 1 while
//    the prep waves fill buffer (c+1) & 1;
//  * the multi-request walk (MULTI, its own instantiation): a workgroup runs
//    a run of consecutive short requests of one (value head, slice) as one
//    chunk stream, the state swapped at each request boundary, so the
//    kernel's start is paid once per workgroup (see pair_multi_walk);
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
  // (I + A_ii)^-1 of the current chunk, bf16: one copy per state wave, each
  // computed by that wave alone
  alignas(16) __bf16 tinv[2][NT][16][LDT];
  int prep_cnt;  // staging halves written by the prep waves so far
  int nrm_cnt;   // norm halves written by the prep waves so far (L2 norm only)
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

// One prep wave's half of a chunk, as loaded from global memory: Q and K rows
// 32pw .. 32pw+31 as whole rows, DK/8 lanes per row (load u: row 32pw +
// RPL u + lane / (DK/8), 16-byte slot lane % (DK/8), RPL = 512 / DK rows per
// load), so each load covers whole 128-byte lines; V rows 32pw .. 32pw+31
// (row 32pw + 8u + lane/8, columns 8 (lane % 8) .. +7); the gate of token
// `lane`.
template <int DK>
struct PairPrepSet {
  static constexpr int NLD = DK / 16;  // loads of whole rows per operand
  u32x4 q[NLD];
  u32x4 k[NLD];
  u32x4 v[4];
  float gd, bt;      // decay and beta of token `lane` as loaded (clamped to the chunk)
  __bf16 ga, gbr;    // or the fused gate's raw a and b
};

// acc[j] += row K's arow[j] * nt for the listed j, one fused DPP
// multiply-add each (v_fmac_f32_dpp with row_newbcast:K, which reads the
// operand from lane K of the lane's 16-lane row).  The compiler does not see
// the DPP read inside the asm, so it cannot insert the 2 wait states a DPP
// read needs after a VALU write of its source.  None is needed: the DPP
// sources are the rows of A as read from LDS, which no VALU instruction
// writes (a test scans the kernels' assembly for such a write).
template <int K>
__device__ __forceinline__ void fmac_bcast1(float& a0, float b0, float nt) {
  asm volatile(
      "v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(a0)
      : "v"(b0), "v"(nt), "n"(K));
}
template <int K>
__device__ __forceinline__ void fmac_bcast4(float& a0, float& a1, float& a2, float& a3, float b0, float b1, float b2,
                                            float b3, float nt) {
  asm volatile(
      "v_fmac_f32_dpp %0, %4, %8 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %5, %8 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %6, %8 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %7, %8 row_newbcast:%9 row_mask:0xf bank_mask:0xf"
      : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)
      : "v"(b0), "v"(b1), "v"(b2), "v"(b3), "v"(nt), "n"(K));
}

// One right-looking step of pair_tri_inverse4 and the steps below it: with
// t = T[r][K] final, T[r][j] -= t A[K][j] for every j < K, where A[K][j] is
// row K's value held by lane K of this lane's 16-lane row.  The entry step
// K-1 reads first is updated first.
template <int K>
__device__ __forceinline__ void tri_inverse_steps(float (&acc)[16], const float (&arow)[16]) {
  const float nt = -acc[K];
  // the order of updates: K-1, then 0 .. K-2
  constexpr int NG = K / 4;  // full groups of four
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    auto jj = [](int i) { return i == 0 ? K - 1 : i - 1; };
    const int j0 = jj(4 * gi), j1 = jj(4 * gi + 1), j2 = jj(4 * gi + 2), j3 = jj(4 * gi + 3);
    fmac_bcast4<K>(acc[j0], acc[j1], acc[j2], acc[j3], arow[j0], arow[j1], arow[j2], arow[j3], nt);
  }
#pragma unroll
  for (int i = 4 * NG; i < K; ++i) {
    const int j = i == 0 ? K - 1 : i - 1;
    fmac_bcast1<K>(acc[j], arow[j], nt);
  }
  if constexpr (K > 1) tri_inverse_steps<K - 1>(acc, arow);
}

// Inverses of the four unit-lower diagonal blocks I + A_i of a chunk (A_i
// strictly lower, fp32 rows in `ad` as the prep waves lay them out: row k of
// block i at ad[i][20 k ..], A_i[k][j] at 20 k + 8 (j & 1) + (j >> 1)).
// Lane l owns row r = l % 16 of block i = l / 16 -- block i is DPP row i --
// holding row r of A_i and row r of T_i = (I + A_i)^-1 in registers.
// Right-looking: T[r][j] = [j == r] - sum_{k > j} T[r][k] A[k][j]; with k
// falling from 15, T[r][k] is final when step k reads it (entries k > r
// stay 0: T is lower triangular), and row k of A comes from lane k by a DPP
// broadcast, so the steps touch neither LDS nor other rows' registers.
// Writes row r of T_i in bf16 to tout[i][r][0..15].
template <int LDT>
__device__ __forceinline__ void pair_tri_inverse4(const float (*ad)[16 * 20 + 4], __bf16 (*tout)[16][LDT],
                                                  int lane) {
  const int i = lane >> 4, r = lane & 15;
  const float* a = &ad[i][20 * r];
  const f4 e0 = *reinterpret_cast<const f4*>(a);       // A[r][0, 2, 4, 6]
  const f4 e1 = *reinterpret_cast<const f4*>(a + 4);   // A[r][8, 10, 12, 14]
  const f4 o0 = *reinterpret_cast<const f4*>(a + 8);   // A[r][1, 3, 5, 7]
  const f4 o1 = *reinterpret_cast<const f4*>(a + 12);  // A[r][9, 11, 13, 15]
  float arow[16], acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int jj = j >> 1;
    arow[j] = (j & 1) ? (jj < 4 ? o0[jj] : o1[jj - 4]) : (jj < 4 ? e0[jj] : e1[jj - 4]);
    acc[j] = j == r ? 1.f : 0.f;
  }
  tri_inverse_steps<15>(acc, arow);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<bf4*>(&tout[i][r][4 * q]) = to_bf4(f4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]});
}

// Prep wave PW of the pair kernel (see the header comment).  FUSED: the gates
// come from A_log, dt_bias, a, b (computed here); NORM: the in-kernel q/k L2
// norm.  Each combination is its own instantiation, so none carries branches
// for the options it does not use.
// Multi-request walk: a workgroup takes up to kMultiMax consecutive requests
// for one (value head, slice) and runs their chunks as one stream, request
// after request (each request's chunks start at its own first token).  The
// group's token ranges sit in LDS (mt[i] start, mt[kMultiMax + i] end of the
// group's request i); a cursor (request, chunk) walks the stream, skipping
// empty requests.
constexpr int kMultiMax = 64;
struct PairCursor {
  int r, c;
};
__device__ __forceinline__ int multi_nch(const int64_t* mt, int i) {
  return (int)((mt[kMultiMax + i] - mt[i] + 63) / 64);
}
__device__ __forceinline__ int multi_next(const int64_t* mt, int nreq, int i) {
  do ++i;
  while (i < nreq && multi_nch(mt, i) == 0);
  return i;
}
__device__ __forceinline__ void multi_advance(const int64_t* mt, int nreq, PairCursor& u) {
  if (u.r >= nreq) return;
  if (++u.c >= multi_nch(mt, u.r)) {
    u.c = 0;
    u.r = multi_next(mt, nreq, u.r);
  }
}
// Chunk at the cursor: first token and row count (have false past the end).
__device__ __forceinline__ void multi_chunk(const int64_t* mt, int nreq, const PairCursor& u, bool& have,
                                            int64_t& t0, int& rem) {
  have = u.r < nreq;
  t0 = have ? mt[u.r] + (int64_t)u.c * 64 : 0;
  rem = have ? (int)min((int64_t)64, mt[kMultiMax + u.r] - t0) : 0;
}

template <int DK, int PW, bool FUSED, bool NORM, bool MULTI>
__device__ __forceinline__ void pair_prep(const PrefillParams& p, PairSmem<DK>& sm, int64_t start,
                                          int64_t end, int nch, const __bf16* gq, const __bf16* gk,
                                          const __bf16* gv, int v_st, int h, const int64_t* mt, int nreq) {
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

  // Loads chunk c into `s`: always the same 22 buffer loads, whether or not
  // the chunk exists, so that the compiler counts the loads in flight
  // exactly -- a branch around them makes that count conservative, and then
  // every iteration waits for the other set's loads too.  Every offset is in
  // the VGPR offset, which the buffer range check covers: rows past the
  // chunk's last token, and every row of a chunk past the request
  // (num_records 0), read zeros without touching memory.  The values are
  // kept exactly as loaded: nothing here may wait on these loads (padding
  // and the fused gate are applied when the set is staged).
  auto prefetch_at = [&](bool have, int64_t t0, int rem, PairPrepSet<DK>& s, int part) {
    rem = have ? rem : 1;  // rows of the chunk
    const int qst = (int)p.q_st, kst = (int)p.k_st, vst = v_st;
    auto rsrc = [&](const void* base, int bytes) { return buf_rsrc_n(base, have ? (uint32_t)bytes : 0u); };
    if (part == 0) {
      const uint32_t toff = (uint32_t)(min(lane, rem - 1) * p.hv);  // token `lane`, clamped to the chunk
      if constexpr (FUSED) {
        s.ga = buf_load<__bf16>(rsrc(gga + ((t0 * p.hv) & p.dmask), -1), (toff & (uint32_t)p.dmask) * 2, 0);
        s.gbr = buf_load<__bf16>(rsrc(ggb + ((t0 * p.hv) & p.bmask), -1), (toff & (uint32_t)p.bmask) * 2, 0);
      } else {
        s.gd = buf_load<float>(rsrc(gdec + ((t0 * p.hv) & p.dmask), -1), (toff & (uint32_t)p.dmask) * 4, 0);
        s.bt = buf_load<float>(rsrc(gbet + ((t0 * p.hv) & p.bmask), -1), (toff & (uint32_t)p.bmask) * 4, 0);
      }
    }
    // in range: the bytes up to the end of row rem - 1
    const __amdgpu_buffer_rsrc_t rq = rsrc(gq + t0 * p.q_st, ((rem - 1) * qst + DK) * 2);
    const __amdgpu_buffer_rsrc_t rk = rsrc(gk + t0 * p.k_st, ((rem - 1) * kst + DK) * 2);
    const __amdgpu_buffer_rsrc_t rv = rsrc(gv + t0 * v_st, ((rem - 1) * vst + 64) * 2);
#pragma unroll
    for (int u = 0; u < DK / 16; ++u) {
      const int row = 32 * PW + (512 / DK) * u + lane / (DK / 8), slot = lane % (DK / 8);
      if (part == 1) s.q[u] = buf_load16(rq, (uint32_t)((row * qst + 8 * slot) * 2), 0);
      if (part == 2) s.k[u] = buf_load16(rk, (uint32_t)((row * kst + 8 * slot) * 2), 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (part == 0)
        s.v[u] = buf_load16(rv, (uint32_t)(((32 * PW + 8 * u + (lane >> 3)) * vst + 8 * (lane & 7)) * 2), 0);
  };
  // chunk c of the request (single-request walk), or the prefetch cursor's
  // chunk (multi-request walk; the cursor moves on once per iteration)
  PairCursor cp{0, 0}, cs{0, 0};
  if constexpr (MULTI) {
    cp.r = mt[0 + kMultiMax] > mt[0] ? 0 : multi_next(mt, nreq, 0);
    cs = cp;
  }
  bool hp = false;
  int64_t tp = 0;
  int rp = 0;
  auto prefetch = [&](int c, PairPrepSet<DK>& s, int part) {
    if constexpr (MULTI) {
      prefetch_at(hp, tp, rp, s, part);
    } else {
      const bool have = c < nch;
      const int64_t t0 = start + (int64_t)(have ? c : 0) * C;
      prefetch_at(have, t0, have ? (int)min((int64_t)C, end - t0) : 1, s, part);
    }
  };
  auto next_prefetch_chunk = [&]() {
    if constexpr (MULTI) {
      multi_chunk(mt, nreq, cp, hp, tp, rp);
      multi_advance(mt, nreq, cp);
    }
  };

  auto frag_col = [&](int row, int pp) -> int { return 8 * pair_swz(row, 4 * pp + g); };

  int staged = 0;  // chunks staged by this wave so far
  // One iteration: prepare chunk c+1 from `s`, and refill `s` with chunk c+3
  // in three batches spread over the iteration (gates and V, then Q, then K),
  // so that each batch finds the memory pipeline with room and the wave does
  // not stall issuing 22 loads at once.  The iteration has no branches: past
  // the request's last chunk it runs on zeros (the loads of a missing chunk
  // read zeros) into the buffer no state wave reads any more.  Loads behind a
  // branch make the compiler's count of loads in flight conservative (every
  // iteration would then wait for the other set's loads too), and loads on
  // two paths get different registers and copies that wait for them.
  auto iter = [&](int c, PairPrepSet<DK>& s) {
    float gd = 0.f, btl = 0.f;
    {
      typename Sm::Buf& B = sm.buf[(c + 1) & 1];
      // ---- stage this wave's half
#pragma unroll
      for (int u = 0; u < DK / 16; ++u) {
        const int r = 32 * PW + (512 / DK) * u + lane / (DK / 8), slot = lane % (DK / 8);
        *reinterpret_cast<u32x4*>(&B.q[r][8 * pair_swz(r, slot)]) = s.q[u];
        *reinterpret_cast<u32x4*>(&B.k[r][8 * pair_swz(r, slot)]) = s.k[u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<u32x4*>(&B.v[32 * PW + 8 * u + (lane >> 3)][8 * (lane & 7)]) = s.v[u];
      // gates of token `lane`; padded tokens: no decay (log-decay 0 / gamma
      // 1) and beta 0
      int srows;
      if constexpr (MULTI) {
        bool hs;
        int64_t ts;
        multi_chunk(mt, nreq, cs, hs, ts, srows);
        multi_advance(mt, nreq, cs);
      } else {
        srows = (int)min((int64_t)C, end - (start + (int64_t)(c + 1) * C));
      }
      const bool live = lane < srows;
      if constexpr (FUSED) {  // an absent input: no decay, beta 1
        gd = live && p.dmask ? gate_log_decay_fast(ealog, dtb, (float)s.ga) : 0.f;
        btl = live ? (p.bmask ? sigmoid_fast((float)s.gbr) : 1.f) : 0.f;
      } else {
        gd = live ? s.gd : (p.decay_is_gamma ? 1.f : 0.f);
        btl = live ? s.bt : 0.f;
      }
      // ---- signal this half written; the wait for the other prep wave's
      // half comes after the scan.  Both prep waves stage every chunk, so
      // that wait ends; its bound only guards against a wave that never
      // arrives.
      ++staged;
      if (lane == 0) __hip_atomic_fetch_add(&sm.prep_cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    next_prefetch_chunk();
    prefetch(c + 3, s, 0);
    {
      typename Sm::Buf& B = sm.buf[(c + 1) & 1];
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
      prefetch(c + 3, s, 1);
      wait_lds_count(&sm.prep_cnt, 2 * staged, p.wait_err);
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
      prefetch(c + 3, s, 2);
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
        wait_lds_count(&sm.nrm_cnt, 2 * staged, p.wait_err);
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

  // Two iterations per trip, both always run; iteration c prepares chunk
  // c + 1, so the trips end once chunk nch - 1 is prepared: nch + (nch & 1)
  // barriers in all (one iteration on a chunk past the request when nch is
  // odd), matched by the state waves.
  // The two first sets load in the loop's order (no instruction scheduled
  // across), so the loop head's wait for `sa` leaves `sb` in flight.
  PairPrepSet<DK> sa, sb;
  next_prefetch_chunk();
  for (int part = 0; part < 3; ++part) prefetch(0, sa, part);
  __builtin_amdgcn_sched_barrier(0);
  next_prefetch_chunk();
  for (int part = 0; part < 3; ++part) prefetch(1, sb, part);
  for (int c = -1; c < nch - 1; c += 2) {
    iter(c, sa);
    iter(c + 1, sb);
  }
}

// The state waves' side of the multi-request walk.  Every request's chunks
// run as in the single-request walk; at a request's first chunk the state
// becomes its initial state, after its last chunk the state is stored to
// its final slot.  The pool rules hold per request: a request whose read
// slot is outside the pool is skipped under kPoolSkipUnread (no outputs, no
// store; its chunks are still prepared), and an empty request's final state
// is its initial state.  States move through buffer descriptors whose
// range is 0 for a slot outside the pool (such loads read zeros and move no
// data).  The load is not hidden: holding the next request's state in a
// second register set for a chunk made the chunks slower than the load it
// hid.
template <int DK, typename Body>
__device__ __forceinline__ void pair_multi_walk(const PrefillParams& p, const int64_t* mt, int nreq, int rg0,
                                                int h, int v0, int nch, int w, int lane, f4 (&S)[DK / 16][2],
                                                Body& chunk_body) {
  constexpr int NKT = DK / 16;
  constexpr uint32_t kSlice = 64u * DK * 4u;  // bytes of a 64-row state slice
  const int x = lane & 15, g = lane >> 4;
  auto off = [&](int jj, int ct) {
    return (uint32_t)(((32 * w + 16 * ct + x) * DK + dk_of<NKT>(jj, 4 * g)) * 4);
  };
  auto load_state = [&](f4 (&D)[NKT][2], int64_t ib) {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc_n(p.init + (ib >= 0 ? ib : 0), ib >= 0 ? kSlice : 0u);
#pragma unroll
    for (int jj = 0; jj < NKT; ++jj)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) D[jj][ct] = __builtin_bit_cast(f4, buf_load16(rs, off(jj, ct), 0));
  };
  auto store_state = [&](int64_t fb) {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc_n(p.fin + (fb >= 0 ? fb : 0), fb >= 0 ? kSlice : 0u);
#pragma unroll
    for (int jj = 0; jj < NKT; ++jj)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, S[jj][ct]), rs, off(jj, ct), 0, 0);
  };
  auto skipped = [&](int64_t ib) { return (p.pool_flags & kPoolSkipUnread) && ib < 0; };
  for (int i = 0; i < nreq; ++i) {
    if (multi_nch(mt, i) != 0) continue;
    int64_t ib, fb;
    prefill_state_offsets(p, rg0 + i, h, v0, DK, ib, fb);
    if (skipped(ib) || fb < 0) continue;
    load_state(S, ib);
    store_state(fb);
  }
  PairCursor u{0, 0};
  u.r = multi_nch(mt, 0) > 0 ? 0 : multi_next(mt, nreq, 0);
  int64_t ib_cur = -1, fb_cur = -1;
  bool skip = false;
  const int nbar = nch + (nch & 1);  // as the prep waves run them
  for (int c = -1; c < nbar; ++c) {
    if (c >= 0 && c < nch) {
      const bool last = u.c == multi_nch(mt, u.r) - 1;
      if (u.c == 0) {
        prefill_state_offsets(p, rg0 + u.r, h, v0, DK, ib_cur, fb_cur);
        skip = skipped(ib_cur);
        load_state(S, ib_cur);
      }
      const int64_t tok0 = mt[u.r] + (int64_t)u.c * 64;
      if (!skip) chunk_body(c, tok0, (int)min((int64_t)64, mt[kMultiMax + u.r] - tok0));
      if (last && !skip && fb_cur >= 0) store_state(fb_cur);
      multi_advance(mt, nreq, u);
    }
    if (c < nbar - 1) lds_barrier();
  }
}

template <int DK, bool FUSED, bool NORM, bool SEG, bool MULTI>
__global__ void __launch_bounds__(256, 1)
prefill_pair_kernel(const PrefillParams p) {
  typedef PairSmem<DK> Sm;
  constexpr int C = 64, NKT = DK / 16, NPP = DK / 32;
  __shared__ Sm sm;
  __shared__ int64_t mt[MULTI ? 2 * kMultiMax : 1];  // multi-request walk: the group's token ranges

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int x = lane & 15;
  const int g = lane >> 4;

  // unit (request r, segment j, value head h, slice); without segments (SEG
  // false, an instantiation of its own) j = 0 and every slice is a value slice
  const int blk = prefill_block_unit(blockIdx.x, gridDim.x, p.nsplit * max(p.hv / p.hq, 1), p.lpt);
  const int split = blk % p.nsplit;
  const int h = (blk / p.nsplit) % p.hv;
  const int kj = blk / (p.nsplit * p.hv);  // (rank, segment), or the request group
  const int j = SEG ? kj % p.nseg : 0;
  // multi-request walk: requests rg0 .. rg0 + nreq - 1
  const int rg0 = MULTI ? kj * p.rgroup : 0;
  const int nreq = MULTI ? min(p.rgroup, p.n_seqs - rg0) : 1;
  const int r = MULTI ? rg0 : prefill_request_of_rank(p, SEG ? kj / p.nseg : kj, reinterpret_cast<int*>(&sm.buf[1].q[0][0]));
  const int rj = SEG ? r * p.nseg + j : r;  // the unit's workspace index
  const int qh = (int)(((int64_t)h * p.hq) / p.hv);
  const bool trans = SEG && split >= p.nsv;  // transition slice of a local pass
  const int v0 = (trans ? split - p.nsv : split) * 64;

  int64_t start, end;
  prefill_request_bounds(p, r, start, end);
  if constexpr (SEG) prefill_segment_bounds(p.nseg, j, C, start, end);
  int nch = (int)((end - start + C - 1) / C);
  if constexpr (MULTI) {
    if (tid < nreq) {
      int64_t s0, s1;
      prefill_request_bounds(p, rg0 + tid, s0, s1);
      mt[tid] = s0;
      mt[kMultiMax + tid] = s1;
    }
  }

  const __bf16* __restrict__ gq = (const __bf16*)p.q + (int64_t)qh * p.q_sh;
  const __bf16* __restrict__ gk = (const __bf16*)p.k + (int64_t)qh * p.k_sh;
  // a transition slice reads V as zeros: every row from the same 128 zero bytes
  const __bf16* __restrict__ gv = trans ? (const __bf16*)p.vzero : (const __bf16*)p.v + (int64_t)h * p.v_sh + v0;
  const int v_st = trans ? 0 : (int)p.v_st;
  __bf16* __restrict__ gout = (__bf16*)p.out + (int64_t)h * p.o_sh + v0;
  int64_t ibase, fbase;
  if (SEG && p.seg_mode == 1) {
    // value slices: V-major rows v0.. of the segment's state; transition
    // slices: the dk x dk transition block, stored K-major (see below)
    ibase = -1;
    fbase = (((int64_t)rj * p.hv + h) * (p.dv + DK) + (trans ? p.dv : v0)) * DK;
  } else if (SEG) {  // seg_mode 2
    ibase = (((int64_t)rj * p.hv + h) * p.dv + v0) * DK;
    fbase = -1;
  } else {
    prefill_state_offsets(p, r, h, v0, DK, ibase, fbase);
  }
  if (!MULTI && (p.pool_flags & kPoolSkipUnread) && ibase < 0) return;  // uniform over the workgroup

  // The readout pairs each diagonal block of M with the block to its right,
  // which the prep waves never write: clear those two blocks once.
  for (int idx = tid; idx < 2 * 2 * 256; idx += 256) {
    const int b = idx >> 9, blk2 = (idx >> 8) & 1, e = idx & 255;
    sm.buf[b].m[32 * blk2 + (e >> 4)][32 * blk2 + 16 + (e & 15)] = (__bf16)0.f;
  }
  if (tid == 0) {
    sm.prep_cnt = 0;
    sm.nrm_cnt = 0;
  }
  lds_barrier();
  if constexpr (MULTI) {
    // the stream's chunk count
    nch = 0;
    for (int i = 0; i < nreq; ++i) nch += multi_nch(mt, i);
  }

  if (wave >= 2) {
    if (wave == 2) pair_prep<DK, 0, FUSED, NORM, MULTI>(p, sm, start, end, nch, gq, gk, gv, v_st, h, mt, nreq);
    else pair_prep<DK, 1, FUSED, NORM, MULTI>(p, sm, start, end, nch, gq, gk, gv, v_st, h, mt, nreq);
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
  } else if (trans) {
    // the key identity: row i = v0 + column of the V-major state is e_i
#pragma unroll
    for (int j = 0; j < NKT; ++j)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          S[j][ct][e] = dk_of<NKT>(j, 4 * g) + e == v0 + 32 * w + 16 * ct + x ? 1.f : 0.f;
  }
  const bool store_out = !SEG || p.seg_mode != 1;
  const int ost = (int)p.o_st;

  // nch + (nch & 1) barriers, as the prep waves run them in pairs; the last
  // chunk needs none after it (no buffer is written any more)
  const int nbar = nch + (nch & 1);
  // One chunk of the state waves: c is the chunk's place in the stream (its
  // buffer parity), tok0 its first token, nvalid its rows to store.
  auto chunk_body = [&](int c, int64_t tok0, int nvalid) {
      const typename Sm::Buf& B = sm.buf[c & 1];
      // ---- (I + A_ii)^-1 of the four diagonal blocks, this wave's own copy
      pair_tri_inverse4<Sm::LDT>(sm.adiag[c & 1], sm.tinv[w], lane);
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
      // operands of the substitution chain, read before it starts
      bf4 tiv[4], na[4][4];
      f4 dcs[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        tiv[m] = lds_b64(&sm.tinv[w][m][x][4 * g]);
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
  };
  if constexpr (MULTI) {
    pair_multi_walk<DK>(p, mt, nreq, rg0, h, v0, nch, w, lane, S, chunk_body);
    return;
  }
  for (int c = -1; c < nbar; ++c) {
    if (c >= 0 && c < nch) {
      const int64_t tok0 = start + (int64_t)c * C;
      chunk_body(c, tok0, store_out ? (int)min((int64_t)C, end - tok0) : 0);
    }
    if (c < nbar - 1) lds_barrier();
  }
  if (SEG && fbase >= 0 && trans) {
    // transition slice: element (key k, column i) of the K-major state is
    // P[k][i]; stored at k * DK + i, so a row of the block is a key's row of P
#pragma unroll
    for (int j = 0; j < NKT; ++j)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.fin[fbase + (int64_t)(dk_of<NKT>(j, 4 * g) + e) * DK + v0 + 32 * w + 16 * ct + x] = S[j][ct][e];
  } else if (fbase >= 0) {
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
  p.nsv = p.dv / 64;
  p.nsplit = p.nsv + (p.seg_mode == 1 ? DK / 64 : 0);
  const bool multi = !p.seg_mode && p.rgroup > 1;
  const int64_t nunits = multi ? (p.n_seqs + p.rgroup - 1) / p.rgroup : (int64_t)p.n_seqs * p.nseg;
  const int64_t nblk = nunits * p.hv * p.nsplit;
  const dim3 grid((unsigned)nblk), block(256);
  const bool fused = p.ga || p.gb;
#define GDN_PAIR_LAUNCH(SEG, MULTI)                                                                            \
  if (fused && p.qk_norm) hipLaunchKernelGGL((prefill_pair_kernel<DK, true, true, SEG, MULTI>), grid, block, 0, stream, p); \
  else if (fused) hipLaunchKernelGGL((prefill_pair_kernel<DK, true, false, SEG, MULTI>), grid, block, 0, stream, p);       \
  else if (p.qk_norm) hipLaunchKernelGGL((prefill_pair_kernel<DK, false, true, SEG, MULTI>), grid, block, 0, stream, p);   \
  else hipLaunchKernelGGL((prefill_pair_kernel<DK, false, false, SEG, MULTI>), grid, block, 0, stream, p);
  if (p.seg_mode) {
    GDN_PAIR_LAUNCH(true, false)
  } else if (multi) {
    GDN_PAIR_LAUNCH(false, true)
  } else {
    GDN_PAIR_LAUNCH(false, false)
  }
#undef GDN_PAIR_LAUNCH
  return hipGetLastError();
}

hipError_t prefill_pair_bf16(PrefillParams p, int dk, hipStream_t s);

}  // namespace gdn
