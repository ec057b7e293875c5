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
// Mapping onto gfx950.  One workgroup of 8 waves owns one (request, value
// head, slice of DVS <= 64 value columns) and walks the request's chunks in
// order.  The waves are specialised and software-pipelined:
//  * state waves 0..3 each own one 16-column tile of the slice and keep their
//    part of the state in MFMA accumulators for the whole request.  For chunk
//    c they compute, entirely in registers,
//      part 1: R = [Q; K] S0 (MFMA; S0 rounded to the operand type),
//              X = beta (V - Gam R_K), Y = Gam R_Q,
//      part 2: U by block forward substitution over 16-token blocks using the
//              inverted diagonal blocks and the off-diagonal -A blocks,
//              Y += M U, the output store, S <- Gam_{C-1} S + K^T (D(C-1,.) U);
//  * prep waves 4..7 meanwhile
//      part 1: store chunk c+1 (loaded into registers one iteration earlier)
//              into the other LDS buffer -- Q, K and a transposed K -- and
//              issue the global loads of chunk c+2;
//      part 2: scan log2 gamma of chunk c+1, compute the lower-triangular
//              16x16 tiles of K K^T and Q K^T (MFMA), mask and decay them into
//              -A and M = D o (Q K^T), and invert the four unit-lower 16x16
//              diagonal blocks of I + A (fp32 forward substitution).
// Two workgroup barriers per chunk separate the parts.  Accumulator tiles
// are laid out so that they are directly the B operand of the next product
// (see the fragment notes in gdn_device.hpp), so the state chain needs no LDS
// round trip.  The key index of the state tiles is permuted (dk_of) so that
// the [Q; K] S0 product reads its A fragments as 16-byte LDS vectors.
//
// MFMA shapes: an accumulator chain never mixes 16x16x32 and 16x16x16 bf16
// MFMAs.  With this compiler a 16x16x16 MFMA issued right after a 16x16x32
// MFMA into the same accumulator was given no wait states and read a
// partially written accumulator; keeping one shape per chain avoids that.
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
  int qk_norm;      // q, k used as x * rsqrt(sum x^2 + qk_eps)
  float qk_eps;
  const float* A_log;    // fused gate when ga or gb != nullptr (decay is then log-space)
  const float* dt_bias;
  const void* ga;        // [T, hv] io dtype
  const void* gb;        // [T, hv] io dtype
  // Gate inputs a rule does not take: the decay source (decay or ga, with
  // A_log and dt_bias) and the beta source (beta or gb) are indexed through
  // these masks, all ones for a present input and 0 for an absent one, whose
  // pointer then holds a device constant: log-decay 0 (or a = 0, replaced by
  // 0 at staging), beta 1 (or b = 0, replaced by 1).
  int64_t dmask, bmask;
  float rho;             // 1: delta retrieval kept; 0: linear / gated rules
  // State pool: when pool != nullptr the states live in it (init and fin
  // then point at it too) at slot * pss + head * phs; rslot / wslot pick the
  // slots per request (see prefill_state_offsets).
  const float* pool;
  const int32_t* rslot;
  const int32_t* wslot;
  int64_t pss, phs;
  int pool_size;
  int pool_flags;        // kPoolSkipUnread | kPoolNoWrite (the decode's rules)
  // Segmented scan over chunk affine maps (pair kernel only).  seg_mode 0:
  // off (nseg 1, nsv = nsplit).  Otherwise request r is cut into nseg
  // segments of whole chunks (prefill_segment_bounds) and a workgroup runs
  // unit (r, j, h, slice) on segment j:
  //  * seg_mode 1 (local pass): value slices (slice < nsv) start from a zero
  //    state, transition slices (slice >= nsv, nsplit - nsv of them) from the
  //    key identity -- row i of their V-major state is e_i -- and read V from
  //    vzero (zeros), so their final rows are the columns of the segment's
  //    state transition P.  No outputs.  The final states go to fin as
  //    [r * nseg + j, h, dv + dk, dk]: rows < dv the segment's own state
  //    (V-major), then P itself as dk rows of dk (K-major: row k holds
  //    P[k][0 .. dk-1]).
  //  * seg_mode 2 (rerun pass): segment j starts from init
  //    [r * nseg + j, h, dv, dk]; outputs as usual; no final state.
  int nseg, nsv, seg_mode;
  const void* vzero;     // >= 128 zero bytes
  // count of in-kernel waits that ran out of polls (see gdn_wait_timeouts)
  unsigned int* wait_err;
  int lpt;  // take requests longest first (prefill_request_of_rank)
  // Pair kernel: requests per workgroup of the multi-request walk (0 or 1:
  // one request per workgroup).  Consecutive requests rgroup * i ..
  // rgroup * (i + 1) - 1 share workgroup i of each (value head, slice).
  int rgroup;
};

// Token range [start, end) of request r: cu_seqlens clamped to [0, T] (a
// decreasing pair is empty), or uniform packing.
__device__ __forceinline__ void prefill_request_bounds(const PrefillParams& p, int r, int64_t& start,
                                                       int64_t& end) {
  if (p.cu) {
    start = min(max((int64_t)p.cu[r], (int64_t)0), p.T);
    end = min(max((int64_t)p.cu[r + 1], (int64_t)0), p.T);
  } else {
    start = (int64_t)r * p.seq_len;
    end = start + p.seq_len;
  }
  if (end < start) end = start;
}

// Work unit of workgroup b of a prefill grid of nblk workgroups, as an index
// blk = (rank * hv + h) * nsplit + split (the scan's passes put the segment
// between rank and h).  Workgroups are dealt to the 8 XCDs round-robin by
// block index, and the `group` consecutive units that read one query/key
// head (group = nsplit * hv / hq) always stay on one XCD, where they share
// its L2.  spread (requests of different lengths, taken longest first):
// consecutive groups go to different XCDs, so every request is spread over
// the whole chip -- one request's workgroups on one XCD would leave the
// others idle when it is the long one.  Otherwise each XCD takes a
// contiguous eighth of the units (measured faster for many short, equal
// requests).  Identity when nblk does not divide evenly.
__device__ __forceinline__ int prefill_block_unit(int b, int nblk, int group, bool spread) {
  const int x = b & 7, l = b >> 3;
  if (spread) {
    if (group > 0 && nblk % (8 * group) == 0) return ((l / group) * 8 + x) * group + l % group;
  } else if ((nblk & 31) == 0) {
    return x * (nblk >> 3) + l;
  }
  return b;
}

// Requests are taken longest first (list scheduling): the units of rank k
// belong to the k-th longest request (ties: lower index first), so the
// workgroups that run longest start in the first dispatch round and short
// ones fill the CUs that free up.  Done on the device from cu_seqlens when
// the host set lpt (2 to kLptMax requests averaging at least kLptMinTokens
// tokens: below that a workgroup's few chunks do not repay the extra round
// trip); identity otherwise.  Every thread of the workgroup calls it (two
// workgroup barriers when ordering); tmp is LDS scratch of kLptMax + 2 ints
// that nothing else uses until a later barrier.  The result is wave-uniform.
constexpr int kLptMax = 64;
constexpr int kLptMinTokens = 256;
__device__ __forceinline__ int prefill_request_of_rank(const PrefillParams& p, int k, int* tmp) {
  const int n = p.n_seqs;
  if (!p.lpt) return k;
  const int tid = threadIdx.x;
  if (tid <= n) tmp[tid] = (int)min(max((int64_t)p.cu[tid], (int64_t)0), p.T);
  __syncthreads();
  if (tid < n) {
    const int li = max(tmp[tid + 1] - tmp[tid], 0);
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const int lj = max(tmp[j + 1] - tmp[j], 0);
      rank += (lj > li) || (lj == li && j < tid);
    }
    if (rank == k) tmp[kLptMax + 1] = tid;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(tmp[kLptMax + 1]);
}

// Polls an LDS counter until it reaches `target`, at most 2^22 times (far
// beyond any wait of a working schedule); when the polls run out, lane 0
// adds 1 to the call's wait-expiry word and the wave goes on, so a broken
// schedule is reported instead of hanging the GPU.
__device__ __forceinline__ void wait_lds_count(int* cnt, int target, unsigned int* wait_err) {
  for (int spin = 0; spin < (1 << 22); ++spin) {
    if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
  if (__lane_id() == 0) __hip_atomic_fetch_add(wait_err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Segment j of nseg of a request's range: ceil(chunks / nseg) whole chunks of
// C tokens each (the last segments may be shorter or empty).
__device__ __forceinline__ void prefill_segment_bounds(int nseg, int j, int C, int64_t& start, int64_t& end) {
  const int64_t nch = (end - start + C - 1) / C;
  const int64_t L = (nch + nseg - 1) / nseg;
  const int64_t s0 = min(end, start + (int64_t)j * L * C);
  end = min(end, start + (int64_t)(j + 1) * L * C);
  start = s0;
}


// The per-key-decay prefill (gdn_prefill_pk.hip).
hipError_t launch_prefill_pk(const PrefillParams& p, int dk, int dv, bool bf16, hipStream_t s);

// The combine launch of the scan over segment maps (gdn_prefill_scan.hip).
hipError_t launch_scan_combine(const PrefillParams& p, int nseg, int dk, const float* ws_map, float* ws_in,
                               hipStream_t stream);

// Element offsets of the V-major state slice (request r, value head h, value
// columns from v0) to read the initial state from and to write the final
// state to; -1: none (zeros in, nothing out).  Dense states: [r, h] of
// init / fin.  Pool: the read slot (none when rslot is NULL or the entry is
// outside [0, pool_size)) and the write slot (the read slot when wslot is
// NULL; none when outside the pool).
__device__ __forceinline__ void prefill_state_offsets(const PrefillParams& p, int r, int h, int v0, int dk,
                                                      int64_t& ibase, int64_t& fbase) {
  if (p.pool) {
    const int rs = p.rslot ? p.rslot[r] : -1;
    const int ws = p.wslot ? p.wslot[r] : rs;
    const int64_t head = (int64_t)h * p.phs + (int64_t)v0 * dk;
    ibase = (rs >= 0 && rs < p.pool_size) ? (int64_t)rs * p.pss + head : -1;
    fbase = (ws >= 0 && ws < p.pool_size && !(p.pool_flags & kPoolNoWrite)) ? (int64_t)ws * p.pss + head : -1;
  } else {
    const int64_t st = (((int64_t)r * p.hv + h) * p.dv + v0) * dk;
    ibase = p.init ? st : -1;
    fbase = st;
  }
}

// LDS layout of one workgroup.
template <typename E, int DK, int DVS, int C>
struct PrefillSmem {
  static constexpr int PAD = 16 / sizeof(E);  // 16-byte row skew
  static constexpr int NT = C / 16;
  static constexpr int LDK = DK + PAD;        // Q, K rows
  static constexpr int LDC = C + PAD;         // K^T, -A, M rows
  static constexpr int LDT = 16 + PAD;        // inverse blocks
  struct Raw {       // one chunk's inputs
    E q[C][LDK];
    E k[C][LDK];
    E kt[DK][LDC];   // transposed K, 4-token groups XOR-swizzled per row
  };
  struct Derived {   // one chunk's prep results
    E negA[C][LDC];  // -A, off-diagonal 16x16 blocks only
    E m[C][LDC];     // scale * D o (Q K^T), lower-triangular blocks only
    E tinv[NT][16][LDT];
    alignas(16) float F[C];    // prefix sum of log2 gamma over non-zero gammas
    alignas(16) int z[C];      // last index <= t whose gamma is 0, or -1
    alignas(16) float bet[C];  // beta_t (0 on padded tokens)
    alignas(16) float gb[C];   // beta_t Gam_t
    alignas(16) float gs[C];   // scale Gam_t
    alignas(16) float dc[C];   // D(C-1, t)
    alignas(16) float rqn[C];  // 1 / |q_t| and 1 / |k_t| (in-kernel L2 norm only)
    alignas(16) float rkn[C];
    float gC;                  // Gam_{C-1}
    int any_zero;              // some gamma of the chunk is exactly 0
  };
  Raw raw[2];
  Derived der[2];
  // transposed fp32 diagonal blocks of A of the chunk being prepared:
  // adiagT[i][s][t] = A[16i+t][16i+s]; rows padded so the 4 blocks' rows sit
  // in different banks
  alignas(16) float adiagT[4][16][20];
};

// Row r (0..15) of state tile j holds key index dk_of(j, r).  With pairs of
// tiles, lane group g of a 32-key block holds keys 8g .. 8g+7, contiguous.
template <int NKT>
__device__ __forceinline__ int dk_of(int j, int r) {
  if constexpr (NKT % 2 == 0) return 32 * (j >> 1) + 8 * (r >> 2) + 4 * (j & 1) + (r & 3);
  else return 16 * j + r;
}

// 8 consecutive operand elements from LDS as two K16 fragments.
__device__ __forceinline__ void lds_frag8(const __bf16* p, bf4& a0, bf4& a1) {
  const bf8 v = *reinterpret_cast<const bf8*>(p);
  a0 = bf4{v[0], v[1], v[2], v[3]};
  a1 = bf4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void lds_frag8(const float* p, f4& a0, f4& a1) {
  a0 = *reinterpret_cast<const f4*>(p);
  a1 = *reinterpret_cast<const f4*>(p + 4);
}

// Element e of a 16-byte vector of E.
template <typename E> __device__ __forceinline__ E elem16(const u32x4& v, int e);
template <> __device__ __forceinline__ __bf16 elem16<__bf16>(const u32x4& v, int e) {
  const uint32_t word = v[e >> 1];
  return __builtin_bit_cast(__bf16, (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu)));
}
template <> __device__ __forceinline__ float elem16<float>(const u32x4& v, int e) {
  return __uint_as_float(v[e]);
}

// 4 elements of E packed for one LDS store.
template <typename E> struct pack4;
template <> struct pack4<__bf16> { typedef bf4 type; };
template <> struct pack4<float> { typedef f4 type; };
template <typename E>
__device__ __forceinline__ typename pack4<E>::type to_pack4(f4 v) {
  typename pack4<E>::type o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = from_f32<E>(v[e]);
  return o;
}

// EXT compiles the optional fused gate and in-kernel q/k L2 norm in (each
// still switched by its argument); without it the code has neither.
// 16-token chunks, and bf16 32-token chunks, are held to 128 VGPRs (four
// waves per SIMD), so that two workgroups share a CU: their LDS fits twice,
// and calls with many short requests (the chunked multi-token decode: one
// or two chunks per workgroup, thousands of workgroups) hide one
// workgroup's state loads and barriers behind the other's work.  The bf16
// 32-token forms spill a few registers to do so and still gain; the fp32
// 32-token form (the long ragged requests) keeps one workgroup per CU.
template <typename E, int DK, int DVS, int C, bool EXT>
__global__ void __launch_bounds__(512, (C == 16 || (C == 32 && sizeof(E) == 2)) ? 4 : 1)
prefill_kernel(const PrefillParams p) {
  typedef typename frag_of<E>::type Fr;
  typedef PrefillSmem<E, DK, DVS, C> Sm;
  constexpr int NT = C / 16;            // token tiles per chunk
  constexpr int NKT = DK / 16;          // key tiles
  constexpr int NVT = DVS / 16;         // value tiles per workgroup (<= 4)
  constexpr int VE = 16 / sizeof(E);    // elements per 16-byte vector
  constexpr int NOCT = DK / VE;         // 16-byte vectors per token row
  constexpr int NPAIR = (C / 4) * NOCT; // (4-token quad, vector) load units
  constexpr int NPT = (NPAIR + 255) / 256;
  constexpr int NOFF = NT * (NT - 1) / 2;
  static_assert(NVT <= 4, "one value tile per state wave");
  __shared__ Sm sm;
  // Transposed-K layout: token t of key row r lives at column t ^ kt_swz(r)
  // (an XOR of 4-token groups), so that the prep waves' transposed stores --
  // 16 lanes writing rows VE keys apart -- hit distinct banks.
  auto kt_swz = [](int r) { return 4 * ((r / VE) % (C / 4)); };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int x = lane & 15;   // row/column inside a 16x16 tile
  const int g = lane >> 4;   // lane group
  const bool is_prep = wave >= 4;
  const int pw = wave - 4;   // prep wave index
  const int ptid = tid - 256;

  const int blk = prefill_block_unit(blockIdx.x, gridDim.x, p.nsplit * max(p.hv / p.hq, 1), p.lpt);
  const int split = blk % p.nsplit;
  const int h = (blk / p.nsplit) % p.hv;
  const int r = prefill_request_of_rank(p, blk / (p.nsplit * p.hv), reinterpret_cast<int*>(&sm.raw[1].q[0][0]));
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

  const E* __restrict__ gq = (const E*)p.q + (int64_t)qh * p.q_sh;
  const E* __restrict__ gk = (const E*)p.k + (int64_t)qh * p.k_sh;
  const E* __restrict__ gv = (const E*)p.v + (int64_t)h * p.v_sh + v0;
  E* __restrict__ gout = (E*)p.out + (int64_t)h * p.o_sh + v0;
  const float* __restrict__ gdec = p.decay + (h & p.dmask);
  const float* __restrict__ gbet = p.beta + (h & p.bmask);
  int64_t ibase, fbase;
  prefill_state_offsets(p, r, h, v0, DK, ibase, fbase);
  if ((p.pool_flags & kPoolSkipUnread) && ibase < 0) return;  // uniform over the workgroup

  // M is only written on and below the diagonal; the readout reads the 16x16
  // blocks just above the diagonal as zeros, so clear M once.
  for (int idx = tid; idx < 2 * C * Sm::LDC; idx += 512)
    (&sm.der[idx / (C * Sm::LDC)].m[0][0])[idx % (C * Sm::LDC)] = from_f32<E>(0.f);

  // ------------------------------------------------------------ state waves
  // Every role runs its own loop with the same two barriers per chunk, so the
  // registers one role carries across chunks are not live in the other's.
  if (!is_prep) {
    const bool active = wave < NVT;  // waves beyond the slice only keep the barriers
    const int vc = 16 * wave + x;    // this lane's value column inside the slice
    const int vst = (int)p.v_st, ost = (int)p.o_st;
    const int v_lane = 4 * g * vst + x;  // lane part of the V / output offsets
    const int o_lane = 4 * g * ost + x;
    f4 S[NKT];
    E vreg[NT][4];
#pragma unroll
    for (int j = 0; j < NKT; ++j) S[j] = f4{0.f, 0.f, 0.f, 0.f};
    // V(c) in accumulator layout (rows t = 16i+4g+e, column vc): buffer loads
    // with the lane's offset fixed and the row in soffset; predicates only on
    // the last (partial) chunk of a request
    auto load_v = [&](int c) {
      const int64_t t0 = start + (int64_t)c * C;
      const int rem = (int)min((int64_t)C, end - t0);  // >= 1
      const E* vb = gv + t0 * p.v_st + 16 * wave;
      if (rem == C) {
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(vb);
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            vreg[i][e] = buf_load<E>(rs, v_lane * (uint32_t)sizeof(E), (16 * i + e) * vst * (uint32_t)sizeof(E));
      } else {
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * i + 4 * g + e;
            const E v = vb[min(t, rem - 1) * vst + x];  // clamped: inside the request
            vreg[i][e] = t < rem ? v : from_f32<E>(0.f);
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
    f4 X[NT], Y[NT];  // carried from part 1 to part 2
    for (int c = -1; c < nch; ++c) {
      const int cur = c & 1;
      const bool work = active && c >= 0;
      // ============================================================== part 1
      // R = [Q; K] S0 with the key blocks outermost: 2*NT independent
      // accumulator chains per block keep the MFMA pipe and LDS busy.
      if (work) {
        const typename Sm::Raw& R = sm.raw[cur];
        const typename Sm::Derived& Dd = sm.der[cur];
        Fr Sb[NKT];
#pragma unroll
        for (int j = 0; j < NKT; ++j) cvt_frag(S[j], Sb[j]);
        f4 rq[NT], rk[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) rq[i] = rk[i] = f4{0.f, 0.f, 0.f, 0.f};
        if constexpr (NKT % 2 == 0) {
#pragma unroll
          for (int pp = 0; pp < NKT / 2; ++pp) {
            Fr aq0[NT], aq1[NT], ak0[NT], ak1[NT];
#pragma unroll
            for (int i = 0; i < NT; ++i) {
              lds_frag8(&R.q[16 * i + x][32 * pp + 8 * g], aq0[i], aq1[i]);
              lds_frag8(&R.k[16 * i + x][32 * pp + 8 * g], ak0[i], ak1[i]);
            }
#pragma unroll
            for (int i = 0; i < NT; ++i) {
              rq[i] = mma_k32(rq[i], aq0[i], aq1[i], Sb[2 * pp], Sb[2 * pp + 1]);
              rk[i] = mma_k32(rk[i], ak0[i], ak1[i], Sb[2 * pp], Sb[2 * pp + 1]);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NKT; ++j) {
#pragma unroll
            for (int i = 0; i < NT; ++i) {
              Fr aq, ak;
              lds_frag(&R.q[16 * i + x][16 * j + 4 * g], aq);
              lds_frag(&R.k[16 * i + x][16 * j + 4 * g], ak);
              rq[i] = mma_k16(rq[i], aq, Sb[j]);
              rk[i] = mma_k16(rk[i], ak, Sb[j]);
            }
          }
        }
        // X = beta V - beta Gam R_K ; Y = scale Gam R_Q
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const f4 bt = *reinterpret_cast<const f4*>(&Dd.bet[16 * i + 4 * g]);
          const f4 gb = *reinterpret_cast<const f4*>(&Dd.gb[16 * i + 4 * g]);
          const f4 gs = *reinterpret_cast<const f4*>(&Dd.gs[16 * i + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            X[i][e] = bt[e] * to_f32(vreg[i][e]) - gb[e] * rk[i][e];
            Y[i][e] = gs[e] * rq[i][e];
          }
        }
        if (c + 1 < nch) load_v(c + 1);
      }
      lds_barrier();
      // ============================================================== part 2
      // (I + A) U = X, right-looking over 16-token blocks: once U_m is known
      // the products that consume it are issued (-A_im U_m for later blocks,
      // M_im U_m for the readout, K^T D U for the state), paired over two
      // token blocks where possible, so that only U_m -> P_{m+1} -> U_{m+1}
      // is a dependent chain.
      if (work) {
        const typename Sm::Raw& R = sm.raw[cur];
        const typename Sm::Derived& Dd = sm.der[cur];
        const float gC = Dd.gC;
#pragma unroll
        for (int j = 0; j < NKT; ++j) S[j] = gC * S[j];
        Fr Ub[NT], DU[NT];
#pragma unroll
        for (int m = 0; m < NT; ++m) {
          Fr Pb, ti;
          cvt_frag(X[m], Pb);
          lds_frag(&Dd.tinv[m][x][4 * g], ti);
          const f4 U = mma_k16(f4{0.f, 0.f, 0.f, 0.f}, ti, Pb);
          cvt_frag(U, Ub[m]);
          const f4 dc = *reinterpret_cast<const f4*>(&Dd.dc[16 * m + 4 * g]);
          cvt_frag(dc * U, DU[m]);
          if constexpr (NT % 2 == 0) {
            if ((m & 1) == 0) {
              // the next block needs U_m now; the rest waits for the pair
              Fr a;
              lds_frag(&Dd.negA[16 * (m + 1) + x][16 * m + 4 * g], a);
              X[m + 1] = mma_k16(X[m + 1], a, Ub[m]);
            } else {
              const int m0 = m - 1;
#pragma unroll
              for (int i = m + 1; i < NT; ++i) {
                Fr a0, a1;
                lds_frag(&Dd.negA[16 * i + x][16 * m0 + 4 * g], a0);
                lds_frag(&Dd.negA[16 * i + x][16 * m + 4 * g], a1);
                X[i] = mma_k32(X[i], a0, a1, Ub[m0], Ub[m]);
              }
              // every readout update is a 32-deep product (the block above
              // the diagonal, M[m0][m], is zero): one accumulator never mixes
              // MFMA shapes (see the note at the top of this file)
#pragma unroll
              for (int i = m0; i < NT; ++i) {
                Fr a0, a1;
                lds_frag(&Dd.m[16 * i + x][16 * m0 + 4 * g], a0);
                lds_frag(&Dd.m[16 * i + x][16 * m + 4 * g], a1);
                Y[i] = mma_k32(Y[i], a0, a1, Ub[m0], Ub[m]);
              }
#pragma unroll
              for (int j = 0; j < NKT; ++j) {
                const int krow = dk_of<NKT>(j, x);
                const int sw = kt_swz(krow);
                Fr a0, a1;
                lds_frag(&R.kt[krow][(16 * m0 + 4 * g) ^ sw], a0);
                lds_frag(&R.kt[krow][(16 * m + 4 * g) ^ sw], a1);
                S[j] = mma_k32(S[j], a0, a1, DU[m0], DU[m]);
              }
            }
          } else {
#pragma unroll
            for (int i = m + 1; i < NT; ++i) {
              Fr a;
              lds_frag(&Dd.negA[16 * i + x][16 * m + 4 * g], a);
              X[i] = mma_k16(X[i], a, Ub[m]);
            }
#pragma unroll
            for (int i = m; i < NT; ++i) {
              Fr a;
              lds_frag(&Dd.m[16 * i + x][16 * m + 4 * g], a);
              Y[i] = mma_k16(Y[i], a, Ub[m]);
            }
#pragma unroll
            for (int j = 0; j < NKT; ++j) {
              const int krow = dk_of<NKT>(j, x);
              Fr a;
              lds_frag(&R.kt[krow][(16 * m + 4 * g) ^ kt_swz(krow)], a);
              S[j] = mma_k16(S[j], a, DU[m]);
            }
          }
        }
        // output rows (scale already folded into Gam and M)
        const int64_t tok0 = start + (int64_t)c * C;
        const int nvalid = (int)min((int64_t)C, end - tok0);
        E* ob = gout + tok0 * p.o_st + 16 * wave;
        if (nvalid == C) {
          const __amdgpu_buffer_rsrc_t rs = buf_rsrc(ob);
#pragma unroll
          for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              buf_store(rs, o_lane * (uint32_t)sizeof(E), (16 * i + e) * ost * (uint32_t)sizeof(E),
                        from_f32<E>(Y[i][e]));
        } else {
#pragma unroll
          for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = 16 * i + 4 * g + e;
              if (t < nvalid) ob[t * ost + x] = from_f32<E>(Y[i][e]);
            }
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
  // Each prep wave shares its SIMD with a state wave, and the state waves
  // wait for the prep waves at the barriers: the prep waves issue first
  // (the ragged fp32 workload 0.5-0.8% faster, the chunked decode at T = 16
  // 2.5%, same-box A/B runs, bit-identical).
  __builtin_amdgcn_s_setprio(2);
  u32x4 pq[NPT][4], pk[NPT][4];
  float pg = 0.f, pb = 0.f;     // prefetched decay/beta of token `lane`
  E pga = from_f32<E>(0.f), pgb = from_f32<E>(0.f);  // or the fused gate's raw a, b
  bool pvalid = false;
  // gates, each input on its own: given (decay, beta) or fused (the qwen
  // gate from A_log, dt_bias, a; a sigmoid beta from b), computed here per
  // token
  const bool fd = EXT && p.ga != nullptr, fb = EXT && p.gb != nullptr;
  const E* gga = (const E*)p.ga + (h & p.dmask);
  const E* ggb = (const E*)p.gb + (h & p.bmask);
  const float ealog = fd ? expf(p.A_log[h & p.dmask]) : 0.f, dtb = fd ? p.dt_bias[h & p.dmask] : 0.f;
  const bool nrm = EXT && p.qk_norm != 0;

  int prem = 0;  // rows of the prefetched chunk
  auto prefetch = [&](int c) {
    const int64_t t0 = start + (int64_t)c * C;
    const int rem = (int)min((int64_t)C, end - t0);  // >= 1
    prem = rem;
    // the gates first: a wait the compiler places for their registers must
    // not also wait for the row loads (the wait counter is in order)
    {
      pvalid = lane < rem;
      const int tl = min(lane, rem - 1);
      const int64_t tok = (t0 + tl) * p.hv;
      // raw a and b as loaded (the gates are computed in the scan, so that
      // nothing waits on these loads here)
      if (fd) pga = gga[tok & p.dmask];
      else pg = gdec[tok & p.dmask];
      if (fb) pgb = ggb[tok & p.bmask];
      else pb = gbet[tok & p.bmask];
    }
    const E* qb = gq + t0 * p.q_st;
    const E* kb = gk + t0 * p.k_st;
    const int qst = (int)p.q_st, kst = (int)p.k_st;
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int pr = ptid + 256 * u;
      const int quad = pr / NOCT, oct = pr % NOCT;
      if (pr < NPAIR) {
        // rows past the end of the request read its last row (in bounds) and
        // are zeroed when staged, so the loads take no branch
        const __amdgpu_buffer_rsrc_t rq = buf_rsrc(qb), rk = buf_rsrc(kb);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int tc = min(4 * quad + w, rem - 1);
          pq[u][w] = buf_load16(rq, (uint32_t)((tc * qst + oct * VE) * sizeof(E)), 0);
          pk[u][w] = buf_load16(rk, (uint32_t)((tc * kst + oct * VE) * sizeof(E)), 0);
        }
      }
    }
  };

  // 1/|q_t| and 1/|k_t| of the prefetched rows (in-kernel L2 norm): each
  // row's vectors sit on NOCT consecutive lanes; an all-zero row (a padded
  // token, or eps == 0) keeps the factor 0
  auto row_norms = [&](typename Sm::Derived& Dd) {
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int pr = ptid + 256 * u;
      const int quad = pr / NOCT, oct = pr % NOCT;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float sq = 0.f, sk = 0.f;
        if (pr < NPAIR && 4 * quad + w < prem) {
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            const float a = to_f32(elem16<E>(pq[u][w], e)), b = to_f32(elem16<E>(pk[u][w], e));
            sq += a * a;
            sk += b * b;
          }
        }
#pragma unroll
        for (int off = NOCT / 2; off >= 1; off >>= 1) {
          sq += __shfl_xor(sq, off);
          sk += __shfl_xor(sk, off);
        }
        sq += p.qk_eps;
        sk += p.qk_eps;
        if (pr < NPAIR && oct == 0) {
          Dd.rqn[4 * quad + w] = sq > 0.f ? 1.f / sqrtf(sq) : 0.f;
          Dd.rkn[4 * quad + w] = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
        }
      }
    }
  };

  auto store_raw = [&](int buf) {
    typename Sm::Raw& R = sm.raw[buf];
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int pr = ptid + 256 * u;
      if (pr < NPAIR) {
        const int quad = pr / NOCT, oct = pr % NOCT;
        u32x4 kq[4], kk[4];  // padded rows zeroed
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t keep = 4 * quad + w < prem ? 0xffffffffu : 0u;
          kq[w] = pq[u][w] & keep;
          kk[w] = pk[u][w] & keep;
          *reinterpret_cast<u32x4*>(&R.q[4 * quad + w][oct * VE]) = kq[w];
          *reinterpret_cast<u32x4*>(&R.k[4 * quad + w][oct * VE]) = kk[w];
        }
        // transposed K: for each key of the vector, 4 consecutive tokens
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const int krow = oct * VE + e;
          typename pack4<E>::type col;
#pragma unroll
          for (int w = 0; w < 4; ++w) col[w] = elem16<E>(kk[w], e);
          *reinterpret_cast<typename pack4<E>::type*>(&R.kt[krow][(4 * quad) ^ kt_swz(krow)]) = col;
        }
      }
    }
  };

  // scan of the prefetched chunk (prep wave 0): F, z and the per-token factors
  auto scan = [&](typename Sm::Derived& Dd) {
    float lg = 0.f;
    bool reset = false;
    // an absent fused input: no decay, beta 1
    if (fd) pg = p.dmask ? gate_log_decay_fast(ealog, dtb, to_f32(pga)) : 0.f;
    if (fb) pb = p.bmask ? sigmoid_fast(to_f32(pgb)) : 1.f;
    if (pvalid) {
      if (p.decay_is_gamma) {
        reset = !(pg > 0.f);
        lg = reset ? 0.f : __log2f(pg);
      } else {
        reset = !(pg > -INFINITY);
        lg = reset ? 0.f : pg * 1.4426950408889634f;
      }
    }
    const float F = wave_scan_add(lg);
    const int z = wave_scan_max(reset ? lane : -1);
    const float Flast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(F), C - 1));
    const int zlast = __builtin_amdgcn_readlane(z, C - 1);
    if (lane < C) {
      const float gam = z < 0 ? exp2f(F) : 0.f;
      const float bt = pvalid ? pb : 0.f;
      Dd.F[lane] = F;
      Dd.z[lane] = z;
      Dd.bet[lane] = bt;
      Dd.gb[lane] = p.rho * bt * gam;  // the retrieval term of X
      Dd.gs[lane] = p.scale * gam;
      Dd.dc[lane] = zlast <= lane ? exp2f(Flast - F) : 0.f;
      if (lane == C - 1) {
        Dd.gC = gam;
        Dd.any_zero = zlast >= 0;
      }
    }
  };

  // Inverses of the four unit-lower diagonal blocks (I + A_ii) of chunk c, one
  // block per lane group: lane (x, i) computes row x of T_i = (I + A_ii)^-1 by
  // back substitution on the transposed block, T_i[x][j] = [j == x] -
  // sum_{k > j} A_i[k][j] T_i[x][k] for j = 15 .. 0, and stores it as one row.
  auto invert_diag = [&](typename Sm::Derived& Dd) {
    const int i = g;
    if (i >= NT) return;
    float row[16];
    f4 cur[4], nx[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) cur[q4] = *reinterpret_cast<const f4*>(&sm.adiagT[i][15][4 * q4]);
#pragma unroll
    for (int j = 15; j >= 0; --j) {
      if (j > 0) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) nx[q4] = *reinterpret_cast<const f4*>(&sm.adiagT[i][j - 1][4 * q4]);
      }
      // cur[k/4][k%4] = A_i[k][j]
      float a0 = (j == x) ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
      for (int k = 15; k > j + 1; --k) {
        if (k & 1) a1 -= cur[k >> 2][k & 3] * row[k];
        else a0 -= cur[k >> 2][k & 3] * row[k];
      }
      row[j] = j < 15 ? (a0 + a1) - cur[(j + 1) >> 2][(j + 1) & 3] * row[j + 1] : a0;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) cur[q4] = nx[q4];
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<typename pack4<E>::type*>(&Dd.tinv[i][x][4 * q4]) =
          to_pack4<E>(f4{row[4 * q4], row[4 * q4 + 1], row[4 * q4 + 2], row[4 * q4 + 3]});
  };

  if (nch > 0) prefetch(0);
  for (int c = -1; c < nch; ++c) {
    const int cur = c & 1, nxt = (c + 1) & 1;
    const bool work = c + 1 < nch;
    // ================================================================ part 1
    if (work) {
      store_raw(nxt);
      if (nrm) row_norms(sm.der[nxt]);
      if (pw == 0) scan(sm.der[nxt]);
    }
    // the diagonal blocks of chunk c (staged in the previous part 2)
    if (pw == 1 && c >= 0) invert_diag(sm.der[cur]);
    if (work && c + 2 < nch) prefetch(c + 2);
    lds_barrier();
    // ================================================================ part 2
    if (work) {
      const typename Sm::Raw& R = sm.raw[nxt];
      typename Sm::Derived& Dd = sm.der[nxt];
      if (nrm && pw == 0 && lane < C) {
        // fold the norms (written in part 1) into the per-token factors
        Dd.gb[lane] *= Dd.rkn[lane];
        Dd.gs[lane] *= Dd.rqn[lane];
        Dd.dc[lane] *= Dd.rkn[lane];
      }
      // Tiles of K K^T and K Q^T computed transposed -- rows s (key token),
      // columns t (query token) -- so that each lane (t = 16i + x) ends with
      // 4 consecutive s of row t and stores -A and M rows as vectors.  Prep
      // wave pw owns diagonal tile (pw, pw) (slot 0) and the off-diagonal
      // tiles whose list index o has (NT + o) mod 4 == pw (slots 1..), so the
      // off-diagonal tiles start on the waves without a diagonal one (each
      // prep wave shares its SIMD with a state wave: the MFMA load is spread
      // evenly); all of a wave's tiles share one pass over the key blocks.
      constexpr int MT = 1 + (NOFF + 3) / 4;
      int ti[MT], tm[MT];
      bool tv[MT];
      ti[0] = tm[0] = pw;
      tv[0] = pw < NT;
#pragma unroll
      for (int k = 1; k < MT; ++k) {
        const int o = (pw + 4 - NT % 4) % 4 + 4 * (k - 1);
        int i = 1, rem = o;
        while (rem >= i) { rem -= i; ++i; }
        ti[k] = i;
        tm[k] = rem;
        tv[k] = o < NOFF;
      }
      f4 kk[MT], qk[MT];
#pragma unroll
      for (int k = 0; k < MT; ++k) kk[k] = qk[k] = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (NKT % 2 == 0) {
#pragma unroll
        for (int pp = 0; pp < NKT / 2; ++pp) {
#pragma unroll
          for (int k = 0; k < MT; ++k) {
            if (!tv[k]) continue;
            Fr as0, as1, bk0, bk1, bq0, bq1;
            lds_frag8(&R.k[16 * tm[k] + x][32 * pp + 8 * g], as0, as1);
            lds_frag8(&R.k[16 * ti[k] + x][32 * pp + 8 * g], bk0, bk1);
            lds_frag8(&R.q[16 * ti[k] + x][32 * pp + 8 * g], bq0, bq1);
            kk[k] = mma_k32(kk[k], as0, as1, bk0, bk1);
            qk[k] = mma_k32(qk[k], as0, as1, bq0, bq1);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NKT; ++j) {
#pragma unroll
          for (int k = 0; k < MT; ++k) {
            if (!tv[k]) continue;
            Fr as, bk, bq;
            lds_frag(&R.k[16 * tm[k] + x][16 * j + 4 * g], as);
            lds_frag(&R.k[16 * ti[k] + x][16 * j + 4 * g], bk);
            lds_frag(&R.q[16 * ti[k] + x][16 * j + 4 * g], bq);
            kk[k] = mma_k16(kk[k], as, bk);
            qk[k] = mma_k16(qk[k], as, bq);
          }
        }
      }
      const bool any_zero = Dd.any_zero;
      // D(t, s) for this lane's row t = 16i+x and columns s = 16m+4g+e
      auto decay4 = [&](int i, int m, bool diag) -> f4 {
        const int t = 16 * i + x;
        const float Ft = Dd.F[t];
        const f4 Fs = *reinterpret_cast<const f4*>(&Dd.F[16 * m + 4 * g]);
        f4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = exp2f(Ft - Fs[e]);
        if (diag) {
#pragma unroll
          for (int e = 0; e < 4; ++e) d[e] = (16 * m + 4 * g + e <= t) ? d[e] : 0.f;
        }
        if (any_zero) {  // a gamma of 0 between s and t cuts the product
          const int zt = Dd.z[t];
#pragma unroll
          for (int e = 0; e < 4; ++e) d[e] = (zt <= 16 * m + 4 * g + e) ? d[e] : 0.f;
        }
        return d;
      };
      // off-diagonal tiles: M and -A
#pragma unroll
      for (int k = 1; k < MT; ++k) {
        if (!tv[k]) continue;
        const int t = 16 * ti[k] + x;
        f4 d = decay4(ti[k], tm[k], false);
        const float bt = p.rho * Dd.bet[t];  // A carries the retrieval term
        f4 dq = d, dk = d;
        if (nrm) {
          const f4 rks = *reinterpret_cast<const f4*>(&Dd.rkn[16 * tm[k] + 4 * g]);
          dq = d * (rks * Dd.rqn[t]);
          dk = d * (rks * Dd.rkn[t]);
        }
        *reinterpret_cast<typename pack4<E>::type*>(&Dd.m[t][16 * tm[k] + 4 * g]) =
            to_pack4<E>(p.scale * dq * qk[k]);
        *reinterpret_cast<typename pack4<E>::type*>(&Dd.negA[t][16 * tm[k] + 4 * g]) =
            to_pack4<E>(-bt * dk * kk[k]);
      }
      // diagonal tile: M, and A_ii (fp32, transposed) for the inverse that the
      // next staging part computes
      if (tv[0]) {
        const int i = pw;
        const int t = 16 * i + x;
        const f4 d = decay4(i, i, true);
        const float bt = p.rho * Dd.bet[t];  // A carries the retrieval term
        f4 dq = d, dk = d;
        if (nrm) {
          const f4 rks = *reinterpret_cast<const f4*>(&Dd.rkn[16 * i + 4 * g]);
          dq = d * (rks * Dd.rqn[t]);
          dk = d * (rks * Dd.rkn[t]);
        }
        *reinterpret_cast<typename pack4<E>::type*>(&Dd.m[t][16 * i + 4 * g]) =
            to_pack4<E>(p.scale * dq * qk[0]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sm.adiagT[i][4 * g + e][x] = (4 * g + e < x) ? bt * dk[e] * kk[0][e] : 0.f;
      }
    }
    lds_barrier();
  }
}

// Value columns per workgroup: one 16-column tile per state wave.
template <int DV>
constexpr int prefill_dvs() {
  return DV < 64 ? DV : 64;
}

// Whether the chunk fits the 160 KiB of LDS a workgroup may use on gfx950.
template <typename E, int DK, int DV, int C>
constexpr bool prefill_fits() {
  return sizeof(PrefillSmem<E, DK, prefill_dvs<DV>(), C>) <= 160 * 1024;
}

template <typename E, int DK, int DV, int C>
hipError_t launch_prefill_t(PrefillParams p, hipStream_t stream) {
  if constexpr (!prefill_fits<E, DK, DV, C>()) {
    return hipErrorInvalidValue;  // the host never selects such a chunk
  } else {
    constexpr int DVS = prefill_dvs<DV>();
    p.nsplit = DV / DVS;
    const int64_t nblk = (int64_t)p.n_seqs * p.hv * p.nsplit;
    if (p.ga || p.gb || p.qk_norm)
      hipLaunchKernelGGL((prefill_kernel<E, DK, DVS, C, true>), dim3((unsigned)nblk), dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL((prefill_kernel<E, DK, DVS, C, false>), dim3((unsigned)nblk), dim3(512), 0, stream, p);
    return hipGetLastError();
  }
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

// Largest chunk <= hint (16, 32 or 64) whose working set fits LDS.
template <typename E>
int prefill_chunk_for(int dk, int dv, int hint) {
  auto fits = [&](int c) -> bool {
#define GDN_FIT(DK, DV)                                                              \
  if (dk == DK && dv == DV)                                                          \
    return c == 64 ? prefill_fits<E, DK, DV, 64>()                                   \
                   : (c == 32 ? prefill_fits<E, DK, DV, 32>() : prefill_fits<E, DK, DV, 16>());
#define GDN_FIT_DK(DK) GDN_FIT(DK, 16) GDN_FIT(DK, 32) GDN_FIT(DK, 64) GDN_FIT(DK, 128)
    GDN_FIT_DK(16) GDN_FIT_DK(32) GDN_FIT_DK(64) GDN_FIT_DK(128)
#undef GDN_FIT_DK
#undef GDN_FIT
    return false;
  };
  for (int c = hint; c >= 16; c >>= 1)
    if (fits(c)) return c;
  return 16;
}

// One instantiation unit per (operand type, chunk): gdn_prefill_<t>_c<C>.hip
hipError_t prefill_bf16_c16(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_bf16_c32(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_bf16_c64(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_f32_c16(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_f32_c32(PrefillParams p, int dk, int dv, hipStream_t s);
hipError_t prefill_f32_c64(PrefillParams p, int dk, int dv, hipStream_t s);

}  // namespace gdn
