// gdn_prefill_scan.hip -- prefill of few, long requests as a scan over the
// affine maps of request segments (gfx950).
//
// Over any run of tokens the recurrence of "Gated DeltaNet State Update"
// (statement; each step S <- gamma (I - beta k k^T) S + beta k v^T is affine
// in S) maps the state entering the run to the state leaving it by
//     S_out = P S_in + R        (K-major: P is dk x dk, R is dk x dv),
// and maps compose: (P2, R2) after (P1, R1) is (P2 P1, P2 R1 + R2).  The
// "com.microsoft.GatedDeltaNet" card's chunk_size attribute makes the chunk
// a scheduling choice that never changes the result; the "Circuit.LLM.Mixer"
// module's chunkedLinearAttn carries a state across chunks the same way.
// Cutting one request into nseg segments of whole chunks gives three
// launches instead of one serial walk over all its chunks:
//  1. local pass (the pair kernel, seg_mode 1): every segment runs from a
//     zero state, giving R, and from the key identity with zero values on
//     dk extra "transition" rows, giving the columns of P; all segments in
//     parallel, no outputs;
//  2. combine (this file): per (request, value head, 16 value rows), walk the
//     segments in order: S_in(0) is the request's initial state and
//     S_in(j+1) = P_j S_in(j) + R_j, stored for pass 3; after the last
//     segment it is the request's final state;
//  3. rerun (the pair kernel, seg_mode 2): every segment again from its true
//     S_in(j), with outputs, in parallel.
// That is about three times the work of the serial walk, spread over nseg
// times as many workgroups: it pays when a call has few (request, head,
// slice) units, e.g. one long request with a few value heads.
//
// V-major rows: a state row s (one value index over all keys) maps as
// s_out = s_in P^T + r, i.e. for a block X of 16 rows,
//     X_out^T = P X^T + R^T.
// The local pass stores P K-major (row k = P[k][0 .. dk-1]), so a lane's
// 8 consecutive contraction indices of the A operand (a key row of P) and of
// the B operand (a row of X, held in LDS) are both contiguous.  The product
// runs on bf16 MFMAs in split form: with v = hi + lo (hi = bf16(v), lo =
// bf16(v - hi), 16 significant bits together), P X^T is taken as
// Phi Xhi + Phi Xlo + Plo Xhi, accumulated in fp32 (relative error about
// 2^-15 per segment, far below the bf16 operand rounding of the chunk
// kernel that produced P).  An empty segment is skipped (its map is the
// identity), so an empty request keeps its state bit for bit.
#include <hip/hip_runtime.h>

#include "gdn_prefill.hpp"

namespace gdn {

struct ScanParams {
  PrefillParams p;       // the call: request bounds, initial / final state or pool
  int nseg, dk;
  const float* ws_map;   // [n_seqs * nseg, hv, dv + dk, dk]: R rows (V-major), then P (K-major)
  float* ws_in;          // [n_seqs * nseg, hv, dv, dk]: S_in of every segment
};

typedef __bf16 sbf8 __attribute__((ext_vector_type(8)));
typedef float sf2 __attribute__((ext_vector_type(2)));
typedef __bf16 sbf2 __attribute__((ext_vector_type(2)));

// 8 fp32 values -> (hi, lo) bf16 operands, both rounded to nearest even.
__device__ __forceinline__ void split8(f4 a, f4 b, sbf8& hi, sbf8& lo) {
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const sbf2 h2 = __builtin_convertvector((sf2){v[e], v[e + 1]}, sbf2);
    const sbf2 l2 = __builtin_convertvector((sf2){v[e] - (float)h2[0], v[e + 1] - (float)h2[1]}, sbf2);
    hi[e] = h2[0];
    hi[e + 1] = h2[1];
    lo[e] = l2[0];
    lo[e + 1] = l2[1];
  }
}

// One workgroup per (request r, value head h, 16 value rows); wave w owns the
// NTW 16-key tiles from key 16 NTW w of the rows' next state.
template <int DK>
__global__ void __launch_bounds__(256) scan_combine_kernel(const ScanParams s) {
  constexpr int NTW = DK / 64;  // 16-key tiles per wave
  constexpr int NKS = DK / 32;  // 32-deep contraction steps
  constexpr int LDX = DK + 4;   // padded fp32 rows
  __shared__ float xs[16][LDX];
  const PrefillParams& p = s.p;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, x = lane & 15, g = lane >> 4;
  const int nrg = p.dv / 16;
  const int rg = blockIdx.x % nrg;
  const int h = (blockIdx.x / nrg) % p.hv;
  const int r = blockIdx.x / (nrg * p.hv);
  const int row0 = 16 * rg;
  int64_t ibase, fbase;
  prefill_state_offsets(p, r, h, row0, DK, ibase, fbase);
  int64_t rstart, rend;
  prefill_request_bounds(p, r, rstart, rend);

  for (int idx = tid; idx < 16 * DK; idx += 256) {
    const int rr = idx / DK, k = idx % DK;
    xs[rr][k] = ibase >= 0 ? p.init[ibase + (int64_t)rr * DK + k] : 0.f;
  }
  __syncthreads();

  auto map_of = [&](int j) -> const float* {
    return s.ws_map + (((int64_t)r * s.nseg + j) * p.hv + h) * (int64_t)(p.dv + DK) * DK;
  };
  // A operand of segment j: lane (x, g) holds P[key][32 ks + 8 g .. + 7] of
  // key 16 (NTW w + t) + x
  f4 pa[NTW][NKS][2], pn[NTW][NKS][2];
  auto load_p = [&](int j, f4 (&dst)[NTW][NKS][2]) {
    const float* pk = map_of(j) + (int64_t)p.dv * DK;
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const float* q = pk + (int64_t)(16 * (NTW * w + t) + x) * DK + 32 * ks + 8 * g;
        dst[t][ks][0] = *reinterpret_cast<const f4*>(q);
        dst[t][ks][1] = *reinterpret_cast<const f4*>(q + 4);
      }
  };
  load_p(0, pa);
  for (int j = 0; j < s.nseg; ++j) {
    if (j + 1 < s.nseg) load_p(j + 1, pn);
    const int64_t seg = (int64_t)r * s.nseg + j;
    float* win = s.ws_in + ((seg * p.hv + h) * p.dv + row0) * DK;
    for (int idx = tid; idx < 16 * DK; idx += 256) win[idx] = xs[idx / DK][idx % DK];
    int64_t a = rstart, b = rend;
    prefill_segment_bounds(s.nseg, j, 64, a, b);
    if (b > a) {
      // D[key][row] = R[row][key] + sum_i P[key][i] X[row][i]; lane (x, g)
      // holds keys 4g .. 4g+3 of the tile for row x
      const float* map = map_of(j);
      f4 acc[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        acc[t] = *reinterpret_cast<const f4*>(map + (int64_t)(row0 + x) * DK + 16 * (NTW * w + t) + 4 * g);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        sbf8 bh, bl;
        split8(*reinterpret_cast<const f4*>(&xs[x][32 * ks + 8 * g]),
               *reinterpret_cast<const f4*>(&xs[x][32 * ks + 8 * g + 4]), bh, bl);
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          sbf8 ah, al;
          split8(pa[t][ks][0], pa[t][ks][1], ah, al);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[t], 0, 0, 0);
        }
      }
      __syncthreads();  // every wave has read the rows
#pragma unroll
      for (int t = 0; t < NTW; ++t) *reinterpret_cast<f4*>(&xs[x][16 * (NTW * w + t) + 4 * g]) = acc[t];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        pa[t][ks][0] = pn[t][ks][0];
        pa[t][ks][1] = pn[t][ks][1];
      }
  }
  if (fbase >= 0)
    for (int idx = tid; idx < 16 * DK; idx += 256) p.fin[fbase + idx] = xs[idx / DK][idx % DK];
}

hipError_t launch_scan_combine(const PrefillParams& p, int nseg, int dk, const float* ws_map, float* ws_in,
                               hipStream_t stream) {
  ScanParams s;
  s.p = p;
  s.nseg = nseg;
  s.dk = dk;
  s.ws_map = ws_map;
  s.ws_in = ws_in;
  const dim3 grid((unsigned)((int64_t)p.n_seqs * p.hv * (p.dv / 16))), block(256);
  if (dk == 64) hipLaunchKernelGGL(scan_combine_kernel<64>, grid, block, 0, stream, s);
  else if (dk == 128) hipLaunchKernelGGL(scan_combine_kernel<128>, grid, block, 0, stream, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gdn
