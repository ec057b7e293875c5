// gdn_prefill_pk.hip -- chunked prefill with a per-key decay.
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
//   S_C = diag(Gam_C) S0 + sum_s diag(Gam_{C/s}) k_s u_s^T
// Every factor is a product of decays <= 1: the log2-decays are summed per key
// inside the chunk and differences F_t - F_s taken, and a decay of exactly 0
// (log-decay -inf, or gamma 0) is tracked by the index of the last one per key
// (as the scalar kernels do per head), so no -inf - (-inf) is formed.
//
// One workgroup of 256 threads per (request, value head, slice of DVS value
// columns); TPC = 256 / DVS threads share a value column and hold DK / TPC
// keys of its state in registers.  The per-pair Gram sums are elementwise
// (each key has its own decay, so they are not plain dot products): one
// (t, s) pair per thread.  Everything is fp32 on the VALU: this kernel
// favours a plain, checkable structure over speed.
#include "gdn_device.hpp"
#include "gdn_prefill.hpp"

namespace gdn {

template <typename E, int DK, int DVS>
__global__ void __launch_bounds__(256)
prefill_pk_kernel(const PrefillParams p) {
  constexpr int C = 16;
  constexpr int TPC = 256 / DVS;    // threads per value column
  constexpr int KPT = DK / TPC;     // keys per thread
  constexpr int LDK = DK + 1;       // odd row stride: the Gram reads of 16 rows hit 16 banks
  static_assert(KPT >= 1 && DK % TPC == 0, "key split");
  __shared__ float sk[C][LDK], sq[C][LDK], sF[C][LDK];
  __shared__ int sz[C][LDK];
  __shared__ __attribute__((aligned(16))) float skg[C][DK], sqg[C][DK], skc[C][DK];
  __shared__ float sA[C][C], sM[C][C], sv[C][DVS], sbet[C], snq[C], snk[C];

  const int tid = threadIdx.x;
  const int nsplit = p.nsplit;
  const int blk = blockIdx.x;
  const int split = blk % nsplit;
  const int h = (blk / nsplit) % p.hv;
  const int r = blk / (nsplit * p.hv);
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
  int64_t ibase, fbase;
  prefill_state_offsets(p, r, h, v0, DK, ibase, fbase);
  if ((p.pool_flags & kPoolSkipUnread) && ibase < 0) return;  // uniform over the workgroup

  const E* __restrict__ gq = (const E*)p.q + (int64_t)qh * p.q_sh;
  const E* __restrict__ gk = (const E*)p.k + (int64_t)qh * p.k_sh;
  const E* __restrict__ gv = (const E*)p.v + (int64_t)h * p.v_sh + v0;
  E* __restrict__ gout = (E*)p.out + (int64_t)h * p.o_sh + v0;
  const float* __restrict__ gdec = p.decay + (int64_t)h * DK;  // [T, hv, DK]
  const float* __restrict__ gbet = p.beta + (h & p.bmask);

  const int jc = tid / TPC;          // value column of this thread (inside the slice)
  const int kp = tid % TPC;          // key part
  const int i0 = kp * KPT;           // first key of this thread
  float S[KPT];
#pragma unroll
  for (int m = 0; m < KPT; ++m) S[m] = 0.f;
  if (ibase >= 0) {
#pragma unroll
    for (int m = 0; m < KPT; ++m) S[m] = p.init[ibase + (int64_t)jc * DK + i0 + m];
  }

  const int nch = (int)((end - start + C - 1) / C);
  // The next chunk's inputs are loaded into registers while the current one
  // is computed, exactly as loaded (no conversion or select on them before
  // they are staged, which would make the loads block).  Rows past the end of
  // a request read the request's first row of the chunk instead (always in
  // bounds) and are zeroed when staged.
  constexpr int NLD = (C * DK + 255) / 256, NLV = (C * DVS + 255) / 256;
  E pk[NLD], pq[NLD];
  float pg[NLD], pbt = 0.f;
  E pv[NLV];
  auto prefetch = [&](int cc) {
    const int64_t t0 = start + (int64_t)cc * C;
    const int nv = (int)min((int64_t)C, end - t0);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + 256 * u;
      if (idx < C * DK) {
        const int t = idx / DK, i = idx % DK;
        const int64_t tok = t0 + min(t, nv - 1);
        pk[u] = gk[tok * p.k_st + i];
        pq[u] = gq[tok * p.q_st + i];
        pg[u] = gdec[tok * (int64_t)p.hv * DK + i];
      }
    }
#pragma unroll
    for (int u = 0; u < NLV; ++u) {
      const int idx = tid + 256 * u;
      if (idx < C * DVS) {
        const int t = idx / DVS, j = idx % DVS;
        pv[u] = gv[(t0 + min(t, nv - 1)) * p.v_st + j];
      }
    }
    if (tid < C) pbt = gbet[((t0 + min(tid, nv - 1)) * p.hv) & p.bmask];
  };
  auto stage = [&](int nv) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + 256 * u;
      if (idx < C * DK) {
        const int t = idx / DK, i = idx % DK;
        const bool live = t < nv;
        sk[t][i] = live ? to_f32(pk[u]) : 0.f;
        sq[t][i] = live ? to_f32(pq[u]) : 0.f;
        const float d = pg[u];
        // log2 of the decay: the factors below are exp2 of differences
        const float g = p.decay_is_gamma ? (d > 0.f ? __log2f(d) : -INFINITY) : d * 1.4426950408889634f;
        sF[t][i] = live ? g : 0.f;  // raw log2-decay; the scan turns it into prefix sums
      }
    }
#pragma unroll
    for (int u = 0; u < NLV; ++u) {
      const int idx = tid + 256 * u;
      if (idx < C * DVS) sv[idx / DVS][idx % DVS] = idx / DVS < nv ? to_f32(pv[u]) : 0.f;
    }
    if (tid < C) sbet[tid] = tid < nv ? pbt : 0.f;
  };
  if (nch > 0) prefetch(0);
  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = start + (int64_t)c * C;
    const int nvalid = (int)min((int64_t)C, end - t0);
    // ---- stage the chunk: q, k (fp32), log-decays, v slice, beta; padded
    // tokens are k = q = v = 0, no decay, beta 0; then start the next loads
    stage(nvalid);
    if (c + 1 < nch) prefetch(c + 1);
    __syncthreads();
    // ---- in-kernel L2 norm of q and k rows (one wave per 4 rows)
    if (p.qk_norm) {
      const int w = tid >> 6, lane = tid & 63;
      for (int t = w; t < C; t += 4) {
        float a = 0.f, b = 0.f;
        for (int i = lane; i < DK; i += 64) {
          a += sq[t][i] * sq[t][i];
          b += sk[t][i] * sk[t][i];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          a += __shfl_xor(a, off);
          b += __shfl_xor(b, off);
        }
        a += p.qk_eps;
        b += p.qk_eps;
        if (lane == 0) {
          snq[t] = a > 0.f ? 1.f / sqrtf(a) : 0.f;
          snk[t] = b > 0.f ? 1.f / sqrtf(b) : 0.f;
        }
      }
      __syncthreads();
      for (int idx = tid; idx < C * DK; idx += 256) {
        const int t = idx / DK, i = idx % DK;
        sq[t][i] *= snq[t];
        sk[t][i] *= snk[t];
      }
      __syncthreads();
    }
    // ---- per-key scan over the chunk (one thread per key): F_t = sum of the
    // finite log2-decays up to t, z_t = last t with a decay of 0 (-1: none);
    // then the decayed copies of k and q used by the state pass
    if (tid < DK) {
      const int i = tid;
      float F = 0.f;
      int z = -1;
      for (int t = 0; t < C; ++t) {
        const float g = sF[t][i];
        if (g > -INFINITY) F += g;
        else z = t;
        sF[t][i] = F;
        sz[t][i] = z;
      }
      const float FC = F;
      const int zC = z;
      for (int t = 0; t < C; ++t) {
        const float Ft = sF[t][i];
        const float gam = sz[t][i] >= 0 ? 0.f : __builtin_amdgcn_exp2f(Ft);        // Gam_t
        const float gct = zC > t ? 0.f : __builtin_amdgcn_exp2f(FC - Ft);          // Gam_{C/t}
        skg[t][i] = sk[t][i] * gam;
        sqg[t][i] = sq[t][i] * gam;
        skc[t][i] = sk[t][i] * gct;
      }
    }
    __syncthreads();
    // ---- Gram pairs: A_ts (s < t) and M_ts (s <= t), one (t, s) per thread
    {
      const int t = tid >> 4, s = tid & 15;
      float a = 0.f, m = 0.f;
      if (s <= t) {
        for (int i = 0; i < DK; ++i) {
          const float f = sz[t][i] > s ? 0.f : __builtin_amdgcn_exp2f(sF[t][i] - sF[s][i]);
          const float ks = sk[s][i] * f;
          a += sk[t][i] * ks;
          m += sq[t][i] * ks;
        }
      }
      sA[t][s] = s < t ? p.rho * sbet[t] * a : 0.f;
      sM[t][s] = s <= t ? p.scale * m : 0.f;
    }
    __syncthreads();
    // ---- state pass for column jc, token by token: r_k = S0^T (Gam_t o k_t),
    // u_t by forward substitution, y_t = scale S0^T (Gam_t o q_t) + M u; then
    // the state update.  Only u and this thread's state slice stay live.
    float u[C];
#pragma unroll
    for (int t = 0; t < C; ++t) {
      float ak = 0.f, aq = 0.f;
      if constexpr (KPT % 4 == 0) {  // 16-byte reads (i0 is a multiple of 4)
#pragma unroll
        for (int m = 0; m < KPT; m += 4) {
          const f4 kg = *reinterpret_cast<const f4*>(&skg[t][i0 + m]);
          const f4 qg = *reinterpret_cast<const f4*>(&sqg[t][i0 + m]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ak += kg[e] * S[m + e];
            aq += qg[e] * S[m + e];
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
          ak += skg[t][i0 + m] * S[m];
          aq += sqg[t][i0 + m] * S[m];
        }
      }
      const float rk = group_sum<TPC>(ak), rq = group_sum<TPC>(aq);
      float x = sbet[t] * (sv[t][jc] - p.rho * rk);
#pragma unroll
      for (int s2 = 0; s2 < t; ++s2) x -= sA[t][s2] * u[s2];
      u[t] = x;
      if (kp == 0 && t < nvalid) {
        float y = p.scale * rq;
#pragma unroll
        for (int s2 = 0; s2 <= t; ++s2) y += sM[t][s2] * u[s2];
        gout[(t0 + t) * p.o_st + jc] = from_f32<E>(y);
      }
    }
    // S_C = diag(Gam over the whole chunk) S0 + sum_t diag(Gam_{C/t}) k_t u_t^T
    // (padded tokens do not decay, so the scan's last row covers the chunk)
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int i = i0 + m;
      S[m] *= sz[C - 1][i] >= 0 ? 0.f : __builtin_amdgcn_exp2f(sF[C - 1][i]);
    }
#pragma unroll
    for (int t = 0; t < C; ++t) {
      if constexpr (KPT % 4 == 0) {
#pragma unroll
        for (int m = 0; m < KPT; m += 4) {
          const f4 kc = *reinterpret_cast<const f4*>(&skc[t][i0 + m]);
#pragma unroll
          for (int e = 0; e < 4; ++e) S[m + e] += kc[e] * u[t];
        }
      } else {
#pragma unroll
        for (int m = 0; m < KPT; ++m) S[m] += skc[t][i0 + m] * u[t];
      }
    }
    __syncthreads();  // the next chunk restages the shared arrays
  }
  if (fbase >= 0) {
#pragma unroll
    for (int m = 0; m < KPT; ++m) p.fin[fbase + (int64_t)jc * DK + i0 + m] = S[m];
  }
}

template <typename E, int DK, int DVS>
static hipError_t launch_pk_t(PrefillParams p, hipStream_t stream) {
  p.nsplit = p.dv / DVS;
  const int64_t nblk = (int64_t)p.n_seqs * p.hv * p.nsplit;
  hipLaunchKernelGGL((prefill_pk_kernel<E, DK, DVS>), dim3((unsigned)nblk), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename E, int DK>
static hipError_t launch_pk_dv(const PrefillParams& p, int dv, hipStream_t s) {
  switch (dv) {
    case 16: return launch_pk_t<E, DK, 16>(p, s);
    case 32: case 64: case 128: return launch_pk_t<E, DK, 32>(p, s);  // 32-column slices: 5.99 vs 6.40 ms with 64
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
