// gdn_gate.hip -- fused gate kernel (elementwise, HBM-bound).
//
// log_decay = -exp(A_log[h]) * softplus20(a + dt_bias[h]), gamma = exp(log_decay),
// beta = sigmoid(b): the "qwen" gate_activation of "com.microsoft.GatedDeltaNet"
// (Attributes) and the fused gate of the FlashInfer decode page.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

// Elements per thread.  The gate is latency-bound at the sizes it runs at
// (a few MB of traffic), so threads are many and short.
constexpr int kGateEPT = 4;

// The gates from the hardware exp2 / log2 / reciprocal (relative error about
// 1e-6, the forms the fused-gate prefill uses), which shorten each thread's
// dependent chain against the libm expf / log1pf forms.
__device__ __forceinline__ float gate_ld(float A_log, float dt_bias, float a) {
  return gate_log_decay_fast(__builtin_amdgcn_exp2f(A_log * 1.4426950408889634f), dt_bias, a);
}
__device__ __forceinline__ float exp_fast(float g) { return __builtin_amdgcn_exp2f(g * 1.4426950408889634f); }

__device__ __forceinline__ void store4f(float* p, const float* v) {
  *reinterpret_cast<f4*>(p) = f4{v[0], v[1], v[2], v[3]};
}

// Each thread handles kGateEPT consecutive elements of the flattened
// [n_tokens, hv] arrays.  VEC (every pointer 16-byte aligned): whole groups
// use one vector load per input and one 16-byte store per output; the
// ragged end and unaligned calls take the element loop.  The head of element
// i is i mod hv, found once per thread and stepped from there.
template <typename IN, bool VEC>
__global__ void __launch_bounds__(256)
gate_kernel(const float* __restrict__ A_log, const float* __restrict__ dt_bias,
            const IN* __restrict__ a, const IN* __restrict__ b, int64_t n_elems, int hv,
            float* __restrict__ log_decay, float* __restrict__ gamma, float* __restrict__ beta) {
  constexpr int N = kGateEPT;
  static_assert(N == 4, "one f4 per input and output");
  const int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * N;
  if (base >= n_elems) return;
  int h0 = n_elems <= 0xffffffffLL ? (int)((uint32_t)base % (uint32_t)hv) : (int)(base % hv);
  int hs[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    hs[e] = h0;
    h0 = h0 + 1 == hv ? 0 : h0 + 1;
  }
  if (VEC && base + N <= n_elems) {
    float o[N];
    if (a) {
      const f4 v = load4(a + base);
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = gate_ld(A_log[hs[e]], dt_bias[hs[e]], v[e]);
      if (log_decay) store4f(log_decay + base, o);
      if (gamma) {
#pragma unroll
        for (int e = 0; e < N; ++e) o[e] = exp_fast(o[e]);
        store4f(gamma + base, o);
      }
    }
    if (b) {
      const f4 v = load4(b + base);
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = sigmoid_fast(v[e]);
      store4f(beta + base, o);
    }
    return;
  }
  for (int e = 0; e < N && base + e < n_elems; ++e) {
    const int64_t i = base + e;
    if (a) {
      const float g = gate_ld(A_log[hs[e]], dt_bias[hs[e]], to_f32(a[i]));
      if (log_decay) log_decay[i] = g;
      if (gamma) gamma[i] = exp_fast(g);
    }
    if (b) beta[i] = sigmoid_fast(to_f32(b[i]));
  }
}

template <typename IN>
static void launch_gate_t(dim3 grid, hipStream_t stream, bool vec, const float* A_log, const float* dt_bias,
                          const IN* a, const IN* b, int64_t n, int hv, float* log_decay, float* gamma,
                          float* beta) {
  if (vec)
    hipLaunchKernelGGL((gate_kernel<IN, true>), grid, dim3(256), 0, stream, A_log, dt_bias, a, b, n, hv,
                       log_decay, gamma, beta);
  else
    hipLaunchKernelGGL((gate_kernel<IN, false>), grid, dim3(256), 0, stream, A_log, dt_bias, a, b, n, hv,
                       log_decay, gamma, beta);
}

hipError_t launch_gate(const float* A_log, const float* dt_bias, const void* a, const void* b,
                       int ab_dtype, int64_t n_tokens, int hv, float* log_decay, float* gamma,
                       float* beta, hipStream_t stream) {
  const int64_t n = n_tokens * hv;
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + kGateEPT - 1) / kGateEPT;
  const dim3 grid((unsigned)((threads + 255) / 256));
  auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const bool vec = al(a) && al(b) && al(log_decay) && al(gamma) && al(beta);
  if (ab_dtype == GDN_BF16)
    launch_gate_t(grid, stream, vec, A_log, dt_bias, (const __bf16*)a, (const __bf16*)b, n, hv, log_decay, gamma,
                  beta);
  else
    launch_gate_t(grid, stream, vec, A_log, dt_bias, (const float*)a, (const float*)b, n, hv, log_decay, gamma,
                  beta);
  return hipGetLastError();
}

}  // namespace gdn
