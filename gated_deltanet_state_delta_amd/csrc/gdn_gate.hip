// gdn_gate.hip -- fused gate kernel (elementwise, HBM-bound).
//
// log_decay = -exp(A_log[h]) * softplus20(a + dt_bias[h]), gamma = exp(log_decay),
// beta = sigmoid(b): the "qwen" gate_activation of "com.microsoft.GatedDeltaNet"
// (Attributes) and the fused gate of the FlashInfer decode page.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

// Eight consecutive io elements of a or b at an element index that is a
// multiple of 8, widened to fp32 (one 16-byte or two 16-byte loads).
__device__ __forceinline__ void load8f(const __bf16* p, float* v) {
  const bf8 x = *reinterpret_cast<const bf8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}
__device__ __forceinline__ void load8f(const float* p, float* v) {
  const f4 x0 = reinterpret_cast<const f4*>(p)[0], x1 = reinterpret_cast<const f4*>(p)[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = x0[e];
    v[4 + e] = x1[e];
  }
}
__device__ __forceinline__ void store8f(float* p, const float* v) {
  reinterpret_cast<f4*>(p)[0] = f4{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f4*>(p)[1] = f4{v[4], v[5], v[6], v[7]};
}

// Each thread handles eight consecutive elements of the flattened
// [n_tokens, hv] arrays.  VEC (every pointer 16-byte aligned): whole groups
// of eight use vector loads and stores; the ragged end and unaligned calls
// take the element loop.  The head of element i is i mod hv, found once per
// thread and stepped from there.
template <typename IN, bool VEC>
__global__ void __launch_bounds__(256)
gate_kernel(const float* __restrict__ A_log, const float* __restrict__ dt_bias,
            const IN* __restrict__ a, const IN* __restrict__ b, int64_t n_elems, int hv,
            float* __restrict__ log_decay, float* __restrict__ gamma, float* __restrict__ beta) {
  const int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (base >= n_elems) return;
  int h0 = n_elems <= 0xffffffffLL ? (int)((uint32_t)base % (uint32_t)hv) : (int)(base % hv);
  int hs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hs[e] = h0;
    h0 = h0 + 1 == hv ? 0 : h0 + 1;
  }
  if (VEC && base + 8 <= n_elems) {
    float v[8], o[8];
    if (a) {
      load8f(a + base, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = gate_log_decay(A_log[hs[e]], dt_bias[hs[e]], v[e]);
      if (log_decay) store8f(log_decay + base, o);
      if (gamma) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = expf(o[e]);
        store8f(gamma + base, o);
      }
    }
    if (b) {
      load8f(b + base, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = sigmoidf(v[e]);
      store8f(beta + base, o);
    }
    return;
  }
  for (int e = 0; e < 8 && base + e < n_elems; ++e) {
    const int64_t i = base + e;
    if (a) {
      const float g = gate_log_decay(A_log[hs[e]], dt_bias[hs[e]], to_f32(a[i]));
      if (log_decay) log_decay[i] = g;
      if (gamma) gamma[i] = expf(g);
    }
    if (b) beta[i] = sigmoidf(to_f32(b[i]));
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
  const int64_t threads = (n + 7) / 8;
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
