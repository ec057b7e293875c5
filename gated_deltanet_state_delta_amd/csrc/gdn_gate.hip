// gdn_gate.hip -- fused gate kernel (elementwise, HBM-bound).
//
// log_decay = -exp(A_log[h]) * softplus20(a + dt_bias[h]), gamma = exp(log_decay),
// beta = sigmoid(b): the "qwen" gate_activation of "com.microsoft.GatedDeltaNet"
// (Attributes) and the fused gate of the FlashInfer decode page.  Each thread
// handles four consecutive elements of the flattened [n_tokens, hv] arrays.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

template <typename IN>
__global__ void __launch_bounds__(256)
gate_kernel(const float* __restrict__ A_log, const float* __restrict__ dt_bias,
            const IN* __restrict__ a, const IN* __restrict__ b, int64_t n_elems, int hv,
            float* __restrict__ log_decay, float* __restrict__ gamma, float* __restrict__ beta) {
  const int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t i = base + e;
    if (i >= n_elems) return;
    if (a) {
      const int h = (int)(i % hv);
      const float g = gate_log_decay(A_log[h], dt_bias[h], to_f32(a[i]));
      if (log_decay) log_decay[i] = g;
      if (gamma) gamma[i] = expf(g);
    }
    if (b) beta[i] = sigmoidf(to_f32(b[i]));
  }
}

hipError_t launch_gate(const float* A_log, const float* dt_bias, const void* a, const void* b,
                       int ab_dtype, int64_t n_tokens, int hv, float* log_decay, float* gamma,
                       float* beta, hipStream_t stream) {
  const int64_t n = n_tokens * hv;
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (ab_dtype == GDN_BF16) {
    hipLaunchKernelGGL(gate_kernel<__bf16>, grid, dim3(256), 0, stream, A_log, dt_bias,
                       (const __bf16*)a, (const __bf16*)b, n, hv, log_decay, gamma, beta);
  } else {
    hipLaunchKernelGGL(gate_kernel<float>, grid, dim3(256), 0, stream, A_log, dt_bias,
                       (const float*)a, (const float*)b, n, hv, log_decay, gamma, beta);
  }
  return hipGetLastError();
}

}  // namespace gdn
