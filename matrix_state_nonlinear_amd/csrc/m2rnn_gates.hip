// Forget-gate precompute for gfx950.
//
// The gate never reads the recurrent state (M²RNN review, section 2.2), so the
// whole [B, T, N] sequence is one elementwise pass, bound by HBM bandwidth:
//   sigmoid:       f = 1 / (1 + e^{-g})                    (pararnn "ParaM2RNN", Recurrence)
//   exp-softplus:  f = exp(-alpha_n softplus(a + beta_n))   (review Eq. 13 / 17)
// softplus(x) = max(x, 0) + log1p(e^{-|x|}) and the sigmoid is split at 0, so
// no intermediate overflows.  exp / log1p are HIP's device-library functions.

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

__device__ __forceinline__ float dev_exp(float x) { return expf(x); }
__device__ __forceinline__ double dev_exp(double x) { return exp(x); }
__device__ __forceinline__ float dev_log1p(float x) { return log1pf(x); }
__device__ __forceinline__ double dev_log1p(double x) { return log1p(x); }

template <typename Real>
__device__ __forceinline__ Real gate_sigmoid(Real x) {
  if (x >= Real(0)) return Real(1) / (Real(1) + dev_exp(-x));
  const Real e = dev_exp(x);
  return e / (Real(1) + e);
}

template <typename Real>
__device__ __forceinline__ Real gate_softplus(Real x) {
  const Real ax = x < Real(0) ? -x : x;
  return (x > Real(0) ? x : Real(0)) + dev_log1p(dev_exp(-ax));
}

template <typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_gates_kernel(int64_t total, int64_t N, int kind, const Real* __restrict__ logit,
                       const Real* __restrict__ alpha, const Real* __restrict__ beta,
                       Real* __restrict__ f) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const Real x = logit[i];
    if (kind == kGateSigmoid) {
      f[i] = gate_sigmoid(x);
    } else {
      const int64_t n = i % N;
      f[i] = dev_exp(-alpha[n] * gate_softplus(x + beta[n]));
    }
  }
}

hipError_t launch_gates(int64_t B, int64_t T, int64_t N, int gate_kind, int dtype,
                        const void* logit, const void* alpha, const void* beta, void* f,
                        hipStream_t stream) {
  const int64_t total = B * T * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (dtype == kF32) {
    hipLaunchKernelGGL(m2rnn_gates_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       total, N, gate_kind, (const float*)logit, (const float*)alpha,
                       (const float*)beta, (float*)f);
  } else if (dtype == kF64) {
    hipLaunchKernelGGL(m2rnn_gates_kernel<double>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       total, N, gate_kind, (const double*)logit, (const double*)alpha,
                       (const double*)beta, (double*)f);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace m2rnn
