// The elementwise parts of the M²RNN block around the recurrence, for gfx950
// (review of "M²RNN: Non-Linear RNNs with Matrix-Valued States for Scalable
// Language Modeling", section 2.3, Eq. 14-23):
//   prologue  out = SiLU(u),  u_t = bias + sum_{i<4} w[i] x_{t-3+i}   (depthwise,
//             causal, zero history), on each of q, k, v after their projections;
//   epilogue  out = gamma (.) z / sqrt(mean(z^2) + eps),  z = y (.) SiLU(g_pre)
//             (gate first, then RMSNorm over the token's channels);
// and their backwards.  All of it is bound by HBM bandwidth: every kernel
// streams its tensors once with coalesced accesses (threads of a wave on
// consecutive channels), computes in the state precision and rounds outputs
// stored as bf16 to nearest even.  Parameter gradients (dw, dbias, dgamma)
// are sums over the batch and time, formed as per-block partials and summed
// in a fixed order by a second kernel (no atomics: reproducible).

#include <type_traits>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

namespace {

constexpr int kConvTaps = 4;
constexpr int kConvRun = 64;   // time steps per thread in the convolution backward
constexpr int kConvRunFwd = 16;  // and in the forward (more threads in flight)
constexpr int kColRows = 256;  // rows per partial of the dgamma column sums

__device__ __forceinline__ float dev_exp_(float x) { return __expf(x); }
__device__ __forceinline__ double dev_exp_(double x) { return exp(x); }
__device__ __forceinline__ float dev_rsqrt_(float x) { return __frsqrt_rn(x); }
__device__ __forceinline__ double dev_rsqrt_(double x) { return 1.0 / sqrt(x); }

// sigmoid split at 0 so that the exponential never overflows
template <typename Real>
__device__ __forceinline__ Real sigmoid_(Real x) {
  const Real e = dev_exp_(x >= Real(0) ? -x : x);
  return x >= Real(0) ? Real(1) / (Real(1) + e) : e / (Real(1) + e);
}

// storage conversions: bf16 values widen exactly and are written rounded to
// nearest even (finite values)
template <typename T>
struct Io;
template <>
struct Io<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
};
template <>
struct Io<double> {
  __device__ static double load(const double* p) { return *p; }
  __device__ static void store(double* p, double v) { *p = v; }
};
template <>
struct Io<uint16_t> {
  __device__ static float load(const uint16_t* p) {
    return __builtin_bit_cast(float, (uint32_t)(*p) << 16);
  }
  __device__ static void store(uint16_t* p, double v) { store(p, (float)v); }
  __device__ static void store(uint16_t* p, float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    *p = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  }
};

}  // namespace

// ---------------------------------------------------------------- prologue

// Four consecutive channels of an io array: 16-byte (fp32) or 8-byte (bf16)
// accesses.
__device__ __forceinline__ f32x4 load4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 load4(const uint16_t* p) {
  const uint2 u = *(const uint2*)p;
  return f32x4{__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xFFFF0000u),
               __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xFFFF0000u)};
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *(f32x4*)p = v; }
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ void store4(uint16_t* p, f32x4 v) {
  *(uint2*)p = uint2{bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16)};
}


// One thread per (b, channel, run of kConvRun steps); the threads of a wave
// take consecutive channels, so every load and store of a step is one
// contiguous segment.  The last three inputs slide through registers.
template <typename IoT, typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_conv_silu_kernel(int64_t T, int64_t C, int64_t runs, const IoT* __restrict__ x,
                           const Real* __restrict__ w, const Real* __restrict__ bias,
                           IoT* __restrict__ out) {
  // workgroup id = (b * runs + run) * cblocks + channel block
  const int64_t cblocks = (C + 255) / 256;
  const int64_t row = (int64_t)blockIdx.x / cblocks;
  const int64_t c = ((int64_t)blockIdx.x % cblocks) * 256 + threadIdx.x;
  if (c >= C) return;
  const int64_t b = row / runs;
  const int64_t t0 = (row % runs) * kConvRunFwd;
  const int64_t t1 = t0 + kConvRunFwd < T ? t0 + kConvRunFwd : T;
  const Real w0 = w[c * kConvTaps], w1 = w[c * kConvTaps + 1], w2 = w[c * kConvTaps + 2],
             w3 = w[c * kConvTaps + 3];
  const Real bc = bias ? bias[c] : Real(0);
  const IoT* xp = x + b * T * C + c;
  IoT* op = out + b * T * C + c;
  // x_{t0-3}, x_{t0-2}, x_{t0-1} (zero before the sequence)
  Real xm3 = t0 >= 3 ? (Real)Io<IoT>::load(xp + (t0 - 3) * C) : Real(0);
  Real xm2 = t0 >= 2 ? (Real)Io<IoT>::load(xp + (t0 - 2) * C) : Real(0);
  Real xm1 = t0 >= 1 ? (Real)Io<IoT>::load(xp + (t0 - 1) * C) : Real(0);
#pragma unroll 8
  for (int64_t t = t0; t < t1; ++t) {
    const Real xt = (Real)Io<IoT>::load(xp + t * C);
    const Real u = bc + w0 * xm3 + w1 * xm2 + w2 * xm1 + w3 * xt;
    Io<IoT>::store(op + t * C, u * sigmoid_(u));
    xm3 = xm2;
    xm2 = xm1;
    xm1 = xt;
  }
}

// Backward, same decomposition.  du_t = dout_t silu'(u_t) is recomputed for
// t0 <= t < t1 + 3 (x from t0 - 3); dx_s = sum_i w[i] du_{s+3-i} is emitted
// once du_{s+3} is known.  The run's sums of du_t x_{t-3+i} and du_t go to a
// partial [b * runs + run][c][5].
template <typename IoT, typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_conv_silu_bwd_kernel(int64_t T, int64_t C, int64_t runs, const IoT* __restrict__ x,
                               const Real* __restrict__ w, const Real* __restrict__ bias,
                               const Real* __restrict__ dout, Real* __restrict__ dx,
                               Real* __restrict__ part) {
  const int64_t cblocks = (C + 255) / 256;
  const int64_t row = (int64_t)blockIdx.x / cblocks;
  const int64_t c = ((int64_t)blockIdx.x % cblocks) * 256 + threadIdx.x;
  if (c >= C) return;
  const int64_t b = row / runs;
  const int64_t t0 = (row % runs) * kConvRun;
  const int64_t t1 = t0 + kConvRun < T ? t0 + kConvRun : T;
  const int64_t t2 = t1 + 3 < T ? t1 + 3 : T;  // du is needed up to t1 + 2
  const Real w0 = w[c * kConvTaps], w1 = w[c * kConvTaps + 1], w2 = w[c * kConvTaps + 2],
             w3 = w[c * kConvTaps + 3];
  const Real bc = bias ? bias[c] : Real(0);
  const IoT* xp = x + b * T * C + c;
  const Real* gp = dout + b * T * C + c;
  Real* dxp = dx + b * T * C + c;
  Real xm3 = t0 >= 3 ? (Real)Io<IoT>::load(xp + (t0 - 3) * C) : Real(0);
  Real xm2 = t0 >= 2 ? (Real)Io<IoT>::load(xp + (t0 - 2) * C) : Real(0);
  Real xm1 = t0 >= 1 ? (Real)Io<IoT>::load(xp + (t0 - 1) * C) : Real(0);
  Real d3 = 0, d2 = 0, d1 = 0;  // du_{t-3}, du_{t-2}, du_{t-1}
  Real s0 = 0, s1 = 0, s2 = 0, s3 = 0, sb = 0;
  for (int64_t t = t0; t < t1 + 3; ++t) {
    Real du = 0;
    if (t < t2) {
      const Real xt = (Real)Io<IoT>::load(xp + t * C);
      const Real u = bc + w0 * xm3 + w1 * xm2 + w2 * xm1 + w3 * xt;
      const Real sg = sigmoid_(u);
      du = gp[t * C] * sg * (Real(1) + u * (Real(1) - sg));
      if (t < t1) {
        s0 += du * xm3;
        s1 += du * xm2;
        s2 += du * xm1;
        s3 += du * xt;
        sb += du;
      }
      xm3 = xm2;
      xm2 = xm1;
      xm1 = xt;
    }
    // dx_{t-3} = w3 du_{t-3} + w2 du_{t-2} + w1 du_{t-1} + w0 du_t
    if (t - 3 >= t0) dxp[(t - 3) * C] = w3 * d3 + w2 * d2 + w1 * d1 + w0 * du;
    d3 = d2;
    d2 = d1;
    d1 = du;
  }
  Real* pp = part + (row * C + c) * 5;
  pp[0] = s0;
  pp[1] = s1;
  pp[2] = s2;
  pp[3] = s3;
  pp[4] = sb;
}

// The same two kernels for fp32 parameters and C % 4 == 0: a thread takes
// four consecutive channels (16-byte fp32 / 8-byte bf16 accesses).
template <typename IoT>
__global__ void __launch_bounds__(256)
    m2rnn_conv_silu_vec_kernel(int64_t T, int64_t C, int64_t runs, const IoT* __restrict__ x,
                               const float* __restrict__ w, const float* __restrict__ bias,
                               IoT* __restrict__ out) {
  const int64_t C4 = C / 4;
  const int64_t cblocks = (C4 + 255) / 256;
  const int64_t row = (int64_t)blockIdx.x / cblocks;
  const int64_t c4 = ((int64_t)blockIdx.x % cblocks) * 256 + threadIdx.x;
  if (c4 >= C4) return;
  const int64_t c = c4 * 4;
  const int64_t b = row / runs;
  const int64_t t0 = (row % runs) * kConvRunFwd;
  const int64_t t1 = t0 + kConvRunFwd < T ? t0 + kConvRunFwd : T;
  f32x4 wt[kConvTaps];  // wt[i][k] = w[c + k][i]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x4 wk = *(const f32x4*)(w + (c + k) * kConvTaps);
#pragma unroll
    for (int i = 0; i < kConvTaps; ++i) wt[i][k] = wk[i];
  }
  const f32x4 bc = bias ? *(const f32x4*)(bias + c) : f32x4{0, 0, 0, 0};
  const IoT* xp = x + b * T * C + c;
  IoT* op = out + b * T * C + c;
  const f32x4 zero{0, 0, 0, 0};
  f32x4 xm3 = t0 >= 3 ? load4(xp + (t0 - 3) * C) : zero;
  f32x4 xm2 = t0 >= 2 ? load4(xp + (t0 - 2) * C) : zero;
  f32x4 xm1 = t0 >= 1 ? load4(xp + (t0 - 1) * C) : zero;
#pragma unroll 8
  for (int64_t t = t0; t < t1; ++t) {
    const f32x4 xt = load4(xp + t * C);
    const f32x4 u = bc + wt[0] * xm3 + wt[1] * xm2 + wt[2] * xm1 + wt[3] * xt;
    f32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = u[k] * sigmoid_(u[k]);
    store4(op + t * C, o);
    xm3 = xm2;
    xm2 = xm1;
    xm1 = xt;
  }
}

template <typename IoT>
__global__ void __launch_bounds__(256)
    m2rnn_conv_silu_bwd_vec_kernel(int64_t T, int64_t C, int64_t runs, const IoT* __restrict__ x,
                                   const float* __restrict__ w, const float* __restrict__ bias,
                                   const float* __restrict__ dout, float* __restrict__ dx,
                                   float* __restrict__ part) {
  const int64_t C4 = C / 4;
  const int64_t cblocks = (C4 + 255) / 256;
  const int64_t row = (int64_t)blockIdx.x / cblocks;
  const int64_t c4 = ((int64_t)blockIdx.x % cblocks) * 256 + threadIdx.x;
  if (c4 >= C4) return;
  const int64_t c = c4 * 4;
  const int64_t b = row / runs;
  const int64_t t0 = (row % runs) * kConvRun;
  const int64_t t1 = t0 + kConvRun < T ? t0 + kConvRun : T;
  const int64_t t2 = t1 + 3 < T ? t1 + 3 : T;
  f32x4 wt[kConvTaps];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x4 wk = *(const f32x4*)(w + (c + k) * kConvTaps);
#pragma unroll
    for (int i = 0; i < kConvTaps; ++i) wt[i][k] = wk[i];
  }
  const f32x4 zero{0, 0, 0, 0};
  const f32x4 bc = bias ? *(const f32x4*)(bias + c) : zero;
  const IoT* xp = x + b * T * C + c;
  const float* gp = dout + b * T * C + c;
  float* dxp = dx + b * T * C + c;
  f32x4 xm3 = t0 >= 3 ? load4(xp + (t0 - 3) * C) : zero;
  f32x4 xm2 = t0 >= 2 ? load4(xp + (t0 - 2) * C) : zero;
  f32x4 xm1 = t0 >= 1 ? load4(xp + (t0 - 1) * C) : zero;
  f32x4 d3 = zero, d2 = zero, d1 = zero;
  f32x4 s0 = zero, s1 = zero, s2 = zero, s3 = zero, sb = zero;
  for (int64_t t = t0; t < t1 + 3; ++t) {
    f32x4 du = zero;
    if (t < t2) {
      const f32x4 xt = load4(xp + t * C);
      const f32x4 u = bc + wt[0] * xm3 + wt[1] * xm2 + wt[2] * xm1 + wt[3] * xt;
      const f32x4 g = *(const f32x4*)(gp + t * C);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float sg = sigmoid_(u[k]);
        du[k] = g[k] * sg * (1.0f + u[k] * (1.0f - sg));
      }
      if (t < t1) {
        s0 += du * xm3;
        s1 += du * xm2;
        s2 += du * xm1;
        s3 += du * xt;
        sb += du;
      }
      xm3 = xm2;
      xm2 = xm1;
      xm1 = xt;
    }
    if (t - 3 >= t0) store4(dxp + (t - 3) * C, wt[3] * d3 + wt[2] * d2 + wt[1] * d1 + wt[0] * du);
    d3 = d2;
    d2 = d1;
    d1 = du;
  }
  float* pp = part + (row * C + c) * 5;  // [row][c + k][5]: 20 consecutive values
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    pp[5 * k + 0] = s0[k];
    pp[5 * k + 1] = s1[k];
    pp[5 * k + 2] = s2[k];
    pp[5 * k + 3] = s3[k];
    pp[5 * k + 4] = sb[k];
  }
}

// Column sums of a [P, ncol] array of partials: one block per 64 columns, its
// four waves summing rows p = grp, grp + 4, ..., the four group sums added in
// a fixed order.  MODE 0 writes out0[col]; MODE 1 splits the convolution's
// columns col = 5 c + i into dw[c][i] (i < 4) and dbias[c] (i = 4).
template <typename Real, int MODE>
__global__ void __launch_bounds__(256)
    m2rnn_rows_sum_kernel(int64_t P, int64_t ncol, const Real* __restrict__ part,
                          Real* __restrict__ out0, Real* __restrict__ out1) {
  __shared__ Real red[4][64];
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * 64 + lane;
  Real sum = 0;
  if (col < ncol) {
#pragma unroll 8
    for (int64_t q = grp; q < P; q += 4) sum += part[q * ncol + col];
  }
  red[grp][lane] = sum;
  __syncthreads();
  if (grp != 0 || col >= ncol) return;
  const Real total = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
  if (MODE == 0) {
    out0[col] = total;
  } else {
    const int64_t c = col / 5, i = col % 5;
    if (i < kConvTaps) out0[c * kConvTaps + i] = total;
    else if (out1) out1[c] = total;
  }
}

// ---------------------------------------------------------------- epilogue

// Sum over the 64 lanes of a wave (DPP row sums, then across the rows); every
// lane gets the same value, in a fixed association order.
template <typename Real>
__device__ __forceinline__ Real wave_sum(Real x) {
  return cross_row_sum(row16_sum(x));
}

// One wave per token row (four rows per workgroup): the sum of z^2 over the
// row's D channels, then the normalised, scaled output.  The second pass
// reads the row again (it is still in cache).  rstd [rows] keeps
// 1 / sqrt(mean(z^2) + eps) for the backward (optional).
template <typename IoT, typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_gate_rmsnorm_kernel(int64_t rows, int64_t D, Real eps, const Real* __restrict__ y,
                              const IoT* __restrict__ g_pre, const Real* __restrict__ gamma,
                              IoT* __restrict__ out, Real* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves leave together
  const Real* yp = y + row * D;
  const IoT* gp = g_pre + row * D;
  Real ss = 0;
  for (int64_t d = lane; d < D; d += 64) {
    const Real gv = (Real)Io<IoT>::load(gp + d);
    const Real z = yp[d] * gv * sigmoid_(gv);
    ss += z * z;
  }
  const Real r = dev_rsqrt_(wave_sum(ss) / Real(D) + eps);
  if (rstd && lane == 0) rstd[row] = r;
  IoT* op = out + row * D;
  for (int64_t d = lane; d < D; d += 64) {
    const Real gv = (Real)Io<IoT>::load(gp + d);
    const Real z = yp[d] * gv * sigmoid_(gv);
    Io<IoT>::store(op + d, gamma[d] * z * r);
  }
}

// Backward per row: with zh = z r, dzh = dout gamma, m = mean(dzh zh):
// dz = r (dzh - zh m), dy = dz SiLU(g_pre), dg_pre = dz y silu'(g_pre).
// r is recomputed (one pass), m takes a second, the outputs a third; rstd
// [rows] receives r for the dgamma column sums.
template <typename IoT, typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_gate_rmsnorm_bwd_kernel(int64_t rows, int64_t D, Real eps, const Real* __restrict__ y,
                                  const IoT* __restrict__ g_pre, const Real* __restrict__ gamma,
                                  const Real* __restrict__ dout, Real* __restrict__ dy,
                                  Real* __restrict__ dg_pre, Real* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const Real* yp = y + row * D;
  const IoT* gp = g_pre + row * D;
  const Real* dp = dout + row * D;
  Real ss = 0, sm = 0;
  for (int64_t d = lane; d < D; d += 64) {
    const Real gv = (Real)Io<IoT>::load(gp + d);
    const Real z = yp[d] * gv * sigmoid_(gv);
    ss += z * z;
    sm += dp[d] * gamma[d] * z;
  }
  const Real r = dev_rsqrt_(wave_sum(ss) / Real(D) + eps);
  const Real m = wave_sum(sm) * r / Real(D);  // mean(dzh zh) = r mean(dzh z)
  if (lane == 0) rstd[row] = r;
  Real* dyp = dy + row * D;
  Real* dgp = dg_pre + row * D;
  for (int64_t d = lane; d < D; d += 64) {
    const Real gv = (Real)Io<IoT>::load(gp + d);
    const Real sg = sigmoid_(gv);
    const Real g = gv * sg;
    const Real yv = yp[d];
    const Real z = yv * g;
    const Real dz = r * (dp[d] * gamma[d] - z * r * m);
    dyp[d] = dz * g;
    dgp[d] = dz * yv * sg * (Real(1) + gv * (Real(1) - sg));
  }
}

// Rows of at most kVecChunks * 256 channels, fp32 parameters, D % 4 == 0: each
// lane holds chunks of four consecutive channels (chunk j covers channels
// 4 (64 j + lane) ..), so one pass over the row reads it once and keeps z in
// registers for the output.
constexpr int kVecChunks = 4;

template <typename IoT>
__global__ void __launch_bounds__(256)
    m2rnn_gate_rmsnorm_vec_kernel(int64_t rows, int64_t D, float eps, const float* __restrict__ y,
                                  const IoT* __restrict__ g_pre, const float* __restrict__ gamma,
                                  IoT* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* yp = y + row * D;
  const IoT* gp = g_pre + row * D;
  f32x4 z[kVecChunks];
  float ss = 0;
#pragma unroll
  for (int j = 0; j < kVecChunks; ++j) {
    const int64_t d0 = (int64_t)(j * 64 + lane) * 4;
    z[j] = f32x4{0, 0, 0, 0};
    if (d0 < D) {
      const f32x4 y4 = load4(yp + d0), g4 = load4(gp + d0);
#pragma unroll
      for (int r = 0; r < 4; ++r) z[j][r] = y4[r] * g4[r] * sigmoid_(g4[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) ss += z[j][r] * z[j][r];
  }
  const float rs = dev_rsqrt_(wave_sum(ss) / (float)D + eps);
  IoT* op = out + row * D;
#pragma unroll
  for (int j = 0; j < kVecChunks; ++j) {
    const int64_t d0 = (int64_t)(j * 64 + lane) * 4;
    if (d0 < D) store4(op + d0, load4(gamma + d0) * z[j] * rs);
  }
}

// Backward on the same layout.  Each wave takes rows row0 + k * stride in
// turn and keeps its lanes' shares of dgamma in registers; the four waves of
// a workgroup add theirs into LDS in wave order and the workgroup writes one
// partial row [blockIdx][D] (summed afterwards by m2rnn_rows_sum_kernel).
template <typename IoT>
__global__ void __launch_bounds__(256)
    m2rnn_gate_rmsnorm_bwd_vec_kernel(int64_t rows, int64_t D, float eps,
                                      const float* __restrict__ y, const IoT* __restrict__ g_pre,
                                      const float* __restrict__ gamma,
                                      const float* __restrict__ dout, float* __restrict__ dy,
                                      float* __restrict__ dg_pre, float* __restrict__ part) {
  __shared__ f32x4 acc_l[kVecChunks * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  f32x4 gm[kVecChunks], dga[kVecChunks];
#pragma unroll
  for (int j = 0; j < kVecChunks; ++j) {
    const int64_t d0 = (int64_t)(j * 64 + lane) * 4;
    gm[j] = d0 < D ? load4(gamma + d0) : f32x4{0, 0, 0, 0};
    dga[j] = f32x4{0, 0, 0, 0};
  }
  const int64_t stride = (int64_t)gridDim.x * 4;
  for (int64_t row = (int64_t)blockIdx.x * 4 + w; row < rows; row += stride) {
    const float* yp = y + row * D;
    const IoT* gp = g_pre + row * D;
    const float* dp = dout + row * D;
    f32x4 y4[kVecChunks], g4[kVecChunks], d4[kVecChunks];
    float ss = 0, sm = 0;
#pragma unroll
    for (int j = 0; j < kVecChunks; ++j) {
      const int64_t d0 = (int64_t)(j * 64 + lane) * 4;
      y4[j] = g4[j] = d4[j] = f32x4{0, 0, 0, 0};
      if (d0 < D) {
        y4[j] = load4(yp + d0);
        g4[j] = load4(gp + d0);
        d4[j] = load4(dp + d0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float z = y4[j][r] * g4[j][r] * sigmoid_(g4[j][r]);
        ss += z * z;
        sm += d4[j][r] * gm[j][r] * z;
      }
    }
    const float rs = dev_rsqrt_(wave_sum(ss) / (float)D + eps);
    const float m = wave_sum(sm) * rs / (float)D;
#pragma unroll
    for (int j = 0; j < kVecChunks; ++j) {
      const int64_t d0 = (int64_t)(j * 64 + lane) * 4;
      f32x4 dyv, dgv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = g4[j][r], sg = sigmoid_(gv), g = gv * sg;
        const float z = y4[j][r] * g;
        const float dz = rs * (d4[j][r] * gm[j][r] - z * rs * m);
        dyv[r] = dz * g;
        dgv[r] = dz * y4[j][r] * sg * (1.0f + gv * (1.0f - sg));
        dga[j][r] += d4[j][r] * z * rs;
      }
      if (d0 < D) {
        store4(dy + row * D + d0, dyv);
        store4(dg_pre + row * D + d0, dgv);
      }
    }
  }
  // the workgroup's dgamma partial: waves add in order 0, 1, 2, 3
  for (int k = 0; k < 4; ++k) {
    if (w == k) {
#pragma unroll
      for (int j = 0; j < kVecChunks; ++j)
        acc_l[j * 64 + lane] = k == 0 ? dga[j] : acc_l[j * 64 + lane] + dga[j];
    }
    __syncthreads();
  }
  for (int64_t d = threadIdx.x; d < D; d += 256)
    part[(int64_t)blockIdx.x * D + d] = ((const float*)acc_l)[d];
}

// dgamma[d] = sum_rows dout[row][d] z[row][d] rstd[row]: stage 1, one block per
// (kColRows rows, 256 channels), one channel per thread, rows in order.
template <typename IoT, typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_dgamma_part_kernel(int64_t rows, int64_t D, const Real* __restrict__ y,
                             const IoT* __restrict__ g_pre, const Real* __restrict__ dout,
                             const Real* __restrict__ rstd, Real* __restrict__ part) {
  // workgroup id = row block * dblocks + channel block
  const int64_t dblocks = (D + 255) / 256;
  const int64_t blk = (int64_t)blockIdx.x / dblocks;
  const int64_t d = ((int64_t)blockIdx.x % dblocks) * 256 + threadIdx.x;
  if (d >= D) return;
  const int64_t r0 = blk * kColRows;
  const int64_t r1 = r0 + kColRows < rows ? r0 + kColRows : rows;
  Real s = 0;
  for (int64_t r = r0; r < r1; ++r) {
    const Real gv = (Real)Io<IoT>::load(g_pre + r * D + d);
    s += dout[r * D + d] * y[r * D + d] * gv * sigmoid_(gv) * rstd[r];
  }
  part[blk * D + d] = s;
}

// ---------------------------------------------------------------- launchers

size_t conv_bwd_workspace_elems(int64_t B, int64_t T, int64_t C) {
  const int64_t runs = (T + kConvRun - 1) / kConvRun;
  return (size_t)B * runs * C * 5;
}

// workgroups of the vectorised epilogue backward (each writes one dgamma partial)
static int64_t rms_bwd_vec_groups(int64_t rows) {
  const int64_t g = (rows + 3) / 4;
  return g < 1024 ? g : 1024;
}

size_t rmsnorm_bwd_workspace_elems(int64_t rows, int64_t D) {
  const int64_t nblk = (rows + kColRows - 1) / kColRows;
  const int64_t vg = rms_bwd_vec_groups(rows);
  return align_up((size_t)rows, 64) + (size_t)(nblk > vg ? nblk : vg) * D;
}

namespace {

// the four-channel convolution kernels apply: fp32 parameters, C % 4 == 0,
// 16-byte aligned fp32 arrays and 8-byte aligned bf16 ones
template <typename IoT, typename Real>
bool conv_vec_ok(const BlockConvArgs& a, bool bwd) {
  if (!std::is_same_v<Real, float> || (a.C & 3) != 0) return false;
  auto al = [](const void* p, uintptr_t n) { return p == nullptr || ((uintptr_t)p % n) == 0; };
  const uintptr_t io_al = sizeof(IoT) == 2 ? 8 : 16;
  bool ok = al(a.x, io_al) && al(a.w, 16) && al(a.bias, 16);
  if (bwd) ok = ok && al(a.dout, 16) && al(a.dx, 16);
  else ok = ok && al(a.out, io_al);
  return ok;
}

template <typename IoT, typename Real>
hipError_t conv_fwd_t(const BlockConvArgs& a, hipStream_t stream) {
  const int64_t runs = (a.T + kConvRunFwd - 1) / kConvRunFwd;
  if constexpr (std::is_same_v<Real, float>) {
    if (conv_vec_ok<IoT, Real>(a, false)) {
      const dim3 grid((unsigned)((a.C / 4 + 255) / 256 * a.B * runs));
      hipLaunchKernelGGL((m2rnn_conv_silu_vec_kernel<IoT>), grid, dim3(256), 0, stream, a.T,
                         a.C, runs, (const IoT*)a.x, (const float*)a.w, (const float*)a.bias,
                         (IoT*)a.out);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)((a.C + 255) / 256 * a.B * runs));
  hipLaunchKernelGGL((m2rnn_conv_silu_kernel<IoT, Real>), grid, dim3(256), 0, stream, a.T, a.C,
                     runs, (const IoT*)a.x, (const Real*)a.w, (const Real*)a.bias, (IoT*)a.out);
  return hipGetLastError();
}

template <typename IoT, typename Real>
hipError_t conv_bwd_t(const BlockConvArgs& a, hipStream_t stream) {
  const int64_t runs = (a.T + kConvRun - 1) / kConvRun;
  const int64_t rows = a.B * runs;
  Real* part = (Real*)a.ws;
  bool done = false;
  if constexpr (std::is_same_v<Real, float>) {
    if (conv_vec_ok<IoT, Real>(a, true)) {
      const dim3 grid((unsigned)((a.C / 4 + 255) / 256 * rows));
      hipLaunchKernelGGL((m2rnn_conv_silu_bwd_vec_kernel<IoT>), grid, dim3(256), 0, stream, a.T,
                         a.C, runs, (const IoT*)a.x, (const float*)a.w, (const float*)a.bias,
                         (const float*)a.dout, (float*)a.dx, part);
      done = true;
    }
  }
  if (!done) {
    const dim3 grid((unsigned)((a.C + 255) / 256 * rows));
    hipLaunchKernelGGL((m2rnn_conv_silu_bwd_kernel<IoT, Real>), grid, dim3(256), 0, stream, a.T,
                       a.C, runs, (const IoT*)a.x, (const Real*)a.w, (const Real*)a.bias,
                       (const Real*)a.dout, (Real*)a.dx, part);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((m2rnn_rows_sum_kernel<Real, 1>), dim3((unsigned)((a.C * 5 + 63) / 64)),
                     dim3(256), 0, stream, rows, a.C * 5, (const Real*)part, (Real*)a.dw,
                     (Real*)a.dbias);
  return hipGetLastError();
}

// the vectorised epilogue kernels apply: fp32 parameters, D % 4 == 0, at most
// kVecChunks * 256 channels, 16-byte aligned fp32 arrays and 8-byte aligned
// bf16 ones
template <typename IoT, typename Real>
bool rms_vec_ok(const BlockNormArgs& a, bool bwd) {
  if (!std::is_same_v<Real, float> || (a.D & 3) != 0 || a.D > kVecChunks * 256) return false;
  auto al = [](const void* p, uintptr_t n) { return p == nullptr || ((uintptr_t)p % n) == 0; };
  const uintptr_t io_al = sizeof(IoT) == 2 ? 8 : 16;
  bool ok = al(a.y, 16) && al(a.gamma, 16) && al(a.g_pre, io_al);
  if (bwd) ok = ok && al(a.dout, 16) && al(a.dy, 16) && al(a.dg_pre, 16);
  else ok = ok && al(a.out, io_al);
  return ok;
}

template <typename IoT, typename Real>
hipError_t rms_fwd_t(const BlockNormArgs& a, hipStream_t stream) {
  if constexpr (std::is_same_v<Real, float>) {
    if (rms_vec_ok<IoT, Real>(a, false)) {
      hipLaunchKernelGGL((m2rnn_gate_rmsnorm_vec_kernel<IoT>), dim3((unsigned)((a.rows + 3) / 4)),
                         dim3(256), 0, stream, a.rows, a.D, (float)a.eps, (const float*)a.y,
                         (const IoT*)a.g_pre, (const float*)a.gamma, (IoT*)a.out);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((m2rnn_gate_rmsnorm_kernel<IoT, Real>), dim3((unsigned)((a.rows + 3) / 4)),
                     dim3(256), 0, stream, a.rows, a.D, (Real)a.eps, (const Real*)a.y,
                     (const IoT*)a.g_pre, (const Real*)a.gamma, (IoT*)a.out, (Real*)nullptr);
  return hipGetLastError();
}

template <typename IoT, typename Real>
hipError_t rms_bwd_t(const BlockNormArgs& a, hipStream_t stream) {
  Real* rstd = (Real*)a.ws;
  Real* part = rstd + align_up((size_t)a.rows, 64);
  hipError_t err;
  if constexpr (std::is_same_v<Real, float>) {
    if (rms_vec_ok<IoT, Real>(a, true)) {
      const int64_t groups = rms_bwd_vec_groups(a.rows);
      hipLaunchKernelGGL((m2rnn_gate_rmsnorm_bwd_vec_kernel<IoT>), dim3((unsigned)groups),
                         dim3(256), 0, stream, a.rows, a.D, (float)a.eps, (const float*)a.y,
                         (const IoT*)a.g_pre, (const float*)a.gamma, (const float*)a.dout,
                         (float*)a.dy, (float*)a.dg_pre, part);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      hipLaunchKernelGGL((m2rnn_rows_sum_kernel<Real, 0>), dim3((unsigned)((a.D + 63) / 64)),
                         dim3(256), 0, stream, groups, a.D, (const Real*)part, (Real*)a.dgamma,
                         (Real*)nullptr);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((m2rnn_gate_rmsnorm_bwd_kernel<IoT, Real>),
                     dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0, stream, a.rows, a.D,
                     (Real)a.eps, (const Real*)a.y, (const IoT*)a.g_pre, (const Real*)a.gamma,
                     (const Real*)a.dout, (Real*)a.dy, (Real*)a.dg_pre, rstd);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t nblk = (a.rows + kColRows - 1) / kColRows;
  hipLaunchKernelGGL((m2rnn_dgamma_part_kernel<IoT, Real>),
                     dim3((unsigned)((a.D + 255) / 256 * nblk)), dim3(256), 0, stream,
                     a.rows, a.D, (const Real*)a.y, (const IoT*)a.g_pre, (const Real*)a.dout,
                     (const Real*)rstd, part);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((m2rnn_rows_sum_kernel<Real, 0>), dim3((unsigned)((a.D + 63) / 64)),
                     dim3(256), 0, stream, nblk, a.D, (const Real*)part, (Real*)a.dgamma,
                     (Real*)nullptr);
  return hipGetLastError();
}

template <template <typename, typename> class F, typename Args>
hipError_t dispatch(const Args& a, int io_dtype, int param_dtype, hipStream_t stream) {
  if (param_dtype == kF32) {
    if (io_dtype == kF32) return F<float, float>::run(a, stream);
    if (io_dtype == kBF16) return F<uint16_t, float>::run(a, stream);
  } else if (param_dtype == kF64) {
    if (io_dtype == kF64) return F<double, double>::run(a, stream);
    if (io_dtype == kBF16) return F<uint16_t, double>::run(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename IoT, typename Real>
struct ConvFwd {
  static hipError_t run(const BlockConvArgs& a, hipStream_t s) { return conv_fwd_t<IoT, Real>(a, s); }
};
template <typename IoT, typename Real>
struct ConvBwd {
  static hipError_t run(const BlockConvArgs& a, hipStream_t s) { return conv_bwd_t<IoT, Real>(a, s); }
};
template <typename IoT, typename Real>
struct RmsFwd {
  static hipError_t run(const BlockNormArgs& a, hipStream_t s) { return rms_fwd_t<IoT, Real>(a, s); }
};
template <typename IoT, typename Real>
struct RmsBwd {
  static hipError_t run(const BlockNormArgs& a, hipStream_t s) { return rms_bwd_t<IoT, Real>(a, s); }
};

}  // namespace

hipError_t launch_conv_silu(const BlockConvArgs& a, int io_dtype, int param_dtype, bool bwd,
                            hipStream_t stream) {
  return bwd ? dispatch<ConvBwd>(a, io_dtype, param_dtype, stream)
             : dispatch<ConvFwd>(a, io_dtype, param_dtype, stream);
}

hipError_t launch_gate_rmsnorm(const BlockNormArgs& a, int io_dtype, int param_dtype, bool bwd,
                               hipStream_t stream) {
  return bwd ? dispatch<RmsBwd>(a, io_dtype, param_dtype, stream)
             : dispatch<RmsFwd>(a, io_dtype, param_dtype, stream);
}

}  // namespace m2rnn
