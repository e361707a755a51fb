// Device-side building blocks shared by the gfx950 M²RNN kernels.
//
// Everything here is written for CDNA4 (gfx950): 64-lane wavefronts, the
// 16x16x4 fp32 / fp64 MFMA instructions, DPP row operations over 16-lane rows,
// and 8 XCDs that each own an L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2rnn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

template <typename Real>
struct Vec2;
template <>
struct Vec2<float> {
  using type = f32x2;
};
template <>
struct Vec2<double> {
  using type = f64x2;
};

template <typename Real>
struct Vec4;
template <>
struct Vec4<float> {
  using type = f32x4;
};
template <>
struct Vec4<double> {
  using type = f64x4;
};

// D = A * B + C for one 16x16 tile with a contraction of 4.  Lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] (both precisions); element r of its
// result holds D[acc_m<Real>(l / 16, r)][l % 16], where the row index differs
// between the two instructions: 4 g + r for fp32, 4 r + g for fp64 (rows are
// interleaved across the four 16-lane groups in the fp64 instruction).
__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f64x4 mfma_16x16x4(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

template <typename Real>
__device__ __forceinline__ constexpr int acc_m(int g, int r) {
  return sizeof(Real) == 4 ? 4 * g + r : 4 * r + g;
}
// Inverse of acc_m: the lane group and element holding accumulator row m.
template <typename Real>
__device__ __forceinline__ constexpr int acc_g(int m) {
  return sizeof(Real) == 4 ? (m >> 2) : (m & 3);
}
template <typename Real>
__device__ __forceinline__ constexpr int acc_r(int m) {
  return sizeof(Real) == 4 ? (m & 3) : (m >> 2);
}

// tanh(x) = sign(x) (1 - e) / (1 + e) with e = exp(-2|x|) = 2^(-2 log2(e) |x|).
// e lies in (0, 1], so neither term overflows; 1 - e is exact for e near 1
// (Sterbenz), which keeps the absolute error near 1e-7 over the whole line.
// Uses the hardware base-2 exponential and reciprocal (about 1 ulp each).
// The recurrence step works with the pre-activation scaled by 2 / ln 2,
// A' = (2 / ln 2) A: W and the rank-1 term are scaled once (W when it is
// loaded, k per step), so that the step's exponential needs no extra multiply.
template <typename Real>
constexpr Real kTanhScale = Real(2.8853900817779268147198493620037843);  // 2 / ln 2

// rc = 1 / (1 + e^{2A}) from A' = (2 / ln 2) A, so that tanh(A) = 1 - 2 rc.  For
// large |A| the exponential saturates to inf or 0 and rc to 0 or 1, so the
// identity still gives +-1.  fp32: hardware base-2 exponential and reciprocal.
__device__ __forceinline__ float tanh_rc_scaled(float xs) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(xs));
}
__device__ __forceinline__ double tanh_rc_scaled(double xs) { return 1.0 / (1.0 + ::exp2(xs)); }

// Four values of columns 16 c + m(g, r), r = 0..3 (m the MFMA accumulator row
// map), from a row of values starting at column 16 c.
__device__ __forceinline__ f32x4 cols4(const float* p, int g) {
  return *(const f32x4*)(p + 4 * g);
}
__device__ __forceinline__ f64x4 cols4(const double* p, int g) {
  return f64x4{p[g], p[4 + g], p[8 + g], p[12 + g]};
}

// Forces `x` to be computed at this point of the program (an empty volatile
// asm that reads and writes it cannot move across other volatile operations
// such as a barrier), without emitting any instruction.
__device__ __forceinline__ void pin_value(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin_value(double& x) { asm volatile("" : "+v"(x)); }
template <typename Real>
__device__ __forceinline__ void pin_values(Real& a, Real& b, Real& c, Real& d) {
  asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
// The same for a 4-vector (e.g. MFMA accumulators, which this moves into VGPRs
// at this point of the program).
__device__ __forceinline__ void pin_vec(f32x4& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin_vec(f64x4& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ float fma_r(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_r(double a, double b, double c) { return __builtin_fma(a, b, c); }

// DPP: read the value of another lane of the same 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_move(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// Sum over the 16 lanes of each DPP row (row_ror by 8, 4, 2, 1).  Every lane of
// the row ends with a sum; lane (row * 16) is the one callers read, so the
// association order is fixed and results are reproducible.
constexpr int kDppRowRor1 = 0x121;
constexpr int kDppRowRor2 = 0x122;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
template <typename Real>
__device__ __forceinline__ Real row16_sum(Real x) {
  x += dpp_move<kDppRowRor8>(x);
  x += dpp_move<kDppRowRor4>(x);
  x += dpp_move<kDppRowRor2>(x);
  x += dpp_move<kDppRowRor1>(x);
  return x;
}

// Four independent 16-lane row sums of h[r] * q, computed level by level
// (row_ror by 8, 4, 2, 1) so that each DPP reads a value written three
// instructions earlier (the DPP read-after-VALU-write hazard needs two).
// Lane 16 k of each row holds the row's sums, in a fixed association order.
// The volatile asm also keeps the reduction where it is placed in the step.
__device__ __forceinline__ f32x4 row16_sum_x4(f32x4 h, float q) {
  float y0, y1, y2, y3;
  asm volatile(
      "v_mul_f32 %0, %4, %8\n"
      "v_mul_f32 %1, %5, %8\n"
      "v_mul_f32 %2, %6, %8\n"
      "v_mul_f32 %3, %7, %8\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      : "=&v"(y0), "=&v"(y1), "=&v"(y2), "=&v"(y3)
      : "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(q));
  return f32x4{y0, y1, y2, y3};
}
// row16_sum_x4(h, q) together with the row sum of a fifth value e (returned
// in e), the five chains interleaved level by level.
__device__ __forceinline__ f32x4 row16_sum_x4_e(f32x4 h, float q, float& e) {
  float y0, y1, y2, y3;
  asm volatile(
      "v_mul_f32 %0, %5, %9\n"
      "v_mul_f32 %1, %6, %9\n"
      "v_mul_f32 %2, %7, %9\n"
      "v_mul_f32 %3, %8, %9\n"
      "v_add_f32_dpp %4, %4, %4 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %4, %4, %4 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %4, %4, %4 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %4, %4, %4 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      : "=&v"(y0), "=&v"(y1), "=&v"(y2), "=&v"(y3), "+v"(e)
      : "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(q));
  return f32x4{y0, y1, y2, y3};
}
__device__ __forceinline__ f64x4 row16_sum_x4(f64x4 h, double q);
__device__ __forceinline__ f64x4 row16_sum_x4_e(f64x4 h, double q, double& e) {
  e = row16_sum(e);
  return row16_sum_x4(h, q);
}
__device__ __forceinline__ f64x4 row16_sum_x4(f64x4 h, double q) {
  f64x4 y;
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = row16_sum(h[r] * q);
  return y;
}

// The first two levels of row16_sum_x4 (row_ror by 8, then 4): lane i of each
// 16-lane row ends with the sums of h[r] * q over rows i, i + 4, i + 8, i + 12
// (lanes 0..3 hold the four distinct partials; adding them in lane order
// finishes the row sum).
__device__ __forceinline__ f32x4 row16_partial4_x4(f32x4 h, float q) {
  float y0, y1, y2, y3;
  asm volatile(
      "v_mul_f32 %0, %4, %8\n"
      "v_mul_f32 %1, %5, %8\n"
      "v_mul_f32 %2, %6, %8\n"
      "v_mul_f32 %3, %7, %8\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %1, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %2, %2, %2 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %3, %3, %3 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      : "=&v"(y0), "=&v"(y1), "=&v"(y2), "=&v"(y3)
      : "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(q));
  return f32x4{y0, y1, y2, y3};
}
__device__ __forceinline__ f64x4 row16_partial4_x4(f64x4 h, double q) {
  f64x4 y;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    double x = h[r] * q;
    x += dpp_move<kDppRowRor8>(x);
    x += dpp_move<kDppRowRor4>(x);
    y[r] = x;
  }
  return y;
}

// Sum over the four 16-lane rows (lanes l, l^16, l^32, l^48); every lane gets
// the same value.  fp32: the gfx950 lane-swap instructions (v_permlane32_swap
// exchanges the two halves of the wave between two registers, v_permlane16_swap
// the odd and even rows), written as asm with explicit copies, two wait states
// around each swap.  fp64: cross-lane shuffles.
__device__ __forceinline__ float cross_row_sum(float x) {
  float y;
  asm volatile(
      "v_mov_b32 %1, %0\n"
      "s_nop 1\n"
      "v_permlane32_swap_b32 %0, %1\n"
      "s_nop 1\n"
      "v_add_f32 %0, %0, %1\n"
      "v_mov_b32 %1, %0\n"
      "s_nop 1\n"
      "v_permlane16_swap_b32 %0, %1\n"
      "s_nop 1\n"
      "v_add_f32 %0, %0, %1\n"
      : "+v"(x), "=&v"(y));
  return x;
}
__device__ __forceinline__ double cross_row_sum(double x) {
  x += __shfl_xor(x, 32, 64);
  x += __shfl_xor(x, 16, 64);
  return x;
}

// Workgroup id -> logical work id.  The dispatcher sends workgroup i to XCD
// i % 8; this gives each XCD one contiguous range of logical ids, so units
// with neighbouring ids (the K-row slabs of one head) share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  if (nblocks % kXcd != 0) return bid;
  return (bid % kXcd) * (nblocks / kXcd) + bid / kXcd;
}

// The value of x in lane m (m wave-uniform).
__device__ __forceinline__ float lane_value_r(float x, int m) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), m));
}
__device__ __forceinline__ double lane_value_r(double x, int m) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, m);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), m);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Widening loads of the k / v / q element types.
__device__ __forceinline__ float load_in(const float* p) { return *p; }
__device__ __forceinline__ float load_in(const uint16_t* p) {
  return __builtin_bit_cast(float, (uint32_t)(*p) << 16);
}
__device__ __forceinline__ double load_in(const double* p) { return *p; }

// The same conversions for a value already in a register.
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t x) { return __builtin_bit_cast(float, (uint32_t)x << 16); }
__device__ __forceinline__ double widen(double x) { return x; }

template <typename Real, typename InT>
__device__ __forceinline__ Real load_as(const InT* p) {
  return (Real)load_in(p);
}

// Load p[i] when `ok`, else 0.  The caller passes an index that is in bounds
// either way (clamped), so the load is issued unconditionally and the value is
// selected afterwards: a guarded load would become a branch whose join waits
// for the load, serialising the whole batch of prefetch loads.
template <typename Real, typename InT>
__device__ __forceinline__ Real load_sel(const InT* p, int64_t i, bool ok) {
  const Real x = load_as<Real>(p + i);
  return ok ? x : Real(0);
}
__device__ __forceinline__ int64_t clamp_idx(int64_t x, int64_t hi) { return x < hi ? x : hi; }

// out[row][j] = sum over slabs sl of part[sl][row][j] (in slab order)
//               + w_r[row mod N][j] * x[row][j],   rows = B T N token rows.
// Elementwise and HBM-bound.  `vec` (slab_sum_vec: fp32, V a multiple of 4,
// every array aligned for it): one 16-byte access per array and thread (8-byte
// for bf16 x); 32-bit indices (the launcher checks rows V < 2^31).
template <typename InT, typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_slab_sum_kernel(int rows, int N, int V, int nslab, int64_t slab_stride,
                          const Real* __restrict__ part, const InT* __restrict__ x,
                          const Real* __restrict__ w_r, Real* __restrict__ out, bool vec) {
  const int stride = gridDim.x * blockDim.x;
  if (sizeof(Real) == 4 && vec) {
    const int cpr = V >> 2;  // 4-column groups per row
    const int total = rows * cpr;
    for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
      const int row = c / cpr;
      const int j = (c - row * cpr) << 2;
      const int n = row % N;
      const int64_t i = (int64_t)row * V + j;
      f32x4 acc = *(const f32x4*)((const float*)part + i);
      for (int sl = 1; sl < nslab; ++sl) acc += *(const f32x4*)((const float*)part + sl * slab_stride + i);
      const f32x4 w = *(const f32x4*)((const float*)w_r + (int64_t)n * V + j);
      f32x4 xv;
      if constexpr (sizeof(InT) == 2) {
        const uint2 raw = *(const uint2*)(x + i);
        xv = f32x4{__builtin_bit_cast(float, raw.x << 16), __builtin_bit_cast(float, raw.x & 0xffff0000u),
                   __builtin_bit_cast(float, raw.y << 16), __builtin_bit_cast(float, raw.y & 0xffff0000u)};
      } else {
        xv = *(const f32x4*)((const float*)x + i);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(w[r], xv[r], acc[r]);
      *(f32x4*)((float*)out + i) = acc;
    }
  } else {
    const int total = rows * V;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
      const int row = e / V;
      const int j = e - row * V;
      const int n = row % N;
      Real acc = part[e];
      for (int sl = 1; sl < nslab; ++sl) acc += part[sl * slab_stride + e];
      out[e] = fma_r(w_r[(int64_t)n * V + j], (Real)load_in(x + e), acc);
    }
  }
}

// Whether m2rnn_slab_sum_kernel may take its vector path for these arrays.
template <typename InT, typename Real>
inline bool slab_sum_vec(int64_t V, const void* part, const void* x, const void* w_r,
                         const void* out) {
  const uintptr_t xa = sizeof(InT) == 2 ? 7 : 15;
  return sizeof(Real) == 4 && (V & 3) == 0 && (((uintptr_t)part | (uintptr_t)w_r | (uintptr_t)out) & 15) == 0 &&
         ((uintptr_t)x & xa) == 0;
}

}  // namespace m2rnn
