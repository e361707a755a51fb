// Parallel-in-time forward of the M²RNN recurrence by Newton's method, for gfx950.
//
// Method (pararnn-torch "ParaM2RNN" page, "Jacobian class" and "Parallel path":
// factorized Newton on the matrix residual; "ParaGRU" page, "Parallel path":
// Newton + scan from the guess h_t = F(0, x_t)).  The unknowns are the states
// X_1 .. X_T of every (batch, head) unit, the residual of step t is
// r_t = X_t - F(X_{t-1}) with F(X) = f X + (1 - f) tanh(X W + k v^T).  One
// iteration linearises F at the current iterate and solves the linear
// recurrence for the update d_t = X_t^new - X_t:
//     d_t = d_{t-1} A_t - r_t,   d_0 = 0,
// acting on each state row alone, with the row's V x V step matrix
//     A_t = f_t I + (1 - f_t) W diag(s_t),   s_t = 1 - Z_t^2 of that row
// (the factorization: the (KV)^2 Jacobian is block diagonal over the K rows).
//
// The linear recurrence is solved by a two-level scan over chunks of L steps:
//   maps:  per chunk p and row i, the product M_p = A_{t0} ... A_{t0+L-1}
//          (V x V): the V basis rows of the identity run through the chunk's
//          steps, on the MFMA units (V times the sequential flops);
//   solve: per chunk, the update from a zero start (its end e_p);
//   scan:  per row, sequentially over the chunks, D_p = D_{p-1} M_p + e_p,
//          which gives every chunk's true starting update;
//   solve: per chunk again from its starting update, adding d_t to X_t.
// Everything else is parallel over all steps: the initial guess, the
// linearisation (Z_t from X_{t-1} W on the MFMA units, the residual) and the
// readout y_t = X_t^T q_t + w_r (.) v_t.
//
// Step matrices and residuals are stored per step ([U, T, K, V] each, fp32),
// as (1 - f_t) s_t and r_t, so that a step of maps and solve is one MFMA chain
// and two VALU operations per element.  The MFMA step is the transposed
// product (P W)^T = W^T P^T on the 16x16x4 fp32 instruction, with the
// contraction of MFMA s enumerated so that its accumulator is the next step's
// B operand: lane l holds row l % 16 of a 16-row slab and, in element r of
// tile c, column 16 c + 4 (l / 16) + r.  One wave holds all V / 16 tiles of its
// slab, so no state leaves registers between steps.
//
// Prefetches.  Inputs are loaded one step or group ahead of their use, and
// every such load is issued unconditionally (addresses clamped to the last
// valid step): a prefetch under a condition leaves a different number of loads
// in flight on the two paths, and the wait before the next use then has to
// drain them all, the prefetch included.
//
// Supported: fp32 state, V in {16, 32, 48, 64}, any K <= 256.

#include <type_traits>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"
#include "m2rnn_newton_internal.h"

namespace m2rnn {

namespace {

constexpr int kWavesPerGroup = 4;  // 256-thread workgroups of independent waves

// Column of element r of tile c held by lane group g.
__device__ __forceinline__ constexpr int ncol(int c, int g, int r) { return 16 * c + 4 * g + r; }

// W^T as the A operand: wa[c][s] = scale W[pi(s, g)][16 c + li],
// pi(s, g) = 16 (s / 4) + 4 g + s % 4.
template <int VT>
__device__ __forceinline__ void load_wt(const float* __restrict__ Wn, int li, int g, float scale,
                                        float (&wa)[VT][4 * VT]) {
  constexpr int V = 16 * VT;
#pragma unroll
  for (int c = 0; c < VT; ++c)
#pragma unroll
    for (int s = 0; s < 4 * VT; ++s) {
      const int l = 16 * (s >> 2) + 4 * g + (s & 3);
      wa[c][s] = scale * Wn[l * V + 16 * c + li];
    }
}

// acc[c] += (P W)^T tile c, with P this wave's slab (lane: row li, own columns).
template <int VT>
__device__ __forceinline__ void slab_times_w(const float (&wa)[VT][4 * VT], const f32x4 (&p)[VT],
                                             f32x4 (&acc)[VT]) {
#pragma unroll
  for (int s = 0; s < 4 * VT; ++s)
#pragma unroll
    for (int c = 0; c < VT; ++c) acc[c] = mfma_16x16x4(wa[c][s], p[s >> 2][s & 3], acc[c]);
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ void st4(float* p, f32x4 x) { *(f32x4*)p = x; }

// Four consecutive inputs (16-byte aligned for fp32, 8-byte for bf16) as fp32.
__device__ __forceinline__ f32x4 ld4_in(const float* p) { return ld4(p); }
__device__ __forceinline__ f32x4 ld4_in(const uint16_t* p) {
  const uint2 raw = *(const uint2*)p;
  return f32x4{__builtin_bit_cast(float, raw.x << 16), __builtin_bit_cast(float, raw.x & 0xffff0000u),
               __builtin_bit_cast(float, raw.y << 16), __builtin_bit_cast(float, raw.y & 0xffff0000u)};
}

// Gates of steps t .. t + G - 1 (clamped to t_last), step t + m in lane m (and
// in the lanes congruent to it mod G): the address depends on the lane, so this
// is a vector load, which completes in order with the other vector loads (a
// wave-uniform address would become a scalar load, and waiting for one scalar
// load waits for all of them, prefetched ones included).
__device__ __forceinline__ float load_gates(const float* fp, int64_t N, int64_t t, int64_t t_last,
                                            int G) {
  const int span = G < 2 ? 2 : G;  // at least two distinct steps: the address must vary
  int64_t tt = t + (int64_t)(((int)threadIdx.x & 63) % span);
  if (tt > t_last) tt = t_last;
  return fp[tt * N];
}
// The value of x in lane m (m wave-uniform).
__device__ __forceinline__ float lane_value(float x, int m) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), m));
}

__device__ __forceinline__ int64_t nslab_of(int64_t K) { return (K + 15) / 16; }

// The wave's index in the grid, in a scalar register: everything derived from
// it (unit, chunk, slab, loop bounds) is then wave-uniform to the compiler, so
// the step loops are uniform branches and their addresses scalar arithmetic.
__device__ __forceinline__ int global_wave() {
  return __builtin_amdgcn_readfirstlane((int)blockIdx.x * kWavesPerGroup +
                                        ((int)threadIdx.x >> 6));
}

}  // namespace

// ---- initial guess X_t = F(0, x_t) = (1 - f_t) tanh(k_t v_t^T): a workgroup per
// (unit, step) at a time, a thread per four consecutive columns of the [K, V]
// state (the indices within the state are 32-bit; the step's are per workgroup).
template <typename InT>
__global__ void __launch_bounds__(256) m2rnn_newton_init_kernel(NewtonArgs a) {
  const int64_t K = a.K, T = a.T, N = a.N, V = a.V;
  const int V4 = (int)(V / 4), KV4 = (int)K * V4;
  const int64_t rows = a.B * N * T;
  const int grp = (int)(N / a.NQ);
  for (int64_t rw = blockIdx.x; rw < rows; rw += gridDim.x) {
    const int64_t u = rw / T, t = rw % T;
    const int64_t b = u / N, n = u % N;
    const int64_t tok = b * T + t;
    const InT* kp = (const InT*)a.k + (tok * a.NQ + n / grp) * K;
    const InT* vp = (const InT*)a.v + (tok * N + n) * V;
    const float omf = 1.0f - a.f[tok * N + n];
    float* xp = a.X + rw * K * V;
    for (int e = threadIdx.x; e < KV4; e += blockDim.x) {
      const int i = e / V4, j = (e - i * V4) * 4;
      const float kk = kTanhScale<float> * load_as<float>(kp + i);
      const f32x4 vv = ld4_in(vp + j);
      f32x4 x;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = omf * (1.0f - 2.0f * tanh_rc_scaled(kk * vv[r]));
      st4(xp + (int64_t)i * V + j, x);
    }
  }
}

// ---- linearisation at the current iterate, one wave per (unit, slab, block of
// TL steps): A_t = X_{t-1} W + k_t v_t^T (MFMA), Z_t = tanh(A_t),
// S_t = (1 - f_t)(1 - Z_t^2), R_t = X_t - f_t X_{t-1} - (1 - f_t) Z_t, and the
// largest |R_t| into *res (as the bit pattern of a non-negative float, whose
// unsigned order is the numeric order).  STORE = false only measures the residual.
// X_{t-1} is carried from the previous step; the next step's inputs are loaded
// while the current one is computed.
template <typename InT, int VT, bool STORE>
__global__ void __launch_bounds__(256) m2rnn_newton_linearize_kernel(NewtonArgs a,
                                                                     unsigned* res) {
  constexpr int V = 16 * VT;
  const int gw = global_wave();
  const int64_t nslab = nslab_of(a.K);
  const int64_t U = a.B * a.N;
  if (gw >= U * nslab * a.NTB) return;
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
  const int64_t tb = gw % a.NTB;
  const int64_t slab = (gw / a.NTB) % nslab;
  const int64_t u = gw / a.NTB / nslab;
  const int64_t N = a.N, K = a.K, T = a.T;
  const int64_t b = u / N, n = u % N;
  const int grp = (int)(N / a.NQ);
  const int64_t row = slab * 16 + li;
  const bool row_ok = row < K;
  const int64_t rowc = row_ok ? row : K - 1;
  const int64_t t0 = tb * a.TL;
  const int64_t t1 = t0 + a.TL < T ? t0 + a.TL : T;

  float wa[VT][4 * VT];
  load_wt<VT>(a.W + n * V * V, li, g, kTanhScale<float>, wa);

  // X_{t0 - 1}: H_0 (zero when absent) or the iterate
  f32x4 xp[VT];
  if (t0 == 0) {
#pragma unroll
    for (int c = 0; c < VT; ++c)
      xp[c] = a.H0 ? ld4(a.H0 + (u * K + rowc) * V + ncol(c, g, 0)) : f32x4{0, 0, 0, 0};
  } else {
#pragma unroll
    for (int c = 0; c < VT; ++c) xp[c] = ld4(a.X + ((u * T + t0 - 1) * K + rowc) * V + ncol(c, g, 0));
  }
  const InT* kp = (const InT*)a.k + ((b * T) * a.NQ + n / grp) * K + rowc;
  const InT* vp = (const InT*)a.v + ((b * T) * N + n) * V;
  const float* fp = a.f + (b * T) * N + n;
  // inputs of one step, loaded one step ahead of their use
  struct In {
    f32x4 x[VT];   // X_t (own columns)
    f32x4 v[VT];   // v_t (own columns)
    float k, f;    // k_t of the lane's row; gates of steps t (lane 0) and t + 1
  };
  auto load_in = [&](int64_t t, In& in) {
    const int64_t sidx = ((u * T + t) * K + rowc) * V;
#pragma unroll
    for (int c = 0; c < VT; ++c) {
      in.x[c] = ld4(a.X + sidx + ncol(c, g, 0));
      in.v[c] = ld4_in(vp + t * N * V + ncol(c, g, 0));
    }
    in.k = load_as<float>(kp + t * a.NQ * K);
    in.f = load_gates(fp, N, t, t1 - 1, 2);
  };
  float rmax = 0.0f;
  In cur, nxt;
  load_in(t0, cur);
  for (int64_t t = t0; t < t1; ++t) {
    load_in(t + 1 < t1 ? t + 1 : t, nxt);  // unconditional: see the note on prefetches
    __builtin_amdgcn_sched_barrier(0);
    const int64_t sidx = ((u * T + t) * K + rowc) * V;
    const float ks = kTanhScale<float> * cur.k;
    const float ff = lane_value(cur.f, 0);
    const float omf = 1.0f - ff;
    f32x4 acc[VT];
#pragma unroll
    for (int c = 0; c < VT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[c][r] = ks * cur.v[c][r];
    slab_times_w<VT>(wa, xp, acc);
    f32x4 sv[VT], rv[VT];
#pragma unroll
    for (int c = 0; c < VT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float rc = tanh_rc_scaled(acc[c][r]);
        // F = f X + (1 - f)(1 - 2 rc);  1 - Z^2 = 4 rc (1 - rc)
        const float F = fma_r(-2.0f * omf, rc, fma_r(ff, xp[c][r], omf));
        sv[c][r] = 4.0f * omf * rc * (1.0f - rc);
        rv[c][r] = cur.x[c][r] - F;
        rmax = fmaxf(rmax, fabsf(rv[c][r]));
      }
    if (STORE && row_ok) {
#pragma unroll
      for (int c = 0; c < VT; ++c) {
        st4(a.S + sidx + ncol(c, g, 0), sv[c]);
        st4(a.R + sidx + ncol(c, g, 0), rv[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < VT; ++c) xp[c] = cur.x[c];
    cur = nxt;
  }
  if (res) {
    if (!row_ok) rmax = 0.0f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, o, 64));
    if (lane == 0) atomicMax(res, __float_as_uint(rmax));
  }
}

// ---- chunk maps: one wave per (unit, chunk p, state row i, 16 basis rows):
// P = rows 16 sg .. 16 sg + 15 of the identity, stepped through the chunk as
// P <- f_t P + (P W) (.) S_t[i] (S_t[i] the row's (1 - f_t) s_t, the same for
// all 16 rows), and written to M[u][p][i].  Inputs of G steps are loaded one
// group ahead.
template <int VT>
__global__ void __launch_bounds__(256) m2rnn_newton_maps_kernel(NewtonArgs a) {
  constexpr int V = 16 * VT;
  constexpr int G = VT <= 2 ? 4 : 2;
  const int gw = global_wave();
  const int64_t U = a.B * a.N, K = a.K, T = a.T, N = a.N, P = a.P;
  if (gw >= U * P * K * VT) return;
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
  const int sg = gw % VT;
  const int64_t i = (gw / VT) % K;
  const int64_t p = (gw / VT / K) % P;
  const int64_t u = gw / VT / K / P;
  const int64_t b = u / N, n = u % N;
  const int64_t t0 = p * a.L;
  const int64_t t1 = t0 + a.L < T ? t0 + a.L : T;

  float wa[VT][4 * VT];
  load_wt<VT>(a.W + n * V * V, li, g, 1.0f, wa);
  const int brow = 16 * sg + li;  // basis row of this lane
  f32x4 pm[VT];
#pragma unroll
  for (int c = 0; c < VT; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) pm[c][r] = ncol(c, g, r) == brow ? 1.0f : 0.0f;

  const float* sp = a.S + (u * T * K + i) * V;   // step t: sp + t K V
  const float* fp = a.f + (b * T) * N + n;       // step t: fp + t N
  f32x4 cs[G][VT], ns[G][VT];
  float cf, nf;  // gates of the group, step m in lane m
  auto load_group = [&](int64_t tg, f32x4 (&s4)[G][VT], float& f1) {
#pragma unroll
    for (int m = 0; m < G; ++m) {
      const int64_t t = tg + m < t1 ? tg + m : t1 - 1;  // past the chunk: repeat its last step (unused)
#pragma unroll
      for (int c = 0; c < VT; ++c) s4[m][c] = ld4(sp + t * K * V + ncol(c, g, 0));
    }
    f1 = load_gates(fp, N, tg, t1 - 1, G);
  };
  auto run_group = [&](auto full, int64_t tg, const f32x4 (&s4)[G][VT], float f1) {
#pragma unroll
    for (int m = 0; m < G; ++m) {
      if (decltype(full)::value || tg + m < t1) {
        const float fm = lane_value(f1, m);
        f32x4 acc[VT];
#pragma unroll
        for (int c = 0; c < VT; ++c) acc[c] = f32x4{0, 0, 0, 0};
        slab_times_w<VT>(wa, pm, acc);
#pragma unroll
        for (int c = 0; c < VT; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) pm[c][r] = fma_r(fm, pm[c][r], acc[c][r] * s4[m][c][r]);
      }
    }
  };
  const std::true_type full;
  const std::false_type part;
  load_group(t0, cs, cf);
  int64_t tg = t0;
  for (; tg + 2 * G <= t1; tg += 2 * G) {
    load_group(tg + G, ns, nf);
    __builtin_amdgcn_sched_barrier(0);  // the prefetch stays ahead of the group's steps
    run_group(full, tg, cs, cf);
    load_group(tg + 2 * G, cs, cf);
    __builtin_amdgcn_sched_barrier(0);
    run_group(full, tg + G, ns, nf);
  }
  load_group(tg + G, ns, nf);  // fewer than 2 G steps left
  run_group(part, tg, cs, cf);
  run_group(part, tg + G, ns, nf);
  float* mp = a.M + (((u * P + p) * K + i) * V + brow) * V;
#pragma unroll
  for (int c = 0; c < VT; ++c) st4(mp + ncol(c, g, 0), pm[c]);
}

// ---- chunk solve: one wave per (unit, chunk p, 16-row slab):
//     d <- f_t d + (d W) (.) S_t - R_t
// from d = D[u][p] (or zero), over the chunk's steps.  Without APPLY the
// chunk's end value goes to E[u][p].  APPLY: the new iterate X_t + d_t is
// written to Xn for every step (Xn = X updates in place; with LIN they are two
// buffers, since another wave reads the state before its chunk from X).  LIN
// (with APPLY) also linearises the new
// iterate as it is produced, for the next iteration or its residual: with x the
// new states, Z_t = tanh(x_{t-1} W + k_t v_t^T), S_t = (1 - f_t)(1 - Z_t^2) and
// R_t = x_t - F(x_{t-1}) overwrite S_t and R_t once step t has used them
// (later steps' loads read later indices), and max |R_t| goes to *res.  The
// chunk's first x_{t-1} is H_0 (t = 0) or X_{t0-1} + D[u][p], both known before
// the previous chunk's wave has written anything.
template <typename InT, int VT, bool APPLY, bool LIN>
__global__ void __launch_bounds__(256) m2rnn_newton_solve_kernel(NewtonArgs a, unsigned* res) {
  constexpr int V = 16 * VT;
  // steps per group: two groups of inputs fit in registers
  constexpr int G = VT == 1 ? (LIN ? 4 : 6) : VT == 2 ? 2 : 1;
  const int gw = global_wave();
  const int64_t U = a.B * a.N, K = a.K, T = a.T, N = a.N, P = a.P;
  const int64_t nslab = nslab_of(K);
  if (gw >= U * P * nslab) return;
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
  const int64_t slab = gw % nslab;
  const int64_t p = (gw / nslab) % P;
  const int64_t u = gw / nslab / P;
  const int64_t b = u / N, n = u % N;
  const int grp = (int)(N / a.NQ);
  const int64_t row = slab * 16 + li;
  const bool row_ok = row < K;
  const int64_t rowc = row_ok ? row : K - 1;
  const int64_t t0 = p * a.L;
  const int64_t t1 = t0 + a.L < T ? t0 + a.L : T;

  float wa[VT][4 * VT];
  load_wt<VT>(a.W + n * V * V, li, g, 1.0f, wa);
  f32x4 d[VT];
  const bool from_d = APPLY && a.D != nullptr;
#pragma unroll
  for (int c = 0; c < VT; ++c)
    d[c] = from_d ? ld4(a.D + ((u * P + p) * K + rowc) * V + ncol(c, g, 0)) : f32x4{0, 0, 0, 0};
  // LIN: the new state before the step being computed
  f32x4 xprev[LIN ? VT : 1];
  if constexpr (LIN) {
    if (t0 == 0) {
#pragma unroll
      for (int c = 0; c < VT; ++c)
        xprev[c] = a.H0 ? ld4(a.H0 + (u * K + rowc) * V + ncol(c, g, 0)) : f32x4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int c = 0; c < VT; ++c)
        xprev[c] = ld4(a.X + ((u * T + t0 - 1) * K + rowc) * V + ncol(c, g, 0)) + d[c];
    }
  }
  const InT* kp = (const InT*)a.k + ((b * T) * a.NQ + n / grp) * K + rowc;
  const InT* vp = (const InT*)a.v + ((b * T) * N + n) * V;

  const int64_t base = (u * T * K + rowc) * V;   // step t: base + t K V
  const float* fp = a.f + (b * T) * N + n;
  struct In {
    f32x4 s[G][VT], r[G][VT];
    f32x4 x[APPLY ? G : 1][VT];  // APPLY: X_t of the current iterate
    f32x4 v[LIN ? G : 1][VT];    // LIN: v_t (own columns)
    float k[LIN ? G : 1];        // LIN: k_t of the lane's row
    float f;                     // gates, step m of the group in lane m
  };
  In cur, nxt;
  auto load_group = [&](int64_t tg, In& in) {
#pragma unroll
    for (int m = 0; m < G; ++m) {
      const int64_t t = tg + m < t1 ? tg + m : t1 - 1;
#pragma unroll
      for (int c = 0; c < VT; ++c) {
        in.s[m][c] = ld4(a.S + base + t * K * V + ncol(c, g, 0));
        in.r[m][c] = ld4(a.R + base + t * K * V + ncol(c, g, 0));
        if constexpr (APPLY) in.x[m][c] = ld4(a.X + base + t * K * V + ncol(c, g, 0));
        if constexpr (LIN) in.v[m][c] = ld4_in(vp + t * N * V + ncol(c, g, 0));
      }
      if constexpr (LIN) in.k[m] = load_as<float>(kp + t * a.NQ * K);
    }
    in.f = load_gates(fp, N, tg, t1 - 1, G);
  };
  float rmax = 0.0f;
  auto run_group = [&](auto full, int64_t tg, const In& in) {
#pragma unroll
    for (int m = 0; m < G; ++m) {
      if (decltype(full)::value || tg + m < t1) {
        const float fm = lane_value(in.f, m);
        f32x4 acc[VT];
#pragma unroll
        for (int c = 0; c < VT; ++c) acc[c] = f32x4{0, 0, 0, 0};
        slab_times_w<VT>(wa, d, acc);
#pragma unroll
        for (int c = 0; c < VT; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            d[c][r] = fma_r(fm, d[c][r], fma_r(acc[c][r], in.s[m][c][r], -in.r[m][c][r]));
        if constexpr (APPLY) {
          const int64_t o = base + (tg + m) * K * V;
          f32x4 xn[VT];
#pragma unroll
          for (int c = 0; c < VT; ++c) xn[c] = in.x[m][c] + d[c];
          if (row_ok) {
#pragma unroll
            for (int c = 0; c < VT; ++c) st4(a.Xn + o + ncol(c, g, 0), xn[c]);
          }
          if constexpr (LIN) {
            const float omf = 1.0f - fm;
            f32x4 al[VT];
#pragma unroll
            for (int c = 0; c < VT; ++c) al[c] = f32x4{0, 0, 0, 0};
            slab_times_w<VT>(wa, xprev, al);
            f32x4 sv[VT], rv[VT];
#pragma unroll
            for (int c = 0; c < VT; ++c)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float rc = tanh_rc_scaled(
                    kTanhScale<float> * fma_r(in.k[m], in.v[m][c][r], al[c][r]));
                const float F = fma_r(-2.0f * omf, rc, fma_r(fm, xprev[c][r], omf));
                sv[c][r] = 4.0f * omf * rc * (1.0f - rc);
                rv[c][r] = xn[c][r] - F;
                rmax = fmaxf(rmax, fabsf(rv[c][r]));
              }
            if (row_ok) {
#pragma unroll
              for (int c = 0; c < VT; ++c) {
                st4(a.S + o + ncol(c, g, 0), sv[c]);
                st4(a.R + o + ncol(c, g, 0), rv[c]);
              }
            }
#pragma unroll
            for (int c = 0; c < VT; ++c) xprev[c] = xn[c];
          }
        }
      }
    }
  };
  const std::true_type full;
  const std::false_type part;
  load_group(t0, cur);
  int64_t tg = t0;
  for (; tg + 2 * G <= t1; tg += 2 * G) {
    load_group(tg + G, nxt);
    __builtin_amdgcn_sched_barrier(0);  // the prefetch stays ahead of the group's steps
    run_group(full, tg, cur);
    load_group(tg + 2 * G, cur);
    __builtin_amdgcn_sched_barrier(0);
    run_group(full, tg + G, nxt);
  }
  load_group(tg + G, nxt);  // fewer than 2 G steps left
  run_group(part, tg, cur);
  run_group(part, tg + G, nxt);
  if (!APPLY && row_ok) {
    float* ep = a.E + ((u * P + p) * K + row) * V;
#pragma unroll
    for (int c = 0; c < VT; ++c) st4(ep + ncol(c, g, 0), d[c]);
  }
  if (LIN && res) {
    if (!row_ok) rmax = 0.0f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, o, 64));
    if (lane == 0) atomicMax(res, __float_as_uint(rmax));
  }
}

// ---- scan over the chunks, one wave per (unit, group of 64 / V rows): lane
// (rs, j) holds column j of row i = group (64 / V) + rs.  D[u][0][i] = 0 and
// D[u][p + 1][i] = D[u][p][i] M[u][p][i] + E[u][p][i], sequentially in p; the
// next chunk's column of M is loaded while the current one is applied.
template <int VT>
__global__ void __launch_bounds__(256) m2rnn_newton_scan_kernel(NewtonArgs a) {
  constexpr int V = 16 * VT;
  constexpr int RPW = 64 / V;  // rows per wave (V = 48: one, 16 lanes idle)
  const int gw = global_wave();
  const int64_t U = a.B * a.N, K = a.K, P = a.P;
  const int64_t groups = (K + RPW - 1) / RPW;
  if (gw >= U * groups) return;
  const int lane = threadIdx.x & 63;
  const int rs = lane / V < RPW ? lane / V : RPW - 1;
  const int j = lane % V;
  const int64_t u = gw / groups;
  const int64_t i = (gw % groups) * RPW + rs;
  const bool ok = lane < RPW * V && i < K;
  const int64_t ic = i < K ? i : K - 1;
  const int src0 = rs * V;  // lane holding column 0 of this lane's row

  // column j of M[u][p][i] in m[0 .. V), E[u][p][i][j] in m[V]; a ring of R
  // chunks is in flight (loads clamped to the last chunk: see the note on prefetches)
  constexpr int R = VT == 1 ? 4 : 2;
  float ring[R][V + 1];
  auto load_m = [&](int64_t p, float (&m)[V + 1]) {
    if (p > P - 1) p = P - 1;
    const float* mp = a.M + ((u * P + p) * K + ic) * V * V + j;
#pragma unroll
    for (int l = 0; l < V; ++l) m[l] = mp[l * V];
    m[V] = a.E[((u * P + p) * K + ic) * V + j];
  };
  float dcur = 0.0f;
  auto apply = [&](int64_t p, const float (&m)[V + 1]) {
    const int64_t o = ((u * P + p) * K + ic) * V + j;
    if (ok) a.D[o] = dcur;
    float s0 = m[V], s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
    for (int l = 0; l < V; l += 4) {
      s0 = fma_r(__shfl(dcur, src0 + l, 64), m[l], s0);
      s1 = fma_r(__shfl(dcur, src0 + l + 1, 64), m[l + 1], s1);
      s2 = fma_r(__shfl(dcur, src0 + l + 2, 64), m[l + 2], s2);
      s3 = fma_r(__shfl(dcur, src0 + l + 3, 64), m[l + 3], s3);
    }
    dcur = (s0 + s1) + (s2 + s3);
  };
#pragma unroll
  for (int r = 0; r < R; ++r) load_m(r, ring[r]);
  int64_t p = 0;
  for (; p + R <= P; p += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      apply(p + r, ring[r]);
      load_m(p + r + R, ring[r]);
      __builtin_amdgcn_sched_barrier(0);  // the ring's loads stay R chunks ahead
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (p + r < P) apply(p + r, ring[r]);
}

// ---- readout y_t = X_t^T q_t + w_r (.) v_t, one thread per (unit, step, four
// columns), rows summed in order; the threads of step T - 1 also copy X_T to HT.
template <typename InT>
__global__ void __launch_bounds__(256) m2rnn_newton_readout_kernel(NewtonArgs a) {
  const int64_t V = a.V, V4 = V / 4, K = a.K, T = a.T, N = a.N;
  const int64_t total = a.B * N * T * V4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int grp = (int)(N / a.NQ);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int64_t j = (e % V4) * 4;
    const int64_t t = (e / V4) % T;
    const int64_t u = e / V4 / T;
    const int64_t b = u / N, n = u % N;
    const int64_t tok = b * T + t;
    const InT* qp = (const InT*)a.q + (tok * a.NQ + n / grp) * K;
    const float* xp = a.X + (u * T + t) * K * V + j;
    const bool last = a.HT && t == T - 1;
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll 8
    for (int64_t i = 0; i < K; ++i) {
      const f32x4 x = ld4(xp + i * V);
      const float qq = load_as<float>(qp + i);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = fma_r(x[r], qq, acc[r]);
      if (last) st4(a.HT + (u * K + i) * V + j, x);
    }
    const InT* vp = (const InT*)a.v + (tok * N + n) * V + j;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fma_r(a.w_r[n * V + j + r], load_as<float>(vp + r), acc[r]);
    st4(a.y + (tok * N + n) * V + j, acc);
  }
}

__global__ void __launch_bounds__(64) m2rnn_newton_zero_kernel(unsigned* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}

NewtonLayout newton_layout(int64_t B, int64_t T, int64_t N, int64_t K, int64_t V,
                           bool states_given) {
  NewtonLayout L{};
  const int64_t U = B * N;
  const int64_t VT = V / 16;
  const int64_t nslab = num_slabs(K);
  // Chunks.  The two solves walk L = T / P steps and the scan P chunks, one
  // after the other, so P near sqrt(T) balances them (measured: 2.5 sqrt(T) is
  // slower, the solves being bound by their occupancy rather than by L); the
  // maps want at least eight waves per SIMD (1024 SIMDs).  When the (unit, row)
  // pairs alone fill the device there is nothing to gain from chunks: one
  // chunk, solved directly.
  const int64_t map_waves = U * K * VT;
  int64_t P = 1;
  if (map_waves < 8192) {
    P = (8192 + map_waves - 1) / (map_waves > 0 ? map_waves : 1);
    int64_t sq = 1;
    while (sq * sq < T) ++sq;  // ceil(sqrt(T))
    if (P < sq) P = sq;
  }
  if (P > T) P = T;
  if (P < 1) P = 1;
  L.L = (T + P - 1) / P;
  L.P = (T + L.L - 1) / L.L;
  // Linearisation: about 16 steps or more per wave, some 16K waves.
  const int64_t lin_units = U * nslab;
  int64_t ntb = (16384 + lin_units - 1) / (lin_units > 0 ? lin_units : 1);
  const int64_t max_tb = (T + 15) / 16;
  if (ntb > max_tb) ntb = max_tb;
  if (ntb < 1) ntb = 1;
  L.TL = (T + ntb - 1) / ntb;
  L.NTB = (T + L.TL - 1) / L.TL;
  const size_t seq = (size_t)U * (size_t)T * (size_t)K * (size_t)V;
  const size_t chunk = L.P > 1 ? (size_t)U * (size_t)L.P * (size_t)K * (size_t)V : 0;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o += align_up(n, 64);
    return at;
  };
  L.X = states_given ? 0 : take(seq);
  L.X2 = take(seq);
  L.S = take(seq);
  L.R = take(seq);
  L.M = take(chunk * (size_t)V);
  L.E = take(chunk);
  L.D = take(chunk);
  L.total_floats = o;
  return L;
}

namespace {

inline unsigned grid_of(int64_t waves) {
  return (unsigned)((waves + kWavesPerGroup - 1) / kWavesPerGroup);
}
inline unsigned grid_elems(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  return (unsigned)(b > 0 ? b : 1);
}

template <typename InT, int VT>
hipError_t launch_newton_vt(const NewtonArgs& a, hipStream_t st) {
  const int64_t U = a.B * a.N, K = a.K, nslab = num_slabs(K);
  const int64_t VT64 = VT;
  unsigned* res = a.res;
  if (res) hipLaunchKernelGGL(m2rnn_newton_zero_kernel, dim3(1), dim3(64), 0, st, res, a.iters + 1);
  const unsigned g_solve = grid_of(U * a.P * nslab);
  // Linearise inside the applying solve when its waves cover the 1024 SIMDs
  // (it is then bound by throughput, and the fused pass saves a read of the
  // iterate); with fewer waves the solve is bound by its per-step latency,
  // which the fused work lengthens, and a separate pass is faster (measured).
  const bool fuse = U * a.P * nslab >= 1024;
  // Fused, iteration i reads iterate i from one state buffer and writes
  // iterate i + 1 to the other, and the guess goes where the last iterate must
  // end up after `iters` swaps (a.X: the caller's states or the workspace's
  // first buffer).  Separate, the update is applied in place.
  NewtonArgs c = a;
  if (!fuse) {
    c.Xn = a.X;
  } else if (a.iters & 1) {
    c.X = a.Xn;
    c.Xn = a.X;
  }
  {
    int64_t rows = U * a.T;
    if (rows > 65536) rows = 65536;
    hipLaunchKernelGGL(m2rnn_newton_init_kernel<InT>, dim3((unsigned)rows), dim3(256), 0, st, c);
  }
  if (a.iters > 0 || res)  // the guess's linearisation (and residual)
    hipLaunchKernelGGL((m2rnn_newton_linearize_kernel<InT, VT, true>),
                       dim3(grid_of(U * nslab * a.NTB)), dim3(256), 0, st, c, res);
  for (int it = 0; it < a.iters; ++it) {
    if (!fuse && it > 0)  // the iterate's linearisation (and residual)
      hipLaunchKernelGGL((m2rnn_newton_linearize_kernel<InT, VT, true>),
                         dim3(grid_of(U * nslab * a.NTB)), dim3(256), 0, st, c,
                         res ? res + it : nullptr);
    NewtonArgs b = c;
    if (a.P > 1) {
      hipLaunchKernelGGL((m2rnn_newton_maps_kernel<VT>), dim3(grid_of(U * a.P * K * VT64)),
                         dim3(256), 0, st, c);
      hipLaunchKernelGGL((m2rnn_newton_solve_kernel<InT, VT, false, false>), dim3(g_solve),
                         dim3(256), 0, st, c, nullptr);
      hipLaunchKernelGGL((m2rnn_newton_scan_kernel<VT>),
                         dim3(grid_of(U * ((K + 64 / (16 * VT) - 1) / (64 / (16 * VT))))),
                         dim3(256), 0, st, c);
    } else {
      b.D = nullptr;  // one chunk: the update starts from zero
    }
    // the new iterate is linearised on the way unless it is the last one and
    // no residual is asked for
    if (fuse && (it + 1 < a.iters || res))
      hipLaunchKernelGGL((m2rnn_newton_solve_kernel<InT, VT, true, true>), dim3(g_solve),
                         dim3(256), 0, st, b, res ? res + it + 1 : nullptr);
    else
      hipLaunchKernelGGL((m2rnn_newton_solve_kernel<InT, VT, true, false>), dim3(g_solve),
                         dim3(256), 0, st, b, nullptr);
    float* t = c.X;
    c.X = c.Xn;
    c.Xn = t;  // (the same buffer when not fused)
  }
  if (!fuse && res && a.iters > 0)  // the residual of the last iterate
    hipLaunchKernelGGL((m2rnn_newton_linearize_kernel<InT, VT, false>),
                       dim3(grid_of(U * nslab * a.NTB)), dim3(256), 0, st, c, res + a.iters);
  // c.X now holds the last iterate (a.X)
  hipLaunchKernelGGL(m2rnn_newton_readout_kernel<InT>, dim3(grid_elems(U * a.T * a.V / 4)),
                     dim3(256), 0, st, c);
  return hipGetLastError();
}

template <typename InT>
hipError_t launch_newton_t(const NewtonArgs& a, hipStream_t st) {
  switch (a.V) {
    case 16: return launch_newton_vt<InT, 1>(a, st);
    case 32: return launch_newton_vt<InT, 2>(a, st);
    case 48: return launch_newton_vt<InT, 3>(a, st);
    case 64: return launch_newton_vt<InT, 4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_newton(const NewtonArgs& a, int in_dtype, hipStream_t stream) {
  if (in_dtype == kF32) return launch_newton_t<float>(a, stream);
  if (in_dtype == kBF16) return launch_newton_t<uint16_t>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace m2rnn
