// Reverse-time M²RNN backward for gfx950.
//
// Implements the corrected BPTT chain rule of the M²RNN review (section 2.7),
// with the value-residual branch restored, and the review's section 2.6
// scheme of rerunning the recurrence before the reverse scan -- restricted to
// one checkpoint interval at a time.  For each (b, n) and each interval
// [cC, cC + L) taken from last to first:
//   1. recompute the L steps from ckpt[c] = H_{cC} (same MFMA step as the
//      forward), keeping H_{t-1} and Z_t of every step in a per-slab
//      workspace (each lane stores and reloads its own tiles);
//   2. walk the L steps backwards:
//        R = C + q u^T,  D = (1 - f) R (.) (1 - Z^2),  C <- f R + D W^T  (MFMA)
//        dW += H_{t-1}^T D                                              (MFMA)
//        dq = H_t u, dk = D v (row sums), dv = D^T k (sum over the slab's rows),
//        df = <R, H_{t-1} - Z>.
// As in the forward, a workgroup owns one 16-row slab; rows are independent
// in the backward as well (W^T acts on columns), so only dv, df and dW need
// sums across slabs, done by fixed-order reduction kernels afterwards.
//
// MFMA layouts.  C W-product: (D W^T)^T = W D^T, A = W (registers), B = D^T,
// with the same contraction enumeration pi(s, g) = 16 (s / 4) + m(g, s % 4) as
// the forward, so D's own tiles feed the B operand straight from registers and
// the other waves' tiles come through LDS.  dW: output tile (l, j), A[l][i] =
// H_{t-1}[i][l], B[i][j] = D[i][j], contraction over the 16 slab rows in four
// k-steps; both operands are read transposed from the LDS exchange buffers.

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

BwdWorkspace bwd_workspace_layout(int64_t B, int64_t T, int64_t N, int64_t K, int64_t V,
                                  int64_t C) {
  BwdWorkspace L{};
  const int64_t ns = num_slabs(K);
  const int64_t vt = value_tiles(V);
  const size_t units = (size_t)(B * N * ns);
  const int64_t rows = B * T;
  L.row_blocks = (rows + 255) / 256;
  size_t off = 0;
  auto take = [&](size_t elems) {
    const size_t at = off;
    off = align_up(off + elems, 64);
    return at;
  };
  L.slot_elems = (size_t)vt * 64 * 4;
  L.states = take(units * (size_t)(2 * C + 1) * L.slot_elems);
  L.dv_part = take(ns > 1 ? (size_t)ns * B * T * N * V : 0);
  L.df_part = take((size_t)ns * B * T * N);
  L.dW_part = take((size_t)B * ns * N * V * V);
  L.col_part = take((size_t)L.row_blocks * N * (V + 2));
  L.total_elems = off;
  return L;
}

template <typename Real, int VT>
struct BwdTraits {
  static constexpr int VP = 16 * VT;
  static constexpr int NW = VT <= 4 ? VT : VT / 2;
  static constexpr int TPW = VT / NW;
  static constexpr int NT = 64 * NW;
  static constexpr int NS = 4 * VT;
};

template <typename Real, int VT, int NW>
struct BwdSmem {
  using R4 = typename Vec4<Real>::type;
  R4 xb[2][VT][64];      // H exchange (recompute) / H_{t-1} for dW (reverse)
  R4 xd[2][VT][64];      // D exchange
  Real red[2][2][NW][16];  // per-wave row partials of dq and dk
  Real redf[2][NW];        // per-wave partials of df
};

template <typename InT, typename Real, int VT>
__global__ void __launch_bounds__((BwdTraits<Real, VT>::NT))
    m2rnn_bwd_kernel(BwdArgs a, BwdWorkspace L) {
  using Tr = BwdTraits<Real, VT>;
  using R4 = typename Vec4<Real>::type;
  constexpr int TPW = Tr::TPW, NS = Tr::NS, NW = Tr::NW;
  __shared__ BwdSmem<Real, VT, NW> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int nslab = a.nslab;
  const int slab = unit % nslab;
  const int bn = unit / nslab;
  const int64_t B = a.B, T = a.T, N = a.N, K = a.K, V = a.V, C = a.C;
  const int n = (int)(bn % N);
  const int b = (int)(bn / N);
  const int row = slab * 16 + li;
  const bool row_ok = row < K;
  const int64_t rowc = row_ok ? row : K - 1;  // clamped row for unconditional loads

  const InT* __restrict__ kp = (const InT*)a.k;
  const InT* __restrict__ vp = (const InT*)a.v;
  const InT* __restrict__ qp = (const InT*)a.q;
  const Real* __restrict__ fp = (const Real*)a.f;
  const Real* __restrict__ Wp = (const Real*)a.W;
  const Real* __restrict__ wrp = (const Real*)a.w_r;
  const Real* __restrict__ dyp = (const Real*)a.dy;
  Real* __restrict__ ws = (Real*)a.ws;
  R4* __restrict__ slots = (R4*)(ws + L.states + (size_t)unit * (size_t)(2 * C + 1) * L.slot_elems);
  Real* __restrict__ dv_part = ws + L.dv_part;
  Real* __restrict__ df_part = ws + L.df_part;
  const int64_t tok_stride = B * T * N;

  // A operands: W^T for the recompute (as in the forward), W for C <- f R + D W^T.
  Real wf[TPW][NS], wb[TPW][NS];
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
    const int col = (w * TPW + p) * 16 + li;
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) {
      const int s = (s0 + 4 * TPW * w) % NS;
      const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
      const bool ok = col < V && l < V;
      wf[p][s0] = ok ? Wp[((int64_t)n * V + l) * V + col] : Real(0);
      wb[p][s0] = ok ? Wp[((int64_t)n * V + col) * V + l] : Real(0);
    }
  }

  auto slot_at = [&](int64_t s, int p) -> R4& {
    return slots[((size_t)s * VT + (w * TPW + p)) * 64 + lane];
  };
  auto col_of = [&](int p, int r) { return (w * TPW + p) * 16 + acc_m<Real>(g, r); };
  const int64_t state_base = (((int64_t)b * N + n) * K + row) * V;

  // state gradient C_T = dHT
  R4 Cg[TPW];
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = col_of(p, r);
      Cg[p][r] = (a.dHT && row_ok && col < V) ? ((const Real*)a.dHT)[state_base + col] : Real(0);
    }
  }
  R4 dWacc[TPW][VT];
#pragma unroll
  for (int p = 0; p < TPW; ++p)
#pragma unroll
    for (int jt = 0; jt < VT; ++jt) dWacc[p][jt] = R4{0, 0, 0, 0};

  const int64_t nck = (T + C - 1) / C;
  for (int64_t c = nck - 1; c >= 0; --c) {
    const int64_t t0 = c * C;
    const int64_t Lc = (T - t0) < C ? (T - t0) : C;
    __syncthreads();  // previous interval's LDS reads are done

    // ---------------- 1. recompute the interval from ckpt[c]
    R4 h[TPW];
    const Real* ck = (const Real*)a.ckpt + ((((int64_t)b * N + n) * nck + c) * K + row) * V;
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = col_of(p, r);
        h[p][r] = (row_ok && col < V) ? ck[col] : Real(0);
      }
      slot_at(0, p) = h[p];
    }
    Real hb[NS];
    {
      const int ib = (int)((t0 + 1) & 1);
#pragma unroll
      for (int p = 0; p < TPW; ++p) sm.xb[ib][w * TPW + p][lane] = h[p];
      __syncthreads();
#pragma unroll
      for (int q0 = 0; q0 < VT; ++q0) {
        const R4 t4 = q0 < TPW ? h[q0] : sm.xb[ib][(q0 + TPW * w) % VT][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
      }
    }
    // inputs of one recompute step (issued a step ahead of their use)
    struct FwdIn {
      Real kv, ft;
      R4 vv[TPW];
    };
    auto load_fwd_in = [&](int64_t t) {
      FwdIn in;
      const int64_t tok = ((int64_t)b * T + clamp_idx(t, T - 1)) * N + n;
      in.kv = load_sel<Real>(kp, tok * K + rowc, row_ok);
      in.ft = fp[tok];
#pragma unroll
      for (int p = 0; p < TPW; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = col_of(p, r);
          in.vv[p][r] = load_sel<Real>(vp, tok * V + clamp_idx(col, V - 1), col < V);
        }
      return in;
    };
    FwdIn fin = load_fwd_in(t0);
    for (int64_t tt = 0; tt < Lc; ++tt) {
      const int64_t t = t0 + tt;
      const FwdIn cur = fin;
      fin = load_fwd_in(t + 1);
      R4 acc[TPW];
#pragma unroll
      for (int p = 0; p < TPW; ++p) acc[p] = cur.kv * cur.vv[p];
#pragma unroll
      for (int s0 = 0; s0 < NS; ++s0) {
#pragma unroll
        for (int p = 0; p < TPW; ++p) acc[p] = mfma_16x16x4(wf[p][s0], hb[s0], acc[p]);
      }
      const Real ft = cur.ft;
      const Real omf = Real(1) - ft;
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        R4 z;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          z[r] = tanh_fast(acc[p][r]);
          h[p][r] = ft * h[p][r] + omf * z[r];
        }
        slot_at(C + 1 + tt, p) = z;
        slot_at(tt + 1, p) = h[p];
      }
      const int xbuf = (int)(t & 1);
#pragma unroll
      for (int p = 0; p < TPW; ++p) sm.xb[xbuf][w * TPW + p][lane] = h[p];
      __syncthreads();
#pragma unroll
      for (int q0 = TPW; q0 < VT; ++q0) {
        const R4 t4 = sm.xb[xbuf][(q0 + TPW * w) % VT][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
      }
#pragma unroll
      for (int p = 0; p < TPW; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) hb[4 * p + r] = h[p][r];
    }
    __syncthreads();  // recompute exchange reads are done before xb is reused

    // ---------------- 2. reverse scan over the interval
    // inputs of one reverse step (issued a step ahead of their use)
    struct BwdIn {
      Real kv, qv, ft;
      R4 vv[TPW], uu[TPW], Hp[TPW], Z[TPW];
    };
    auto load_bwd_in = [&](int64_t tt) {
      BwdIn in;
      const int64_t ttc = tt < 0 ? 0 : tt;
      const int64_t tok = ((int64_t)b * T + t0 + ttc) * N + n;
      in.kv = load_sel<Real>(kp, tok * K + rowc, row_ok);
      in.qv = load_sel<Real>(qp, tok * K + rowc, row_ok);
      in.ft = fp[tok];
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        in.Hp[p] = slot_at(ttc, p);
        in.Z[p] = slot_at(C + 1 + ttc, p);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = col_of(p, r);
          const int64_t i = tok * V + clamp_idx(col, V - 1);
          in.vv[p][r] = load_sel<Real>(vp, i, col < V);
          in.uu[p][r] = load_sel<Real>(dyp, i, col < V);
        }
      }
      return in;
    };
    R4 Hc[TPW];  // H_t, the state after the step being reversed
#pragma unroll
    for (int p = 0; p < TPW; ++p) Hc[p] = slot_at(Lc, p);
    BwdIn bin = load_bwd_in(Lc - 1);
    for (int64_t tt = Lc - 1; tt >= 0; --tt) {
      const int64_t t = t0 + tt;
      const int64_t tok = ((int64_t)b * T + t) * N + n;
      const BwdIn cur = bin;
      bin = load_bwd_in(tt - 1);
      const Real kv = cur.kv, qv = cur.qv, ft = cur.ft;
      R4 R[TPW], D[TPW];
      Real dqp = 0, dkp = 0, dfp = 0;
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const Real u = cur.uu[p][r];
          const Real z = cur.Z[p][r];
          R[p][r] = Cg[p][r] + qv * u;
          dqp += Hc[p][r] * u;
          D[p][r] = (Real(1) - ft) * R[p][r] * (Real(1) - z * z);
          dfp += R[p][r] * (cur.Hp[p][r] - z);
          dkp += D[p][r] * cur.vv[p][r];
        }
      }
      const int buf = (int)(t & 1);
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        sm.xd[buf][w * TPW + p][lane] = D[p];
        sm.xb[buf][w * TPW + p][lane] = cur.Hp[p];
        Hc[p] = cur.Hp[p];  // H_{t-1} is the next (earlier) step's H_t
      }
      dqp = cross_row_sum(dqp);
      dkp = cross_row_sum(dkp);
      dfp = cross_row_sum(row16_sum(dfp));
      if (g == 0) {
        sm.red[buf][0][w][li] = dqp;
        sm.red[buf][1][w][li] = dkp;
      }
      if (lane == 0) sm.redf[buf][w] = dfp;
      // dv_t = D^T k over this slab's rows (+ w_r (.) u when the slab is the whole head)
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const Real s = row16_sum(D[p][r] * kv);
          const int col = col_of(p, r);
          if (li == 0 && col < V) {
            if (nslab == 1) {
              ((Real*)a.dv)[tok * V + col] = s + wrp[(int64_t)n * V + col] * cur.uu[p][r];
            } else {
              dv_part[slab * tok_stride * V + tok * V + col] = s;
            }
          }
        }
      }
      __syncthreads();
      if (w == 0) {
        if (lane < 32) {
          const int which = lane >> 4;
          Real s = 0;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) s += sm.red[buf][which][ww][li];
          if (row_ok) ((Real*)(which ? a.dk : a.dq))[tok * K + row] = s;
        } else if (lane == 32) {
          Real s = 0;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) s += sm.redf[buf][ww];
          df_part[slab * tok_stride + tok] = s;
        }
      }
      // C_{t-1} = f R + D W^T
      Real db[NS];
#pragma unroll
      for (int q0 = 0; q0 < VT; ++q0) {
        const R4 t4 = q0 < TPW ? D[q0] : sm.xd[buf][(q0 + TPW * w) % VT][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) db[4 * q0 + r] = t4[r];
      }
#pragma unroll
      for (int p = 0; p < TPW; ++p) Cg[p] = ft * R[p];
#pragma unroll
      for (int s0 = 0; s0 < NS; ++s0) {
#pragma unroll
        for (int p = 0; p < TPW; ++p) Cg[p] = mfma_16x16x4(wb[p][s0], db[s0], Cg[p]);
      }
      // dW += H_{t-1}^T D over the slab's rows
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // element (row 4 kk + g, column 16 c + li) of a tile in the exchange
        // buffer sits in lane 16 acc_g(li) + row, element acc_r(li)
        const int idx = 16 * acc_g<Real>(li) + 4 * kk + g;
        const int rr = acc_r<Real>(li);
        Real aop[TPW];
#pragma unroll
        for (int p = 0; p < TPW; ++p)
          aop[p] = ((const Real*)&sm.xb[buf][w * TPW + p][0])[idx * 4 + rr];
#pragma unroll
        for (int jt = 0; jt < VT; ++jt) {
          const Real bop = ((const Real*)&sm.xd[buf][jt][0])[idx * 4 + rr];
#pragma unroll
          for (int p = 0; p < TPW; ++p) dWacc[p][jt] = mfma_16x16x4(aop[p], bop, dWacc[p][jt]);
        }
      }
    }
  }

  if (a.dH0) {
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = col_of(p, r);
        if (row_ok && col < V) ((Real*)a.dH0)[state_base + col] = Cg[p][r];
      }
    }
  }
  // this slab's share of dW: lane holds dW[16 c + m(g, r)][16 jt + li]
  Real* dWp = ws + L.dW_part + (((size_t)b * nslab + slab) * N + n) * V * V;
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
#pragma unroll
    for (int jt = 0; jt < VT; ++jt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int l = (w * TPW + p) * 16 + acc_m<Real>(g, r);
        const int j = jt * 16 + li;
        if (l < V && j < V) dWp[(int64_t)l * V + j] = dWacc[p][jt][r];
      }
    }
  }
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float dev_expf_(float x) { return expf(x); }
__device__ __forceinline__ double dev_expf_(double x) { return exp(x); }
__device__ __forceinline__ float dev_log1p_(float x) { return log1pf(x); }
__device__ __forceinline__ double dev_log1p_(double x) { return log1p(x); }

template <typename Real>
__device__ __forceinline__ Real softplus_(Real x) {
  const Real ax = x < Real(0) ? -x : x;
  return (x > Real(0) ? x : Real(0)) + dev_log1p_(dev_expf_(-ax));
}
template <typename Real>
__device__ __forceinline__ Real sigmoid_(Real x) {
  if (x >= Real(0)) return Real(1) / (Real(1) + dev_expf_(-x));
  const Real e = dev_expf_(x);
  return e / (Real(1) + e);
}

// Per token: df = sum over slabs; gate chain rule -> dlogit.  df is kept (in
// slab 0's partial) for the alpha reduction.
template <typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_bwd_token_kernel(int64_t total, int64_t N, int nslab, int kind,
                           Real* __restrict__ df_part, const Real* __restrict__ f,
                           const Real* __restrict__ logit, const Real* __restrict__ alpha,
                           const Real* __restrict__ beta, Real* __restrict__ dlogit) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    Real df = df_part[i];
    for (int s = 1; s < nslab; ++s) df += df_part[s * total + i];
    df_part[i] = df;
    const Real fv = f[i];
    if (kind == kGateSigmoid) {
      dlogit[i] = df * fv * (Real(1) - fv);
    } else {
      const int64_t n = i % N;
      const Real x = logit[i] + beta[n];
      dlogit[i] = -df * alpha[n] * sigmoid_(x) * fv;
    }
  }
}

// dv = sum over slabs of the partials + w_r (.) dy
template <typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_bwd_dv_kernel(int64_t total, int64_t N, int64_t V, int nslab,
                        const Real* __restrict__ dv_part, const Real* __restrict__ dy,
                        const Real* __restrict__ w_r, Real* __restrict__ dv) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    Real s = dv_part[i];
    for (int sl = 1; sl < nslab; ++sl) s += dv_part[sl * total + i];
    const int64_t j = i % V;
    const int64_t n = (i / V) % N;
    dv[i] = s + w_r[n * V + j] * dy[i];
  }
}

// dW[n] = sum over (b, slab) partials, in that order
template <typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_bwd_dw_kernel(int64_t per, int64_t parts, const Real* __restrict__ part,
                        Real* __restrict__ dW) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < per; i += stride) {
    Real s = 0;
    for (int64_t p = 0; p < parts; ++p) s += part[p * per + i];
    dW[i] = s;
  }
}

// Column sums over the B*T token rows, stage 1: one block per (row block, head).
// Columns 0..V-1: dy (.) v (-> dw_r); V: -df softplus(x) f (-> dalpha); V+1: dlogit (-> dbeta).
template <typename InT, typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_bwd_colsum_kernel(int64_t rows, int64_t N, int64_t V, int kind,
                            const Real* __restrict__ dy, const InT* __restrict__ v,
                            const Real* __restrict__ df, const Real* __restrict__ f,
                            const Real* __restrict__ logit, const Real* __restrict__ alpha,
                            const Real* __restrict__ beta, const Real* __restrict__ dlogit,
                            Real* __restrict__ col_part) {
  const int64_t rb = blockIdx.x;
  const int64_t n = blockIdx.y;
  const int64_t ncol = V + 2;
  const int64_t r0 = rb * 256;
  const int64_t r1 = (r0 + 256) < rows ? (r0 + 256) : rows;
  for (int64_t col = threadIdx.x; col < ncol; col += blockDim.x) {
    Real s = 0;
    if (col < V) {
      for (int64_t r = r0; r < r1; ++r) {
        const int64_t i = (r * N + n) * V + col;
        s += dy[i] * load_as<Real>(v + i);
      }
    } else if (kind == kGateExpSoftplus) {
      for (int64_t r = r0; r < r1; ++r) {
        const int64_t i = r * N + n;
        if (col == V) {
          s += -df[i] * softplus_(logit[i] + beta[n]) * f[i];
        } else {
          s += dlogit[i];
        }
      }
    }
    col_part[(rb * N + n) * ncol + col] = s;
  }
}

// stage 2: sum the row blocks in order
template <typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_bwd_colsum_final_kernel(int64_t row_blocks, int64_t N, int64_t V, int kind,
                                  const Real* __restrict__ col_part, Real* __restrict__ dw_r,
                                  Real* __restrict__ dalpha, Real* __restrict__ dbeta) {
  const int64_t n = blockIdx.x;
  const int64_t ncol = V + 2;
  for (int64_t col = threadIdx.x; col < ncol; col += blockDim.x) {
    Real s = 0;
    for (int64_t rb = 0; rb < row_blocks; ++rb) s += col_part[(rb * N + n) * ncol + col];
    if (col < V) {
      dw_r[n * V + col] = s;
    } else if (kind == kGateExpSoftplus) {
      if (col == V) dalpha[n] = s;
      else dbeta[n] = s;
    }
  }
}

static unsigned grid_for(int64_t total) {
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

template <typename InT, typename Real, int VT>
static hipError_t launch_bwd_vt(const BwdArgs& a, hipStream_t stream) {
  using Tr = BwdTraits<Real, VT>;
  static_assert(sizeof(BwdSmem<Real, VT, Tr::NW>) <= 160 * 1024, "LDS budget");
  const BwdWorkspace L = bwd_workspace_layout(a.B, a.T, a.N, a.K, a.V, a.C);
  const int64_t units = a.B * a.N * a.nslab;
  hipLaunchKernelGGL((m2rnn_bwd_kernel<InT, Real, VT>), dim3((unsigned)units), dim3(Tr::NT), 0,
                     stream, a, L);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  Real* ws = (Real*)a.ws;
  const int64_t tokens = a.B * a.T * a.N;
  hipLaunchKernelGGL((m2rnn_bwd_token_kernel<Real>), dim3(grid_for(tokens)), dim3(256), 0, stream,
                     tokens, a.N, a.nslab, a.gate_kind, ws + L.df_part, (const Real*)a.f,
                     (const Real*)a.logit, (const Real*)a.alpha, (const Real*)a.beta,
                     (Real*)a.dlogit);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.nslab > 1) {
    const int64_t total = tokens * a.V;
    hipLaunchKernelGGL((m2rnn_bwd_dv_kernel<Real>), dim3(grid_for(total)), dim3(256), 0, stream,
                       total, a.N, a.V, a.nslab, ws + L.dv_part, (const Real*)a.dy,
                       (const Real*)a.w_r, (Real*)a.dv);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int64_t per = a.N * a.V * a.V;
  hipLaunchKernelGGL((m2rnn_bwd_dw_kernel<Real>), dim3(grid_for(per)), dim3(256), 0, stream, per,
                     a.B * a.nslab, ws + L.dW_part, (Real*)a.dW);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((m2rnn_bwd_colsum_kernel<InT, Real>),
                     dim3((unsigned)L.row_blocks, (unsigned)a.N), dim3(256), 0, stream,
                     a.B * a.T, a.N, a.V, a.gate_kind, (const Real*)a.dy, (const InT*)a.v,
                     ws + L.df_part, (const Real*)a.f, (const Real*)a.logit,
                     (const Real*)a.alpha, (const Real*)a.beta, (const Real*)a.dlogit,
                     ws + L.col_part);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((m2rnn_bwd_colsum_final_kernel<Real>), dim3((unsigned)a.N), dim3(256), 0,
                     stream, L.row_blocks, a.N, a.V, a.gate_kind, ws + L.col_part,
                     (Real*)a.dw_r, (Real*)a.dalpha, (Real*)a.dbeta);
  return hipGetLastError();
}

template <typename InT, typename Real>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  switch (value_tiles(a.V)) {
    case 1: return launch_bwd_vt<InT, Real, 1>(a, stream);
    case 2: return launch_bwd_vt<InT, Real, 2>(a, stream);
    case 3: return launch_bwd_vt<InT, Real, 3>(a, stream);
    case 4: return launch_bwd_vt<InT, Real, 4>(a, stream);
    case 6: return launch_bwd_vt<InT, Real, 6>(a, stream);
    case 8: return launch_bwd_vt<InT, Real, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const BwdArgs& a, int in_dtype, int state_dtype, hipStream_t stream) {
  if (state_dtype == kF32) {
    if (in_dtype == kF32) return launch_bwd_t<float, float>(a, stream);
    if (in_dtype == kBF16) return launch_bwd_t<uint16_t, float>(a, stream);
  } else if (state_dtype == kF64) {
    if (in_dtype == kF64) return launch_bwd_t<double, double>(a, stream);
    if (in_dtype == kBF16) return launch_bwd_t<uint16_t, double>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace m2rnn
