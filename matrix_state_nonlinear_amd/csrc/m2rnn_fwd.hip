// Fused M²RNN forward for gfx950.
//
// Computes, for every (batch b, head n), the recurrence of the M²RNN review
// (section 2.1, Eq. 10-12):
//     Z_t = tanh(H_{t-1} W_n + k_t v_t^T),  H_t = f_t H_{t-1} + (1 - f_t) Z_t,
//     y_t = H_t^T q_t + w_r (.) v_t.
//
// Work decomposition.  W mixes value columns only, so the K rows of a head are
// independent recurrences (they meet only in the readout sum over rows).  A
// workgroup owns one 16-row slab of one head for all T steps; a head with K
// rows becomes ceil(K / 16) workgroups on different compute units, and their
// partial readouts are summed by a second, elementwise kernel.
//
// Inside a workgroup each wave owns TPW 16-column tiles of the slab.  The step
// is computed transposed, (H W)^T = W^T H^T, on the 16x16x4 MFMA: W^T is the
// A operand (held in registers for the whole sequence), H^T the B operand.
// The MFMA result layout (lane l holds row l % 16 and, in element r, column
// 16 c + m(g, r) with g = l / 16 and m the instruction's accumulator row map)
// is then exactly the B-operand layout of the next step, provided the
// contraction index of MFMA number s is enumerated as
// pi(s, g) = 16 (s / 4) + m(g, s % 4).  So the state never leaves registers:
// its own tiles stay in the accumulators and the other waves' tiles arrive
// through one 16-byte LDS write and (VT / TPW - 1) 16-byte LDS reads per lane
// per step, with no shuffles or transposes.
//
// Per step: rank-1 term k_i v_j as the accumulator's initial value, 4 * VT
// MFMAs per tile, tanh, the f-lerp, an LDS exchange with one barrier, and the
// readout y_j = sum_i H_ij q_i as a DPP reduction over the 16 lanes of a row.
// k, q, v, f are staged through LDS in chunks of TC steps (coalesced global
// loads issued one chunk ahead); readouts are staged per chunk and written
// back coalesced.

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

template <typename Real, int VT>
struct FwdTraits {
  static constexpr int VP = 16 * VT;                 // padded value width
  static constexpr int NW = VT <= 4 ? VT : VT / 2;   // waves per workgroup
  static constexpr int TPW = VT / NW;                // 16-column tiles per wave
  static constexpr int NT = 64 * NW;                 // threads per workgroup
  static constexpr int NS = 4 * VT;                  // MFMAs per tile per step
  static constexpr int TC = sizeof(Real) == 4 ? (VP <= 64 ? 32 : 16)
                                              : (VP <= 32 ? 32 : (VP <= 64 ? 16 : 4));
  static constexpr int NV_PER = (TC * VP + NT - 1) / NT;   // staged v values per thread
  static constexpr int NKQ_PER = (TC * 32 + NT - 1) / NT;  // staged k and q values per thread
  static constexpr int NY_PER = NV_PER;
};

template <typename Real, int VT, int TC>
struct FwdSmem {
  using R4 = typename Vec4<Real>::type;
  R4 xb[2][VT][64];           // state exchange, double-buffered by step parity
  Real kq[2][TC][16][2];      // staged (k_i, q_i) per step
  Real v[2][TC][16 * VT];     // staged v per step
  Real y[2][TC][16 * VT];     // readouts of a chunk, written back together
  Real f[2][TC];              // staged gate
  Real wr[16 * VT];           // w_r of this head
};

template <typename InT, typename Real, int VT>
__global__ void __launch_bounds__((FwdTraits<Real, VT>::NT))
    m2rnn_fwd_kernel(FwdArgs a) {
  using Tr = FwdTraits<Real, VT>;
  using R4 = typename Vec4<Real>::type;
  constexpr int VP = Tr::VP, TPW = Tr::TPW, NS = Tr::NS, TC = Tr::TC, NT = Tr::NT;
  __shared__ FwdSmem<Real, VT, TC> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int nslab = a.nslab;
  const int slab = unit % nslab;
  const int bn = unit / nslab;
  const int64_t B = a.B, T = a.T, N = a.N, K = a.K, V = a.V;
  const int n = (int)(bn % N);
  const int b = (int)(bn / N);
  const int row = slab * 16 + li;
  const bool row_ok = row < K;

  const InT* __restrict__ kp = (const InT*)a.k;
  const InT* __restrict__ vp = (const InT*)a.v;
  const InT* __restrict__ qp = (const InT*)a.q;
  const Real* __restrict__ fp = (const Real*)a.f;
  const Real* __restrict__ Wp = (const Real*)a.W;
  const Real* __restrict__ wrp = (const Real*)a.w_r;

  // ---- W^T as the MFMA A operand, rotated so this wave's own tiles come first.
  Real wa[TPW][NS];
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
    const int col = (w * TPW + p) * 16 + li;
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) {
      const int s = (s0 + 4 * TPW * w) % NS;
      const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
      wa[p][s0] = (col < V && l < V) ? Wp[((int64_t)n * V + l) * V + col] : Real(0);
    }
  }

  // ---- initial state: own tiles hold row `row`, columns 16 c + m(g, r).
  R4 hown[TPW];
  const int64_t state_base = (((int64_t)b * N + n) * K + row) * V;
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = (w * TPW + p) * 16 + acc_m<Real>(g, r);
      hown[p][r] = (a.H0 && row_ok && col < V) ? ((const Real*)a.H0)[state_base + col] : Real(0);
    }
  }
  const int64_t nck = a.ckpt ? (T + a.C - 1) / a.C : 0;
  auto write_state = [&](Real* dst) {
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = (w * TPW + p) * 16 + acc_m<Real>(g, r);
        if (row_ok && col < V) dst[col] = hown[p][r];
      }
    }
  };
  if (a.ckpt) write_state((Real*)a.ckpt + ((((int64_t)b * N + n) * nck + 0) * K + row) * V);

  // ---- staging of k, q, v, f for one chunk of TC steps.
  Real st_v[Tr::NV_PER], st_kq[Tr::NKQ_PER], st_f = Real(0);
  auto load_chunk = [&](int64_t t0) {
#pragma unroll
    for (int m = 0; m < Tr::NV_PER; ++m) {
      const int e = tid + m * NT;
      const int tt = e / VP, j = e % VP;
      const int64_t t = t0 + tt;
      st_v[m] = (tt < TC && j < V && t < T)
                    ? load_as<Real>(vp + (((int64_t)b * T + t) * N + n) * V + j) : Real(0);
    }
#pragma unroll
    for (int m = 0; m < Tr::NKQ_PER; ++m) {
      const int e = tid + m * NT;
      const int tt = e >> 5, which = (e >> 4) & 1, i = e & 15;
      const int64_t t = t0 + tt;
      const int rr = slab * 16 + i;
      const InT* src = which ? qp : kp;
      st_kq[m] = (tt < TC && rr < K && t < T)
                     ? load_as<Real>(src + (((int64_t)b * T + t) * N + n) * K + rr) : Real(0);
    }
    if (tid < TC) {
      const int64_t t = t0 + tid;
      st_f = (t < T) ? fp[((int64_t)b * T + t) * N + n] : Real(0);
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int m = 0; m < Tr::NV_PER; ++m) {
      const int e = tid + m * NT;
      if (e < TC * VP) sm.v[buf][e / VP][e % VP] = st_v[m];
    }
#pragma unroll
    for (int m = 0; m < Tr::NKQ_PER; ++m) {
      const int e = tid + m * NT;
      if (e < TC * 32) sm.kq[buf][e >> 5][e & 15][(e >> 4) & 1] = st_kq[m];
    }
    if (tid < TC) sm.f[buf][tid] = st_f;
  };

  for (int j = tid; j < VP; j += NT) sm.wr[j] = j < V ? wrp[(int64_t)n * V + j] : Real(0);
  load_chunk(0);
  store_chunk(0);

  // ---- first exchange: the full slab of H_0 as the B operand.
  Real hb[NS];
#pragma unroll
  for (int p = 0; p < TPW; ++p) sm.xb[1][w * TPW + p][lane] = hown[p];
  __syncthreads();
#pragma unroll
  for (int q0 = 0; q0 < VT; ++q0) {
    R4 t4;
    if (q0 < TPW) {
      t4 = hown[q0];
    } else {
      t4 = sm.xb[1][(q0 + TPW * w) % VT][lane];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
  }

  Real* __restrict__ yout = (Real*)a.y;
  Real* __restrict__ ypart = (Real*)a.ypart;
  const int64_t slab_stride = B * T * N * V;

  const int64_t nchunks = (T + TC - 1) / TC;
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t t0 = ch * TC;
    const int tn = (int)((T - t0) < TC ? (T - t0) : TC);
    const int sb = (int)(ch & 1);
    const bool more = ch + 1 < nchunks;
    if (more) load_chunk(t0 + TC);

    for (int tt = 0; tt < tn; ++tt) {
      const int64_t t = t0 + tt;
      const Real kv = sm.kq[sb][tt][li][0];
      const Real qv = sm.kq[sb][tt][li][1];
      const Real ft = sm.f[sb][tt];
      R4 acc[TPW];
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
#pragma unroll
        for (int r = 0; r < 4; ++r)  // rank-1 write k_i v_j
          acc[p][r] = kv * sm.v[sb][tt][(w * TPW + p) * 16 + acc_m<Real>(g, r)];
      }
#pragma unroll
      for (int s0 = 0; s0 < NS; ++s0) {
#pragma unroll
        for (int p = 0; p < TPW; ++p) acc[p] = mfma_16x16x4(wa[p][s0], hb[s0], acc[p]);
      }
      // tanh and the gate interpolation H = f H_prev + (1 - f) Z, written as in
      // Eq. (11) so that f = 1 keeps H exactly and f = 0 gives exactly Z
      const Real omf = Real(1) - ft;
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const Real z = tanh_fast(acc[p][r]);
          hown[p][r] = ft * hown[p][r] + omf * z;
        }
      }
      const int xbuf = (int)(t & 1);
#pragma unroll
      for (int p = 0; p < TPW; ++p) sm.xb[xbuf][w * TPW + p][lane] = hown[p];

      // readout of the updated state: sum over the 16 rows of the slab
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        Real yv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) yv[r] = row16_sum(hown[p][r] * qv);
        if (li == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.y[sb][tt][(w * TPW + p) * 16 + acc_m<Real>(g, r)] = yv[r];
        }
      }
      if (a.ckpt && ((t + 1) % a.C) == 0 && (t + 1) < T) {
        write_state((Real*)a.ckpt + ((((int64_t)b * N + n) * nck + (t + 1) / a.C) * K + row) * V);
      }
      if (more && tt == tn - 1) store_chunk(sb ^ 1);
      __syncthreads();
#pragma unroll
      for (int q0 = TPW; q0 < VT; ++q0) {
        const R4 t4 = sm.xb[xbuf][(q0 + TPW * w) % VT][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
      }
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
#pragma unroll
        for (int r = 0; r < 4; ++r) hb[4 * p + r] = hown[p][r];
      }
    }

    // write back this chunk's readouts (partial over the slab's rows)
#pragma unroll
    for (int m = 0; m < Tr::NY_PER; ++m) {
      const int e = tid + m * NT;
      const int tt = e / VP, j = e % VP;
      if (tt < tn && j < V) {
        const int64_t off = (((int64_t)b * T + t0 + tt) * N + n) * V + j;
        const Real val = sm.y[sb][tt][j];
        if (nslab == 1) {
          yout[off] = val + sm.wr[j] * sm.v[sb][tt][j];
        } else {
          ypart[slab * slab_stride + off] = val;
        }
      }
    }
  }
  if (a.HT) write_state((Real*)a.HT + state_base);
}

// y = sum over slabs of the partial readouts + w_r (.) v   (elementwise, HBM-bound)
template <typename InT, typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_fwd_reduce_kernel(int64_t total, int64_t N, int64_t V, int nslab,
                            const Real* __restrict__ ypart, const InT* __restrict__ v,
                            const Real* __restrict__ w_r, Real* __restrict__ y) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    Real s = ypart[i];
    for (int sl = 1; sl < nslab; ++sl) s += ypart[sl * total + i];
    const int64_t j = i % V;
    const int64_t n = (i / V) % N;
    y[i] = s + w_r[n * V + j] * load_as<Real>(v + i);
  }
}

template <typename InT, typename Real, int VT>
static hipError_t launch_fwd_vt(const FwdArgs& a, hipStream_t stream) {
  using Tr = FwdTraits<Real, VT>;
  static_assert(sizeof(FwdSmem<Real, VT, Tr::TC>) <= 65536, "LDS budget");
  const int64_t units = a.B * a.N * a.nslab;
  hipLaunchKernelGGL((m2rnn_fwd_kernel<InT, Real, VT>), dim3((unsigned)units), dim3(Tr::NT), 0,
                     stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nslab == 1) return err;
  const int64_t total = a.B * a.T * a.N * a.V;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((m2rnn_fwd_reduce_kernel<InT, Real>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, total, a.N, a.V, a.nslab, (const Real*)a.ypart, (const InT*)a.v,
                     (const Real*)a.w_r, (Real*)a.y);
  return hipGetLastError();
}

template <typename InT, typename Real>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  switch (value_tiles(a.V)) {
    case 1: return launch_fwd_vt<InT, Real, 1>(a, stream);
    case 2: return launch_fwd_vt<InT, Real, 2>(a, stream);
    case 3: return launch_fwd_vt<InT, Real, 3>(a, stream);
    case 4: return launch_fwd_vt<InT, Real, 4>(a, stream);
    case 6: return launch_fwd_vt<InT, Real, 6>(a, stream);
    case 8: return launch_fwd_vt<InT, Real, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd(const FwdArgs& a, int in_dtype, int state_dtype, hipStream_t stream) {
  if (state_dtype == kF32) {
    if (in_dtype == kF32) return launch_fwd_t<float, float>(a, stream);
    if (in_dtype == kBF16) return launch_fwd_t<uint16_t, float>(a, stream);
  } else if (state_dtype == kF64) {
    if (in_dtype == kF64) return launch_fwd_t<double, double>(a, stream);
    if (in_dtype == kBF16) return launch_fwd_t<uint16_t, double>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace m2rnn
