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
                                              : (VP <= 32 ? 32 : (VP <= 64 ? 16 : 8));
  static constexpr int NV_PER = (TC * VP + NT - 1) / NT;   // staged v values per thread
  static constexpr int NKQ_PER = (TC * 32 + NT - 1) / NT;  // staged k and q values per thread
  static_assert(TC >= 4, "a staging chunk must hold at least 4 steps");
};

template <typename Real, int VT, int TC, int NT>
struct FwdSmem {
  using R4 = typename Vec4<Real>::type;
  R4 xb[2][VT][64];           // state exchange, double-buffered by step parity
  R4 y[2][TC][4 * VT];        // partial readouts, lane order (16 c + 4 g + r), per chunk
  R4 ydump[NT];               // sink for the readout writes of lanes that hold no result
  Real kq[2][TC][16][2];      // staged (k_i, q_i) per step
  Real v[2][TC][16 * VT];     // staged v per step
  Real f[2][TC];              // staged gate
  Real wr[16 * VT];           // w_r of this head
};

template <typename InT, typename Real, int VT>
__global__ void __launch_bounds__((FwdTraits<Real, VT>::NT))
    m2rnn_fwd_kernel(FwdArgs a) {
  using Tr = FwdTraits<Real, VT>;
  using R4 = typename Vec4<Real>::type;
  constexpr int VP = Tr::VP, TPW = Tr::TPW, NS = Tr::NS, TC = Tr::TC, NT = Tr::NT;
  __shared__ FwdSmem<Real, VT, TC, NT> sm;

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
  Real* ck_next = nullptr;   // where the next checkpoint goes
  if (a.ckpt) {
    Real* ck0 = (Real*)a.ckpt + ((((int64_t)b * N + n) * nck) * K + row) * V;
    write_state(ck0);
    ck_next = ck0 + K * V;
  }
  const int64_t ck_stride = K * V;

  // ---- staging of k, q, v, f for one chunk of TC steps.
  Real st_v[Tr::NV_PER], st_kq[Tr::NKQ_PER], st_f = Real(0);
  // Every load is issued unconditionally from a clamped (in-bounds) address and
  // masked afterwards, so the loads of a chunk are all in flight at once.
  auto load_chunk = [&](int64_t t0) {
#pragma unroll
    for (int m = 0; m < Tr::NV_PER; ++m) {
      const int e = tid + m * NT;
      const int tt = e / VP, j = e % VP;
      const int64_t t = t0 + tt;
      const bool ok = tt < TC && j < V && t < T;
      const int64_t tc = clamp_idx(t, T - 1);
      st_v[m] = load_sel<Real>(vp, (((int64_t)b * T + tc) * N + n) * V + clamp_idx(j, V - 1), ok);
    }
#pragma unroll
    for (int m = 0; m < Tr::NKQ_PER; ++m) {
      const int e = tid + m * NT;
      const int tt = e >> 5, which = (e >> 4) & 1, i = e & 15;
      const int64_t t = t0 + tt;
      const int rr = slab * 16 + i;
      const bool ok = tt < TC && rr < K && t < T;
      const int64_t tc = clamp_idx(t, T - 1);
      const InT* src = which ? qp : kp;
      st_kq[m] = load_sel<Real>(src, (((int64_t)b * T + tc) * N + n) * K + clamp_idx(rr, K - 1), ok);
    }
    {
      const int64_t t = t0 + tid;
      const bool ok = tid < TC && t < T;
      st_f = load_sel<Real>(fp, ((int64_t)b * T + clamp_idx(t, T - 1)) * N + n, ok);
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

  Real* __restrict__ yout = (Real*)a.y;
  Real* __restrict__ ypart = (Real*)a.ypart;
  const int64_t slab_stride = B * T * N * V;
  // write back one chunk of partial readouts (the y staging is in lane order)
  auto flush = [&](int64_t ch, int buf) {
    const int64_t t0 = ch * TC;
    const int tn = (int)((T - t0) < TC ? (T - t0) : TC);
    for (int e = tid; e < TC * VP; e += NT) {
      const int tt = e / VP, jl = e % VP;
      const int c = jl >> 4, gg = (jl >> 2) & 3, rr = jl & 3;
      const int j = c * 16 + acc_m<Real>(gg, rr);
      if (tt < tn && j < V) {
        const int64_t off = (((int64_t)b * T + t0 + tt) * N + n) * V + j;
        const Real val = sm.y[buf][tt][jl >> 2][rr];
        if (nslab == 1) {
          yout[off] = val + sm.wr[j] * sm.v[buf][tt][j];
        } else {
          ypart[slab * slab_stride + off] = val;
        }
      }
    }
  };

  const int64_t nchunks = (T + TC - 1) / TC;
  for (int j = tid; j < VP; j += NT) sm.wr[j] = j < V ? wrp[(int64_t)n * V + j] : Real(0);
  load_chunk(0);
  store_chunk(0);
  if (nchunks > 1) load_chunk(TC);

  // ---- first exchange: the full slab of H_0 as the B operand.
  Real hb[NS];
#pragma unroll
  for (int p = 0; p < TPW; ++p) sm.xb[1][w * TPW + p][lane] = hown[p];
  __syncthreads();
#pragma unroll
  for (int q0 = 0; q0 < VT; ++q0) {
    const R4 t4 = q0 < TPW ? hown[q0] : sm.xb[1][(q0 + TPW * w) % VT][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
  }

  // ---- inputs of step 0
  R4 acc_init[TPW];
  Real q_cur, f_cur;
  {
    const Real kv = sm.kq[0][0][li][0];
    q_cur = sm.kq[0][0][li][1];
    f_cur = sm.f[0][0];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc_init[p][r] = kv * sm.v[0][0][(w * TPW + p) * 16 + acc_m<Real>(g, r)];
  }
  Real q_prev = Real(0);
  // Readout destination of the previous step.  Lane 0 of each 16-lane group
  // holds the row sums and writes them (tile p at yslot + 4 p); every other
  // lane writes its own slot of ydump, so the store needs no branch.  Step 0
  // has no previous step: everyone writes ydump.
  R4* const ydump_me = &sm.ydump[tid];
  R4* yslot = ydump_me;
  const int ystep_writer = li == 0 ? 4 : 0;
  int ystep = 0;
  // y staging address of this lane for circular slot 0 (writers only)
  R4* const ybase = li == 0 ? &sm.y[0][0][(w * TPW) * 4 + g] : ydump_me;
  const int yslot_stride = li == 0 ? 4 * VT : 0;  // R4 elements per staging slot

  // One recurrence step.  si is the circular staging slot (0 .. 2 TC - 1) of
  // step t; the staging arrays are [2][TC] = [2 TC] consecutive slots.
  auto step = [&](int64_t t, int si) {
    const int si1 = si + 1 == 2 * TC ? 0 : si + 1;   // slot of step t + 1
    const Real* kq1 = &sm.kq[0][0][0][0] + si1 * 32;
    const Real* v1 = &sm.v[0][0][0] + si1 * VP;

    R4 acc[TPW];
#pragma unroll
    for (int p = 0; p < TPW; ++p) acc[p] = acc_init[p];
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) {
#pragma unroll
      for (int p = 0; p < TPW; ++p) acc[p] = mfma_16x16x4(wa[p][s0], hb[s0], acc[p]);
    }
    // ---- work independent of the MFMA chain (scheduled into its shadow)
    // readout of the previous step, y_{t-1} = H_t^T q_{t-1} over this slab's rows
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      R4 yv;
#pragma unroll
      for (int r = 0; r < 4; ++r) yv[r] = row16_sum(hown[p][r] * q_prev);
      yslot[p * ystep] = yv;
    }
    // next step's inputs
    const Real kv = kq1[li * 2 + 0];
    const Real qn = kq1[li * 2 + 1];
    const Real fn = (&sm.f[0][0])[si1];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_init[p][r] = kv * v1[(w * TPW + p) * 16 + acc_m<Real>(g, r)];
    q_prev = q_cur;
    q_cur = qn;
    // interleave: one MFMA, then up to two VALU ops and one LDS read
#pragma unroll
    for (int s0 = 0; s0 < NS * TPW; ++s0) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // ---- dependent tail: tanh, gate interpolation H = f H + (1 - f) Z
    const Real ft = f_cur;
    const Real omf = Real(1) - ft;
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const Real z = tanh_fast(acc[p][r]);
        hown[p][r] = ft * hown[p][r] + omf * z;
      }
    }
    f_cur = fn;
    const int xbuf = (int)(t & 1);
#pragma unroll
    for (int p = 0; p < TPW; ++p) sm.xb[xbuf][w * TPW + p][lane] = hown[p];
    // the readout of this step lands in staging slot si
    yslot = ybase + si * yslot_stride;
    ystep = ystep_writer;
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
      for (int r = 0; r < 4; ++r) hb[4 * p + r] = hown[p][r];
  };

  // Steps run in branch-free segments; the rare events (checkpoint, LDS
  // staging of the next chunk, write-back of readouts, prefetch) happen only
  // between segments.  Event points, as the last step of a segment:
  //   local step 0 of chunk ch > 0 : chunk ch - 1 is complete -> write back
  //   local step TC - 3            : stage chunk ch + 1 into LDS
  //   local step TC - 1            : end of chunk -> prefetch chunk ch + 2
  //   (t + 1) % C == 0             : checkpoint H_{t+1}
  int64_t next_ck = a.ckpt ? a.C - 1 : T;  // step after which the next checkpoint is taken
  int64_t ch = 0;
  int64_t t = 0;
  while (t < T) {
    const int64_t t0 = ch * TC;
    const int tt = (int)(t - t0);
    int64_t e = t0 + TC - 1;
    if (tt <= TC - 3) e = t0 + TC - 3;
    if (tt == 0) e = t0;
    if (next_ck < e) e = next_ck;
    if (T - 1 < e) e = T - 1;
    const int sb = (int)(ch & 1);
    int si = sb * TC + tt;
    for (; t <= e; ++t, ++si) step(t, si);
    // ---- events after step e (uniform)
    const int te = (int)(e - t0);
    if (e == next_ck) {
      if (e + 1 < T) {
        write_state(ck_next);
        ck_next += ck_stride;
      }
      next_ck += a.C;
    }
    if (te == 0 && ch > 0) flush(ch - 1, sb ^ 1);
    if (te == TC - 3 && ch + 1 < nchunks) store_chunk(sb ^ 1);
    if (te == TC - 1) {
      if (ch + 2 < nchunks) load_chunk((ch + 2) * TC);
      ++ch;
    }
  }
  // readout of the last step, then the last chunk
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
    R4 yv;
#pragma unroll
    for (int r = 0; r < 4; ++r) yv[r] = row16_sum(hown[p][r] * q_prev);
    yslot[p * ystep] = yv;
  }
  __syncthreads();
  flush(nchunks - 1, (int)((nchunks - 1) & 1));
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
  static_assert(sizeof(FwdSmem<Real, VT, Tr::TC, Tr::NT>) <= 160 * 1024, "LDS budget");
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
