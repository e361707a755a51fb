// Fused M²RNN forward for gfx950.
//
// Computes, for every (batch b, head n), the recurrence of the M²RNN review
// (section 2.1, Eq. 10-12):
//     Z_t = tanh(H_{t-1} W_n + k_t v_t^T),  H_t = f_t H_{t-1} + (1 - f_t) Z_t,
//     y_t = H_t^T q_t + w_r (.) v_t.
//
// Work decomposition.  W mixes value columns only, so the K rows of a head are
// independent recurrences (they meet only in the readout sum over rows).  A
// unit of VT / TPW waves owns one 16-row slab of one head for all T steps; a
// head with K rows becomes ceil(K / 16) units, and their partial readouts are
// summed by a second, elementwise kernel.  A workgroup is one unit, except
// that one-wave units (V <= 16) are packed four to a workgroup so that each
// takes its own SIMD.
//
// MFMA formulation.  The step is computed transposed, (H W)^T = W^T H^T, on
// the 16x16x4 MFMA: W^T is the A operand (held in registers for the whole
// sequence), H^T the B operand.  The MFMA result layout (lane l holds row
// l % 16 and, in element r, column 16 c + m(g, r) with g = l / 16 and m the
// instruction's accumulator row map) is exactly the B-operand layout of the
// next step when the contraction index of MFMA number s is enumerated as
// pi(s, g) = 16 (s / 4) + m(g, s % 4).  So a wave's own 16-column tiles never
// leave registers, and the other tiles of the slab arrive through one 16-byte
// LDS write and (VT / TPW - 1) 16-byte LDS reads per lane per step.  The
// rank-1 write k v^T initialises the accumulators (one multiply per element).
// The step works with the pre-activation scaled by 2 / ln 2 (W^T is scaled
// when loaded, k per step), which the base-2 exponential of tanh takes as is.
//
// Step schedule.  On gfx950 fp32 MFMA and VALU work of a SIMD do not overlap
// (not even for different waves), so every VALU instruction of a step adds to
// the step time.  The step
// is therefore: MFMAs (own tiles first: no LDS wait), tanh and the gate
// interpolation, the exchange write, then the readout y_t = H_t^T q_t as a DPP
// reduction over the 16 rows -- placed where the wave would otherwise wait for
// its exchange write to land -- then the barrier and the exchange reads.
// Inputs come from an LDS staging ring laid out so that each step needs only
// immediate-offset reads; each staging chunk of TC steps is unrolled, and the
// global traffic of inputs and readouts (prefetch, write-back) happens between
// chunks, from pointers that step forward one chunk at a time (no index
// arithmetic in the loop).  Checkpoints are written after the steps they
// follow, counted down on the scalar unit.

#include <type_traits>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

template <typename Real, int VT>
struct FwdTraits {
  static constexpr int VP = 16 * VT;                 // padded value width
  static constexpr int NW = VT <= 4 ? VT : VT / 2;   // waves per workgroup
  static constexpr int TPW = VT / NW;                // 16-column tiles per wave
  static constexpr int NT = 64 * NW;                 // threads per unit (16-row slab)
  // Units per workgroup.  A one-wave unit (V <= 16) shares a workgroup with
  // three others, each wave on its own SIMD of the compute unit: launched as
  // one-wave workgroups, two of them often land on one SIMD and serialise.
  static constexpr int PACK = NW == 1 ? 4 : 1;
  static constexpr int NS = 4 * VT;                  // MFMAs per tile per step (H W)
  static constexpr int TC = sizeof(Real) == 4 ? (VT <= 4 ? 32 : 16) : 8;  // steps per staging chunk (unrolled)
  static constexpr int RING = 2 * TC;                     // staging ring: two chunks
  // per chunk: v [TC][VP], k and q [TC][16], f [TC]
  static constexpr int NV_PER = (TC * VP + NT - 1) / NT;   // v values per thread
  static constexpr int NQ_PER = (TC * 16 + NT - 1) / NT;   // (k, q) pairs per thread
};

template <typename Real, int VT, int NW, int RING>
struct FwdSmem {
  using R4 = typename Vec4<Real>::type;
  using R2 = typename Vec2<Real>::type;
  R4 xb[2][VT][64];           // state exchange, double-buffered by step parity
  // readout partials [slot][tile][g][i]: sums over this slab's rows i, i + 4,
  // i + 8, i + 12 of the lane group's four columns; the write-back adds the four
  R4 y[RING][VT][4][4];
  R4 ydump[NW * 64];          // sink for readout stores of lanes that hold no result
  Real v[RING][16 * VT];      // v_j of a step
  Real k[RING][16];           // k_i of a step (this slab's rows)
  R2 fg[RING];                // (f, 1 - f) of a step
  Real q[RING][16];           // q_i of a step
};

// RCS: also store every step's rc.  FULL: every row of the slab and every
// column of the tiles exists and the state is fp32, so each lane's rc,
// checkpoint and final-state stores are unguarded 16-byte stores; the guards
// (branches on row and column) cost more than the stores themselves.
template <typename InT, typename Real, int VT, bool RCS, bool FULL>
__global__ void __launch_bounds__((FwdTraits<Real, VT>::NT * FwdTraits<Real, VT>::PACK))
    m2rnn_fwd_kernel(FwdArgs a) {
  using Tr = FwdTraits<Real, VT>;
  using R4 = typename Vec4<Real>::type;
  using R2 = typename Vec2<Real>::type;
  constexpr int VP = Tr::VP, TPW = Tr::TPW, NS = Tr::NS, TC = Tr::TC, NT = Tr::NT;
  constexpr int RING = Tr::RING, PACK = Tr::PACK;
  __shared__ FwdSmem<Real, VT, Tr::NW, RING> smp[PACK];

  // with PACK > 1 every wave is a unit of its own: thread indices are
  // wave-relative and the unit's LDS is the wave's own slice
  const int wu = PACK > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
  FwdSmem<Real, VT, Tr::NW, RING>& sm = smp[wu];
  const int tid = PACK > 1 ? (int)threadIdx.x & 63 : (int)threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int unit = xcd_remap(blockIdx.x, gridDim.x) * PACK + wu;
  if (PACK > 1 && unit >= a.B * a.N * a.nslab) return;  // no barrier couples the waves
  // Orders the unit's LDS accesses.  A one-wave unit's LDS operations complete
  // in program order, so only the compiler must not move them across.
  auto unit_sync = [] {
    if constexpr (PACK > 1) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      __syncthreads();
    }
  };
  const int nslab = a.nslab;
  const int slab = unit % nslab;
  const int bn = unit / nslab;
  const int64_t B = a.B, T = a.T, N = a.N, K = a.K, V = a.V;
  const int n = (int)(bn % N);
  const int b = (int)(bn / N);
  const int row = slab * 16 + li;
  const bool row_ok = row < K;
  const int64_t state_base = (((int64_t)b * N + n) * K + row) * V;

  const InT* __restrict__ kp = (const InT*)a.k;
  const InT* __restrict__ vp = (const InT*)a.v;
  const InT* __restrict__ qp = (const InT*)a.q;
  const Real* __restrict__ fp = (const Real*)a.f;
  const Real* __restrict__ Wp = (const Real*)a.W;
  const Real* __restrict__ wrp = (const Real*)a.w_r;
  Real* __restrict__ yout = (Real*)a.y;
  Real* __restrict__ ypart = (Real*)a.ypart;
  const int64_t slab_stride = B * T * N * V;
  auto col_of = [&](int p, int r) { return (w * TPW + p) * 16 + acc_m<Real>(g, r); };

  // ---- W^T as the MFMA A operand, rotated so this wave's own tiles come first,
  // scaled by 2 / ln 2 (the step works with the scaled pre-activation).
  Real wa[TPW][NS];
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
    const int col = (w * TPW + p) * 16 + li;
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) {
      const int s = (s0 + 4 * TPW * w) % NS;
      const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
      wa[p][s0] = Wp[((int64_t)n * V + (l < V ? l : 0)) * V + (col < V ? col : 0)];
    }
  }
  // the loads complete together, then the padding is masked (a guarded load
  // would be a branch whose join waits for it, one load at a time)
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
    const int col = (w * TPW + p) * 16 + li;
#pragma unroll
    for (int s0 = 0; s0 < NS; s0 += 4) pin_values(wa[p][s0], wa[p][s0 + 1], wa[p][s0 + 2], wa[p][s0 + 3]);
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) {
      const int s = (s0 + 4 * TPW * w) % NS;
      const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
      wa[p][s0] = (col < V && l < V) ? kTanhScale<Real> * wa[p][s0] : Real(0);
    }
    // the final operands are held in registers (not recomputed in the loop)
#pragma unroll
    for (int s0 = 0; s0 < NS; s0 += 4) pin_values(wa[p][s0], wa[p][s0 + 1], wa[p][s0 + 2], wa[p][s0 + 3]);
  }

  // ---- initial state: own tiles hold row `row`, columns 16 c + m(g, r).
  R4 hown[TPW];
#pragma unroll
  for (int p = 0; p < TPW; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = col_of(p, r);
      hown[p][r] = (a.H0 && row_ok && col < V) ? ((const Real*)a.H0)[state_base + col] : Real(0);
    }
  const int64_t nck = a.ckpt ? (T + a.C - 1) / a.C : 0;
  // where a lane's four columns are consecutive (fp32) and the arrays are
  // 16-byte aligned, one 16-byte store
  const bool st_vec = sizeof(Real) == 4 && a.st_vec;
  // this lane's values of a [K, V] array (row `row`, its tiles' columns)
  auto write_rows = [&](Real* dst, const R4 (&val)[TPW]) {
    if constexpr (FULL) {  // every row and column exists: one 16-byte store per tile
#pragma unroll
      for (int p = 0; p < TPW; ++p) *(R4*)(dst + col_of(p, 0)) = val[p];
      return;
    }
    if (!row_ok) return;
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      if (st_vec) {
        if (col_of(p, 0) < V) *(R4*)(dst + col_of(p, 0)) = val[p];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = col_of(p, r);
          if (col < V) dst[col] = val[p][r];
        }
      }
    }
  };
  auto write_state = [&](Real* dst) { write_rows(dst, hown); };
  // checkpoints H_{cC}, c = 0 .. nck - 1, are written in order: ckp is the
  // next one's slot, and ck_left counts the steps until it is due
  Real* ckp = a.ckpt ? (Real*)a.ckpt + (((int64_t)b * N + n) * nck * K + row) * V : nullptr;
  const int64_t KV = K * V;
  const int C32 = a.ckpt ? (int)a.C : 0;
  int ck_left = C32;
  if (a.ckpt) {
    write_state(ckp);
    ckp += KV;
  }
  // rc_t = 1 / (1 + e^{2 A_t}) of every step, [B, N, T, K, V] (RCS only)
  Real* rcp = RCS ? (Real*)a.rc + (((int64_t)b * N + n) * T * K + row) * V : nullptr;
  // after step t (t + 1 steps done): write H_{t+1} when it is due and not H_T
  auto ck_step = [&](int t) {
    if (C32 == 0) return;
    if (--ck_left == 0) {
      ck_left = C32;
      if (t + 1 < (int)T) {
        write_state(ckp);
        ckp += KV;
      }
    }
  };

  // ---- staging of one chunk of TC steps.  Each thread owns a fixed set of
  // (step-in-chunk, index) elements, so its global addresses for chunk ch are
  // fixed offsets plus ch * TC * (elements per step); they are computed once.
  // Loads are unconditional (a chunk's loads are all in flight at once); in
  // the last chunk the step index is clamped to T - 1 and the value masked.
  const int64_t NV = N * V, NK = a.NQ * K;
  const int64_t tok0 = (int64_t)b * T * N + n;       // token index of (b, t = 0, n)
  // q and k rows of (b, t = 0): head n / (N / NQ) of the NQ shared heads
  const int64_t tokq0 = (int64_t)b * T * a.NQ + n / (int)(N / a.NQ);
  const int T32 = (int)T;                             // T < 2^30
  // Each thread owns a fixed set of (step-in-chunk, index) elements.  Chunks
  // are loaded in order, so each element's source pointer steps forward by
  // one chunk (TC tokens) per load; the last, partial chunk clamps its steps
  // to T - 1 and masks them.  Loads are unconditional (all of a chunk's loads
  // are in flight at once).
  const InT* v_p[Tr::NV_PER];
  const InT* k_p[Tr::NQ_PER];
  const InT* q_p[Tr::NQ_PER];
  int v_tt[Tr::NV_PER], q_tt[Tr::NQ_PER];
  bool v_ok[Tr::NV_PER], q_ok[Tr::NQ_PER];
#pragma unroll
  for (int m = 0; m < Tr::NV_PER; ++m) {
    const int e = tid + m * NT;                      // [tt][j]
    const int tt = e / VP, j = e % VP;
    v_tt[m] = tt < TC ? tt : 0;
    v_ok[m] = tt < TC && j < V;
    v_p[m] = vp + tok0 * V + (j < V ? j : V - 1) + (int64_t)v_tt[m] * NV;
  }
#pragma unroll
  for (int m = 0; m < Tr::NQ_PER; ++m) {
    const int e = tid + m * NT;                      // [tt][i]
    const int tt = e / 16, i = e % 16, rr = slab * 16 + i;
    q_tt[m] = tt < TC ? tt : 0;
    q_ok[m] = tt < TC && rr < K;
    k_p[m] = kp + tokq0 * K + (rr < K ? rr : K - 1) + (int64_t)q_tt[m] * NK;
    q_p[m] = qp + tokq0 * K + (rr < K ? rr : K - 1) + (int64_t)q_tt[m] * NK;
  }
  const int f_tt = tid < TC ? tid : 0;
  const Real* f_p = fp + tok0 + (int64_t)f_tt * N;
  // Raw loaded values stay in registers until the LDS store during the next
  // chunk (conversion and masking happen there), so nothing waits for the
  // loads at the chunk boundary.
  InT st_v[Tr::NV_PER], st_k[Tr::NQ_PER], st_q[Tr::NQ_PER];
  Real st_f;
  bool st_in[Tr::NV_PER], st_qin[Tr::NQ_PER], st_fin;  // step within T
  // load chunk ch (chunks in order: the pointers are at chunk ch on entry)
  auto load_chunk = [&](int ch) {
    const int t0 = ch * TC;
    if (t0 + TC <= T32) {
#pragma unroll
      for (int m = 0; m < Tr::NV_PER; ++m) {
        st_v[m] = *v_p[m];
        st_in[m] = true;
      }
#pragma unroll
      for (int m = 0; m < Tr::NQ_PER; ++m) {
        st_k[m] = *k_p[m];
        st_q[m] = *q_p[m];
        st_qin[m] = true;
      }
      st_f = *f_p;
      st_fin = true;
    } else {  // the last chunk: steps past T read step T - 1 and are masked
      const int lim = T32 - 1 - t0;  // last step of the chunk within T, relative
#pragma unroll
      for (int m = 0; m < Tr::NV_PER; ++m) {
        const int64_t back = v_tt[m] > lim ? v_tt[m] - lim : 0;
        st_v[m] = v_p[m][-back * NV];
        st_in[m] = v_tt[m] <= lim;
      }
#pragma unroll
      for (int m = 0; m < Tr::NQ_PER; ++m) {
        const int64_t back = q_tt[m] > lim ? q_tt[m] - lim : 0;
        st_k[m] = k_p[m][-back * NK];
        st_q[m] = q_p[m][-back * NK];
        st_qin[m] = q_tt[m] <= lim;
      }
      const int64_t back = f_tt > lim ? f_tt - lim : 0;
      st_f = f_p[-back * N];
      st_fin = f_tt <= lim;
    }
#pragma unroll
    for (int m = 0; m < Tr::NV_PER; ++m) v_p[m] += TC * NV;
#pragma unroll
    for (int m = 0; m < Tr::NQ_PER; ++m) {
      k_p[m] += TC * NK;
      q_p[m] += TC * NK;
    }
    f_p += TC * N;
  };
  // a raw value, converted in a register (a select between a loaded value and
  // zero is otherwise turned into a load from a select of addresses)
  auto held = [&](auto x) -> Real {
    Real y = (Real)widen(x);
    asm volatile("" : "+v"(y));
    return y;
  };
  auto store_chunk = [&](int ch) {
    const int base = (ch & 1) * TC;
#pragma unroll
    for (int m = 0; m < Tr::NV_PER; ++m) {
      const int e = tid + m * NT;
      const Real vv = held(st_v[m]);
      if (e < TC * VP) sm.v[base + e / VP][e % VP] = v_ok[m] && st_in[m] ? vv : Real(0);
    }
#pragma unroll
    for (int m = 0; m < Tr::NQ_PER; ++m) {
      const int e = tid + m * NT;
      const Real kk = held(st_k[m]), qq = held(st_q[m]);
      const bool ok = q_ok[m] && st_qin[m];
      if (e < TC * 16) {
        sm.k[base + e / 16][e % 16] = ok ? kk : Real(0);
        sm.q[base + e / 16][e % 16] = ok ? qq : Real(0);
      }
    }
    if (tid < TC) {
      const Real ff = held(st_f);
      const Real fv = st_fin ? ff : Real(0);
      sm.fg[base + tid] = R2{fv, Real(1) - fv};
    }
  };
  // write back one chunk of readouts (staged in lane order); element e of the
  // chunk is (step e / VP, lane-order column e % VP)
  constexpr int NY_PER = (TC * VP + NT - 1) / NT;
  int64_t y_ofs[NY_PER];
  Real y_wr[NY_PER];
  int y_tt[NY_PER], y_c[NY_PER], y_g[NY_PER], y_r[NY_PER];
  bool y_ok[NY_PER];
#pragma unroll
  for (int k = 0; k < NY_PER; ++k) {
    const int e = tid + k * NT;
    const int tt = e / VP, jl = e % VP;
    y_tt[k] = tt < TC ? tt : 0;
    y_c[k] = jl >> 4;
    y_g[k] = (jl >> 2) & 3;
    y_r[k] = jl & 3;
    const int j = y_c[k] * 16 + acc_m<Real>(y_g[k], y_r[k]);
    y_ok[k] = tt < TC && j < V;
    y_ofs[k] = (tok0 + (int64_t)y_tt[k] * N) * V + (j < V ? j : 0);
    y_wr[k] = j < V ? wrp[(int64_t)n * V + j] : Real(0);
  }
  // readouts of chunk ch; cofs = ch TC N V (the chunk's token offset), stepped per chunk
  int64_t cofs = 0;
  auto flush = [&](int ch) {
    const int t0 = ch * TC;
    const int base = (ch & 1) * TC;
#pragma unroll
    for (int k = 0; k < NY_PER; ++k) {
      if (y_ok[k] && t0 + y_tt[k] < T32) {
        const int slot = base + y_tt[k];
        const R4* yq = sm.y[slot][y_c[k]][y_g[k]];
        const Real val = ((yq[0][y_r[k]] + yq[1][y_r[k]]) + yq[2][y_r[k]]) + yq[3][y_r[k]];
        if (nslab == 1) {
          const Real vv = sm.v[slot][y_c[k] * 16 + acc_m<Real>(y_g[k], y_r[k])];
          yout[y_ofs[k] + cofs] = val + y_wr[k] * vv;
        } else {
          ypart[slab * slab_stride + y_ofs[k] + cofs] = val;
        }
      }
    }
    cofs += TC * NV;
  };

  const int nchunks = (T32 + TC - 1) / TC;
  load_chunk(0);
  store_chunk(0);
  if (nchunks > 1) load_chunk(1);

  // ---- first exchange: the full slab of H_0 as the B operand.
  Real hb[NS];
#pragma unroll
  for (int p = 0; p < TPW; ++p) sm.xb[1][w * TPW + p][lane] = hown[p];
  unit_sync();
#pragma unroll
  for (int q0 = 0; q0 < VT; ++q0) {
    const R4 t4 = q0 < TPW ? hown[q0] : sm.xb[1][(q0 + TPW * w) % VT][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
  }

  R4* const ydump_me = &sm.ydump[tid];

  // Inputs of one step, read from the staging ring one step ahead of use so
  // their LDS latency is hidden behind the previous step's MFMA chain.
  struct StepIn {
    R4 v[TPW];    // v at this lane's columns 16 c + m(g, r) of this wave's tiles
    Real k;       // k_li
    R2 fg;        // (f, 1 - f)
    Real q;       // q_li
  };
  auto read_in = [&](int slot) {
    StepIn in;
#pragma unroll
    for (int p = 0; p < TPW; ++p) in.v[p] = cols4(&sm.v[slot][(w * TPW + p) * 16], g);
    in.k = sm.k[slot][li];
    in.fg = sm.fg[slot];
    in.q = sm.q[slot][li];
    return in;
  };

  // One step; P = parity of the step (static LDS offsets).  `nxt_slot` is the
  // ring slot of the following step, whose inputs are read at the start.
  auto step = [&](auto par, int slot, const StepIn& cur, StepIn& nxt, int nxt_slot) {
    constexpr int P = decltype(par)::value;
    nxt = read_in(nxt_slot);
    // the rank-1 write k v^T (scaled) starts the accumulators; then the own
    // tiles (operands in registers), then the tiles received through LDS
    const Real ks = kTanhScale<Real> * cur.k;
    R4 acc[TPW];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[p][r] = ks * cur.v[p][r];
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) {
#pragma unroll
      for (int p = 0; p < TPW; ++p) acc[p] = mfma_16x16x4(wa[p][s0], hb[s0], acc[p]);
    }
    // the accumulators stay in VGPRs (read by the VALU right away)
#pragma unroll
    for (int p = 0; p < TPW; ++p) pin_vec(acc[p]);
    // H = f H + (1 - f) tanh(A), with tanh(A) = 1 - 2 / (1 + e^{2A}):
    // H = (f H + (1 - f)) - 2 (1 - f) / (1 + e^{2A}).  f = 1 gives H exactly.
    const Real m2omf = Real(-2) * cur.fg[1];
    R4 rcv[TPW];
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rcv[p][r] = tanh_rc_scaled(acc[p][r]);
        hown[p][r] = fma_r(m2omf, rcv[p][r], fma_r(cur.fg[0], hown[p][r], cur.fg[1]));
      }
      if constexpr (Tr::NW > 1) sm.xb[P][w * TPW + p][lane] = hown[p];
    }
    if constexpr (RCS && FULL) {  // the step's rc for the backward (no recompute there)
#pragma unroll
      for (int p = 0; p < TPW; ++p) *(R4*)(rcp + col_of(p, 0)) = rcv[p];
      rcp += KV;
    } else if constexpr (RCS) {
      // non-temporal: rc is read back only by the backward, long after
      if (st_vec) {
        if (row_ok) {
#pragma unroll
          for (int p = 0; p < TPW; ++p)
            if (col_of(p, 0) < V) __builtin_nontemporal_store(rcv[p], (R4*)(rcp + col_of(p, 0)));
        }
      } else {
        write_rows(rcp, rcv);
      }
      rcp += KV;
    }
    // keep the exchange write ahead of the readout, so its latency overlaps it
    __builtin_amdgcn_sched_barrier(0);
    // readout y_t = H_t^T q_t over this slab's rows, while the write lands
    // (the reduction is volatile asm for fp32, so it also stays before the barrier)
    R4 ys[TPW];
#pragma unroll
    for (int p = 0; p < TPW; ++p) ys[p] = row16_partial4_x4(hown[p], cur.q);
    unit_sync();
    // the readout store goes after the barrier (its latency then overlaps the
    // own-tile MFMAs of the next step); the barrier ending the chunk's last
    // step is followed by one more before the write-back reads it
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      R4* dst = li < 4 ? &sm.y[slot][w * TPW + p][g][li] : ydump_me;
      *dst = ys[p];
    }
#pragma unroll
    for (int q0 = TPW; q0 < VT; ++q0) {
      const R4 t4 = sm.xb[P][(q0 + TPW * w) % VT][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
    }
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) hb[4 * p + r] = hown[p][r];
    // the exchange reads are issued before any MFMA of the next step
    __builtin_amdgcn_sched_barrier(0);
  };
  // A whole chunk, unrolled.  Chunk ch + 1 is staged after step TC - 3, so
  // the barrier of step TC - 2 orders it before step TC - 1 reads its first
  // slot.  Inputs alternate between two StepIn buffers by step parity.
  // Checkpoints are checked after every step (a countdown, on the scalar unit).
  StepIn ins[2];
  auto full_chunk = [&](int base, int ch) {
    const int nbase = base ^ TC;
    const int t0 = ch * TC;
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((step(std::integral_constant<int, I & 1>{}, base + I, ins[I & 1], ins[(I + 1) & 1],
             I + 1 < TC ? base + I + 1 : nbase),
        (I == TC - 3 ? store_chunk(ch + 1) : void()), ck_step(t0 + I)),
       ...);
    }(std::make_integer_sequence<int, TC>{});
  };

  ins[0] = read_in(0);

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * TC;
    const int base = (ch & 1) * TC;
    const bool last = ch + 1 == nchunks;
    if (!last) {
      full_chunk(base, ch);
    } else {
      // the last chunk, possibly partial
      const int tn = T32 - t0 < TC ? T32 - t0 : TC;
      for (int tt = 0; tt < tn; ++tt) {
        const int nslot = tt + 1 < TC ? base + tt + 1 : (base ^ TC);
        if ((tt & 1) == 0)
          step(std::integral_constant<int, 0>{}, base + tt, ins[0], ins[1], nslot);
        else
          step(std::integral_constant<int, 1>{}, base + tt, ins[1], ins[0], nslot);
        ck_step(t0 + tt);
      }
    }
    // ---- between chunks: write-back of this chunk, prefetch
    unit_sync();                                 // the chunk's last readout stores
    flush(ch);                                   // readouts of chunk ch are complete
    if (ch + 2 < nchunks) load_chunk(ch + 2);    // into registers; stored during chunk ch + 1
  }
  if (a.HT) write_state((Real*)a.HT + state_base);
}

// y = sum over slabs of the partial readouts + w_r (.) v   (elementwise, HBM-bound;
// 64-bit indices, for sizes beyond m2rnn_slab_sum_kernel's)
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
  static_assert(Tr::PACK * sizeof(FwdSmem<Real, VT, Tr::NW, Tr::RING>) <= 160 * 1024,
                "LDS budget");
  const int64_t units = a.B * a.N * a.nslab;
  const int64_t wgs = (units + Tr::PACK - 1) / Tr::PACK;
  // every tile full: K rows in whole slabs, V columns in whole tiles, fp32
  // state, and the rc, checkpoint and H_T arrays 16-byte aligned
  const bool full = sizeof(Real) == 4 && a.K % 16 == 0 && a.V == Tr::VP && a.st_vec;
  const dim3 grid((unsigned)wgs), block(Tr::NT * Tr::PACK);
  if constexpr (sizeof(Real) == 4) {
    if (full) {
      if (a.rc)  // also store every step's rc
        hipLaunchKernelGGL((m2rnn_fwd_kernel<InT, Real, VT, true, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((m2rnn_fwd_kernel<InT, Real, VT, false, true>), grid, block, 0, stream, a);
    }
  }
  if (!full) {
    if (a.rc)
      hipLaunchKernelGGL((m2rnn_fwd_kernel<InT, Real, VT, true, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((m2rnn_fwd_kernel<InT, Real, VT, false, false>), grid, block, 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nslab == 1) return err;
  const int64_t total = a.B * a.T * a.N * a.V;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (total < ((int64_t)1 << 31)) {
    hipLaunchKernelGGL((m2rnn_slab_sum_kernel<InT, Real>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, (int)(a.B * a.T * a.N), (int)a.N, (int)a.V, a.nslab, total,
                       (const Real*)a.ypart, (const InT*)a.v, (const Real*)a.w_r, (Real*)a.y,
                       slab_sum_vec<InT, Real>(a.V, a.ypart, a.v, a.w_r, a.y));
  } else {
    hipLaunchKernelGGL((m2rnn_fwd_reduce_kernel<InT, Real>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, total, a.N, a.V, a.nslab, (const Real*)a.ypart, (const InT*)a.v,
                       (const Real*)a.w_r, (Real*)a.y);
  }
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

hipError_t launch_fwd(const FwdArgs& a0, int in_dtype, int state_dtype, hipStream_t stream) {
  FwdArgs a = a0;
  a.st_vec = state_dtype == kF32 && (a.V & 3) == 0 && aligned16(a.ckpt) && aligned16(a.HT) &&
             aligned16(a.rc);
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
