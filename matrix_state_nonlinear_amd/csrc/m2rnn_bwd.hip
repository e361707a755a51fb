// Reverse-time M²RNN backward for gfx950.
//
// Implements the corrected BPTT chain rule of the M²RNN review (section 2.7),
// with the value-residual branch restored, and recomputes the forward states
// from checkpoints as the review's section 2.6 describes.  With u_t = dy_t and
// C_t the gradient arriving at the state H_t from later steps:
//   R_t = C_t + q_t u_t^T,  D_t = (1 - f_t) R_t (.) (1 - Z_t^2),
//   C_{t-1} = f_t R_t + D_t W^T,  dW += H_{t-1}^T D_t,
//   dq_t = H_t u_t,  dk_t = D_t v_t,  dv_t = D_t^T k_t + w_r (.) u_t,
//   df_t = <R_t, H_{t-1} - Z_t>.
// Token t here is 0-based: step t reads state S_t and writes S_{t+1}.
//
// Decomposition.  As in the forward, one workgroup per 16-row slab of one
// (b, n): rows are independent in the backward as well (W^T acts on columns),
// so only dv, df and dW need sums across slabs, done by fixed-order reduction
// kernels afterwards.
//
// Three wave roles per workgroup, one wave of each role on every SIMD, so the
// three MFMA streams of a step share each SIMD's matrix unit.  On gfx950 a
// SIMD does not run fp32 MFMA and VALU work at the same time, not even for
// different waves, so the roles do not buy overlap of VALU with MFMA: they
// give the SIMD three independent dependency chains per step, which hide each
// other's latencies (LDS round trips, dependent MFMA chains, the barrier).
//  * forward role: reruns the recurrence chunk by chunk (S steps per chunk,
//    chunks from last to first), each chunk from its stored start state, with
//    exactly the forward kernel's arithmetic.  Every step's state S_{t+1} and
//    rc_t = 1 / (1 + e^{2 A_t}) (tanh(A_t) = 1 - 2 rc_t) go into LDS rings;
//    it forms the per-wave sums of dq_t = S_{t+1} u_t, and it finishes dq and
//    dv (D^T k over the slab rows, by DPP) of the previous phase's steps.
//  * reverse role: walks the chunk recomputed in the previous period from its
//    last step to its first, one phase behind, carrying C through the MFMA
//    product (D W^T)^T = W D^T; it publishes D (plain and transposed) and the
//    lane partials of dk and df.  With one value tile it also reduces dv
//    itself, right after forming D (the forward role's phase is the longest
//    there).
//  * side role: accumulates dW += S_t^T D_t on MFMA one phase behind the
//    reverse role, finishes dk and df, and stages the next chunk's inputs and
//    start state from HBM into LDS.
// All roles finish one step per phase (one barrier per phase).  The rings hold
// 2 S entries; no ring entry, staging slot or buffer is read and written in
// the same phase (the schedule is replayed step by step on the host in the
// tests).
//
// MFMA layouts.  Recompute: A = W^T (registers), B = S^T, as in the forward.
// C-chain: A = W, B = D^T with the forward's contraction enumeration
// pi(s, g) = 16 (s / 4) + m(g, s % 4), so a wave's own D tiles feed the B
// operand from registers and the others come through LDS.  dW: output tile
// (l, j), A[l][i] = S_t[i][l], B[i][j] = D_t[i][j], contraction over the 16
// slab rows in four k-steps; B comes from the transposed D copy in one 16-byte
// read per tile.
//
// The first read of an MFMA result is kept in the basic block of the MFMA
// (the accumulators are pinned right after the chain): behind a branch, the
// compiler did not insert the wait states such a read needs.

#include <type_traits>
#include <utility>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

constexpr size_t kLdsBytes = 160 * 1024;

template <typename Real, int VT>
struct BwdShape {
  static constexpr int VP = 16 * VT;                       // padded value width
  static constexpr int NW = VT <= 4 ? VT : VT / 2;         // waves per role
  static constexpr int TPW = VT / NW;                      // 16-column tiles per wave
  static constexpr int NS = 4 * VT;                        // MFMAs per tile per step
  static constexpr int NT = 3 * 64 * NW;                   // threads (three roles)
  static constexpr int E = (32 + 2 * VP + 1 + 3) / 4 * 4;  // staged values per step
  static constexpr size_t kTileset = (size_t)VT * 64 * 4 * sizeof(Real);
  // the transposed D copy (16-byte dW operand reads) is kept for fp32; the
  // fp64 instantiations read the operands from the plain copy to fit in LDS,
  // and so does one value tile, where the reverse role (which would write the
  // copy with scattered 4-byte stores) has the longest phase
  static constexpr bool kXdt = sizeof(Real) == 4 && VT > 1;
};

constexpr int bwd_slots(int S) { return S >= 4 ? 3 : (S == 2 ? 4 : 5); }

// LDS of the backward for chunk length S: two rings of 2 S slab states, the
// D exchange (plain and transposed, double-buffered), two chunk-start
// buffers, the staging slots and the reduction partials.
template <typename Real, int VT>
constexpr size_t bwd_smem_bytes(int S) {
  using Sh = BwdShape<Real, VT>;
  return (size_t)(4 * S + (Sh::kXdt ? 6 : 4)) * Sh::kTileset +
         (size_t)bwd_slots(S) * S * Sh::E * sizeof(Real) +
         (size_t)(2 * 16 * 4 + 2 * 16 * 20 + 2 * 4 * Sh::NW + Sh::VP) * sizeof(Real) +
         (Sh::kXdt ? (size_t)2 * VT * 16 * 4 * sizeof(Real) : 0);
}

template <typename Real, int VT>
struct BwdTraits : BwdShape<Real, VT> {
  using Sh = BwdShape<Real, VT>;
  // the longest chunk of at most 4 steps (a power of two) whose LDS fits.
  // Longer chunks would fit for V <= 48 but take twice the ring space, so
  // fewer workgroups share a compute unit and large batches run in several
  // rounds (measured at V = 16 and 32 with 1024 units: 4 steps 22-28 % faster;
  // with a single round, within 3 % either way).
  static constexpr int S = bwd_smem_bytes<Real, VT>(4) <= kLdsBytes   ? 4
                           : bwd_smem_bytes<Real, VT>(2) <= kLdsBytes ? 2
                                                                      : 1;
  static constexpr int M = 2 * S;                    // ring length
  static constexpr int NSLOT = bwd_slots(S);         // staging slots (chunks)
  static constexpr int NX = 64 * Sh::NW;             // side-role threads
  static constexpr int NLD = (S * Sh::E + NX - 1) / NX;         // staged values per thread
  static constexpr int NCK = (16 * Sh::VP + NX - 1) / NX;       // start-state values per thread
};

// XT: tiles of the state exchange.  The interval-sweep variant holds every tile
// twice (positions p and p + VT) where LDS allows, so that a wave reads its
// rotated B operand tiles at one base address plus constant offsets.
template <typename Real, int VT, int XT = VT>
struct BwdSmem {
  using Tr = BwdTraits<Real, VT>;
  using R4 = typename Vec4<Real>::type;
  R4 hr[Tr::M][VT][64];            // states S_x at ring position x mod M
  R4 zr[Tr::M][VT][64];            // rc_t at ring position t mod M
  R4 xd[2][VT][64];                // D tiles in register layout, by phase parity
  // D transposed: [tile][column][4 (row % 4) + row / 4] (fp32 only); rows of
  // 20 so that both the scattered writes and the 16-byte reads of 8
  // consecutive lanes spread over the banks
  Real xdT[Tr::kXdt ? 2 : 1][VT][16][Tr::kXdt ? 20 : 1];
  R4 ck[2][XT][64];                // chunk start states in register layout, by chunk parity
                                   // (interval sweep: the exchanged states, by step parity)
  // staged inputs of a chunk, per step: k[16] q[16] v[VP] dy[VP] f (padded)
  Real st[Tr::NSLOT][Tr::S * Tr::E];
  Real rq[2][16][4];               // dq per-wave row sums [row][wave] (at most 4 waves)
  Real rk[2][16][20];              // dk lane partials [row][wave, lane group] (rows of 20)
  Real rf[2][4 * Tr::NW];          // df partials [wave, lane group]
  Real wr[Tr::VP];                 // w_r of the head (interval sweep: dv's value-residual term)
};

// the exchange of the interval sweep: doubled where it fits
template <typename Real, int VT>
constexpr int bwd_sweep_xt() {
  return sizeof(BwdSmem<Real, VT, 2 * VT>) <= kLdsBytes ? 2 * VT : VT;
}

int bwd_period(int state_dtype, int64_t V) {
  const bool f64 = state_dtype == kF64;
  switch (value_tiles(V)) {
    case 1: return f64 ? BwdTraits<double, 1>::S : BwdTraits<float, 1>::S;
    case 2: return f64 ? BwdTraits<double, 2>::S : BwdTraits<float, 2>::S;
    case 3: return f64 ? BwdTraits<double, 3>::S : BwdTraits<float, 3>::S;
    case 4: return f64 ? BwdTraits<double, 4>::S : BwdTraits<float, 4>::S;
    case 6: return f64 ? BwdTraits<double, 6>::S : BwdTraits<float, 6>::S;
    case 8: return f64 ? BwdTraits<double, 8>::S : BwdTraits<float, 8>::S;
    default: return 1;
  }
}

BwdWorkspace bwd_workspace_layout(int64_t B, int64_t T, int64_t N, int64_t NQ, int64_t K,
                                  int64_t V, int64_t C, int state_dtype, bool stored_rc) {
  BwdWorkspace L{};
  const int64_t ns = num_slabs(K);
  L.period = bwd_period(state_dtype, V);
  L.nch = (T + L.period - 1) / L.period;
  // The interval sweep pays at V > 112 (eight value tiles), where it replaces a
  // chunk-start pass that costs a second forward; at V <= 64 its ring traffic and
  // the forward role's extra work outweigh that pass (measured at V = 16, 64 and
  // 128).  One-step chunks (the fp64 state at V > 96) keep the pass as well.
  L.sweep = value_tiles(V) == kMaxValueTiles && L.period >= 2 && C > L.period &&
            C % L.period == 0 && C <= kMaxSweepInterval;
  L.subck_needed = (L.period % C) != 0 && !L.sweep;
  const int64_t rows = B * T;
  L.row_blocks = (rows + 255) / 256;
  size_t off = 0;
  auto take = [&](size_t elems) {
    const size_t at = off;
    off = align_up(off + elems, 64);
    return at;
  };
  L.subck = take(L.subck_needed ? (size_t)B * N * L.nch * K * V : 0);
  const size_t ring = L.sweep ? (size_t)B * N * ns * 2 * C * 16 * (16 * value_tiles(V)) : 0;
  L.ring_s = take(ring);
  L.ring_r = take(stored_rc ? 0 : ring);
  L.dv_part = take(ns > 1 ? (size_t)ns * B * T * N * V : 0);
  L.df_part = take((size_t)ns * B * T * N);
  L.dW_part = take((size_t)B * ns * N * V * V);
  L.col_part = take((size_t)L.row_blocks * N * (V + 2));
  L.dk_part = take(NQ < N ? (size_t)B * T * N * K : 0);
  L.dq_part = take(NQ < N ? (size_t)B * T * N * K : 0);
  L.total_elems = off;
  return L;
}


// RC: rebuild the states from the forward's rc.  FULL: every row of the slab
// and every column of the tiles exists and the state is fp32 (the launcher
// checks), so the per-step row and column guards and the scalar fallbacks of the
// rc loads and dv stores are compiled out.
template <typename InT, typename Real, int VT, bool RC, bool FULL, bool SW>
__global__ void __launch_bounds__((BwdTraits<Real, VT>::NT))
    m2rnn_bwd_kernel(BwdArgs a, BwdWorkspace L) {
  using Tr = BwdTraits<Real, VT>;
  using R4 = typename Vec4<Real>::type;
  constexpr int TPW = Tr::TPW, NS = Tr::NS, NW = Tr::NW, VP = Tr::VP;
  constexpr int S = Tr::S, M = Tr::M, NSLOT = Tr::NSLOT, E = Tr::E;
  constexpr int NX = Tr::NX, NLD = Tr::NLD, NCK = Tr::NCK;
  constexpr int OFF_Q = 16, OFF_V = 32, OFF_U = 32 + VP, OFF_F = 32 + 2 * VP;
  constexpr int XT = SW ? bwd_sweep_xt<Real, VT>() : VT;
  static_assert(sizeof(BwdSmem<Real, VT, XT>) <= kLdsBytes, "LDS budget");
  __shared__ BwdSmem<Real, VT, XT> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int role = w / NW;  // 0 forward, 1 reverse, 2 side
  const int wr = w - role * NW;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int nslab = a.nslab;
  const int slab = unit % nslab;
  const int bn = unit / nslab;
  const int64_t B = a.B, T = a.T, N = a.N, K = a.K, V = a.V;
  const int n = (int)(bn % N);
  const int b = (int)(bn / N);
  const int row = slab * 16 + li;
  const bool row_ok = row < K;
  // phase, step and chunk indices fit in 32 bits (T < 2^30)
  const int T32 = (int)T;
  const int nch = (T32 + S - 1) / S;
  const int jlast = nch * S + S + 1;  // last phase
  const int nper = jlast / S + 1;     // periods of S phases covering 0..jlast
  const int64_t tok0 = (int64_t)b * T * N + n;  // token (b, t, n) is tok0 + t N
  // q and k rows of (b, t): tokq0 + t NQ, head n / (N / NQ) of the NQ shared heads
  const int64_t NQ = a.NQ;
  const int64_t tokq0 = (int64_t)b * T * NQ + n / (int)(N / NQ);
  // dk and dq per value head: the outputs when NQ = N, else partials that
  // are summed over each group of N / NQ heads afterwards
  Real* const dk_base = NQ == N ? (Real*)a.dk : (Real*)a.ws + L.dk_part;
  Real* const dq_base = NQ == N ? (Real*)a.dq : (Real*)a.ws + L.dq_part;
  const int64_t state_base = ((int64_t)bn * K + row) * V;
  const Real* __restrict__ Wp = (const Real*)a.W;
  auto col_of = [&](int p, int r) { return (wr * TPW + p) * 16 + acc_m<Real>(g, r); };
  // the reverse role's step in phase j, and whether it takes one
  auto rstep = [&](int j) { return nch * S + S - j; };
  auto ractive = [&](int j) { return j >= S + 1 && j <= nch * S + S; };
  // With one value tile the reverse role reduces dv_t = D_t^T k_t itself, right
  // after it forms D_t (its phase is the shortest there); otherwise the forward
  // role does it one phase later.
  constexpr bool kDvRev = VT == 1 && !SW;

  if (role == 0) {
    if constexpr (SW) {
    // ======================================================= forward role, interval sweep
    // Checkpoint intervals of C steps (C a multiple of S) are swept forward in time
    // once, one interval ahead of the reverse role: from the interval's checkpoint,
    // the recurrence (MFMA, or the interpolation from the stored rc) produces every
    // S_{x+1} (and rc_x), which this lane stores at its own positions of the unit's
    // ring (two interval slots).  The chunk the reverse role takes next is filled
    // into the LDS rings from there, so no chunk start is ever needed.  Each ring
    // element is written and read back by the same lane.  The first C / S periods
    // (one more with one-step chunks) only sweep (the last interval); after them
    // the sweep runs C / S chunks ahead of the fill, so it finishes each interval before the fill reaches it and
    // starts interval i - 2 (the same slot as i) only after the fill has left i.
    const int Ci = (int)a.C;
    const int CS = Ci / S;                      // chunks per interval
    const int J = (T32 + Ci - 1) / Ci;          // intervals (= checkpoints)
    const int n_last = nch - (J - 1) * CS;      // chunks of the last interval
    // sweep-only periods; one more with one-step chunks, where the fill loads the
    // next chunk's first step in the phase that would sweep it
    const int P0 = CS + (S == 1 ? 1 : 0);
    const int64_t KV = K * V;
    const int64_t n_ckpt = J;
    // W^T as the A operand, rotated and scaled exactly as in the forward kernel
    Real wop[RC ? 1 : TPW][RC ? 1 : NS];
    if constexpr (!RC) {
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        const int col = (wr * TPW + p) * 16 + li;
#pragma unroll
        for (int s0 = 0; s0 < NS; ++s0) {
          const int s = (s0 + 4 * TPW * wr) % NS;
          const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
          wop[p][s0] = Wp[((int64_t)n * V + (l < V ? l : 0)) * V + (col < V ? col : 0)];
        }
      }
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        const int col = (wr * TPW + p) * 16 + li;
#pragma unroll
        for (int s0 = 0; s0 < NS; s0 += 4) pin_values(wop[p][s0], wop[p][s0 + 1], wop[p][s0 + 2], wop[p][s0 + 3]);
#pragma unroll
        for (int s0 = 0; s0 < NS; ++s0) {
          const int s = (s0 + 4 * TPW * wr) % NS;
          const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
          wop[p][s0] = (col < V && l < V) ? kTanhScale<Real> * wop[p][s0] : Real(0);
        }
#pragma unroll
        for (int s0 = 0; s0 < NS; s0 += 4) pin_values(wop[p][s0], wop[p][s0 + 1], wop[p][s0 + 2], wop[p][s0 + 3]);
      }
    }
    // w_r of the head in LDS (read by dv's value-residual term when the slab is the
    // whole head), so that it holds no registers through the step loop
    for (int c = wr * 64 + lane; c < VP; c += NW * 64)
      sm.wr[c] = c < V ? ((const Real*)a.w_r)[(int64_t)n * V + c] : Real(0);
    const bool dv_vec = sizeof(Real) == 4 && (FULL || a.dv_vec);
    Real* const dq_row = dq_base + tok0 * K + row;
    Real* const dv_tok = nslab == 1 ? (Real*)a.dv + tok0 * V
                                    : (Real*)a.ws + L.dv_part + ((int64_t)slab * B * T * N + tok0) * V;
    const int64_t NK = N * K, NV = N * V;
    bool colv[TPW][4];  // this lane's columns exist
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) colv[p][r] = FULL || (row_ok && col_of(p, r) < V);

    // the unit's ring, in R4 units: [slot][position][tile][lane]; step t of
    // interval i = t / C sits in slot i & 1 at position t - i C.  Both walks over
    // it (the sweep and the fill) keep their interval and position in counters,
    // so no step index is ever divided
    const size_t ring_unit = (size_t)unit * 2 * Ci * VT * 64;
    R4* const rs = (R4*)a.ring_s + ring_unit + wr * TPW * 64 + lane;
    R4* const rr = RC ? nullptr : (R4*)a.ring_r + ring_unit + wr * TPW * 64 + lane;
    auto rix = [&](int i, int pos) __attribute__((always_inline)) -> size_t {
      return ((size_t)((i & 1) * Ci + pos) * VT) * 64;
    };

    // ---- sweep inputs of step x, loaded one step ahead (clamped to 0..T - 1;
    // steps past T have f = 1, which keeps the state exactly)
    struct SwIn {
      InT k;
      InT v[TPW][4];
      Real f;          // gate of the step (lane-dependent address, read from lane 0)
      R4 rc[TPW];      // stored rc (RC only)
    };
    const InT* __restrict__ kp = (const InT*)a.k;
    const InT* __restrict__ vp = (const InT*)a.v;
    const Real* __restrict__ fpp = (const Real*)a.f;
    const Real* rc_lane = RC ? (const Real*)a.rc + ((int64_t)bn * T * K + (row_ok ? row : 0)) * V
                             : nullptr;
    const bool rc_vec = sizeof(Real) == 4 && (FULL || a.rc_vec);
    auto load_sw = [&](int x, SwIn& in) __attribute__((always_inline)) {
      const int xc = x < 0 ? 0 : (x < T32 ? x : T32 - 1);
      // gates of steps xc and xc + 1 in alternate lanes: a lane-dependent address
      int xf = xc + (lane & 1);
      if (xf > T32 - 1) xf = T32 - 1;
      in.f = fpp[tok0 + (int64_t)xf * N];
      if constexpr (RC) {
        const Real* src = rc_lane + (int64_t)xc * KV;
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          if (rc_vec) {
            const int c0 = col_of(p, 0);
            in.rc[p] = *(const R4*)(src + (FULL || c0 < V ? c0 : 0));
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int col = col_of(p, r);
              in.rc[p][r] = src[col < V ? col : 0];
            }
          }
        }
      } else {
        in.k = kp[(tokq0 + (int64_t)xc * NQ) * K + (row_ok ? row : 0)];
        const InT* vsrc = vp + (tok0 + (int64_t)xc * N) * V;
#pragma unroll
        for (int p = 0; p < TPW; ++p)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int col = col_of(p, r);
            in.v[p][r] = vsrc[col < V ? col : 0];
          }
      }
    };
    // a raw input converted in a register (kept there before any select)
    auto held = [&](auto x) __attribute__((always_inline)) -> Real {
      Real y = (Real)widen(x);
      asm volatile("" : "+v"(y));
      return y;
    };

    // ---- sweep state: own tiles hs (row `row`, columns col_of(p, r)), published
    // after every step through the exchange buffer, where each tile sits twice
    // (p and p + VT): a wave reads its B operand there in its rotated order
    // (own tiles first, as in the forward kernel) at one base address plus
    // constant offsets.  An interval starts from its checkpoint: its own tiles are
    // loaded after the previous interval's last step and published in place of
    // that step's state
    R4 hs[TPW], ckn[TPW];
    auto load_ck = [&](int i) __attribute__((always_inline)) {
      // the checkpoint H_{iC}, own tiles, from clamped addresses (masked on use)
      const Real* ck = (const Real*)a.ckpt + (((int64_t)bn * n_ckpt + i) * K + (row_ok ? row : 0)) * V;
#pragma unroll
      for (int p = 0; p < TPW; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = col_of(p, r);
          ckn[p][r] = ck[col < V ? col : 0];
        }
    };
    auto take_ck = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        R4 c = ckn[p];
        pin_vec(c);
#pragma unroll
        for (int r = 0; r < 4; ++r) hs[p][r] = colv[p][r] ? c[r] : Real(0);
      }
    };
    // The sweep's order: the intervals from the last to the first, each one's
    // chunks forward in time.  Cursor: interval s_i, the first step of the current
    // chunk within it (s_pos), the steps of the interval (s_len; the last one may
    // be shorter) and the chunks left.
    int s_i = J - 1, s_pos = 0, s_len = n_last * S, s_left = nch;
    int s_next = 0;  // the sweep's next step (whose inputs load_sw takes next)
    SwIn swc;  // the sweep step's inputs (loaded during the previous step)
    auto publish = [&](int par) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        sm.ck[par][wr * TPW + p][lane] = hs[p];
        if constexpr (XT == 2 * VT) sm.ck[par][wr * TPW + p + VT][lane] = hs[p];
      }
    };
    // one sweep step x at ring index ix (phase parity par); nck: the interval
    // that the next step starts, or -1.  When recomputing, the inputs of the next
    // step are loaded at the end of the phase, after every other memory access
    // of the role, so that no wait in between (a spill reload among them) has to
    // include them; the stored rc is loaded as soon as it is consumed.
    auto sweep_step = [&](int par, int x, size_t ix, int nck) __attribute__((always_inline)) {
      const Real f = x < T32 ? lane_value_r(swc.f, 0) : Real(1);
      const Real omf = Real(1) - f;
      const Real m2omf = Real(-2) * omf;
      R4 rcv[TPW];
      if constexpr (RC) {
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          R4 rc = swc.rc[p];
          pin_vec(rc);
#pragma unroll
          for (int r = 0; r < 4; ++r) rc[r] = colv[p][r] ? rc[r] : Real(0.5);
          rcv[p] = rc;
        }
        load_sw(s_next, swc);  // consumed: the next step's rc, a phase ahead
      } else {
        // the scaled rank-1 write k v^T starts the accumulators, as in the forward kernel
        const Real kk = held(swc.k);
        const Real ks = kTanhScale<Real> * (row_ok ? kk : Real(0));
        R4 acc[TPW];
#pragma unroll
        for (int p = 0; p < TPW; ++p)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const Real vv = held(swc.v[p][r]);
            acc[p][r] = ks * (col_of(p, r) < V ? vv : Real(0));
          }
        // H W over the slab, the tiles in the forward kernel's order (own first)
        // from the previous step's exchange, one 16-byte LDS read per tile
        const R4* const xb = &sm.ck[par ^ 1][TPW * wr][lane];
#pragma unroll
        for (int q0 = 0; q0 < VT; ++q0) {
          const R4 t4 = XT == 2 * VT ? xb[q0 * 64] : sm.ck[par ^ 1][(q0 + TPW * wr) % VT][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int p = 0; p < TPW; ++p) acc[p] = mfma_16x16x4(wop[p][4 * q0 + r], t4[r], acc[p]);
        }
#pragma unroll
        for (int p = 0; p < TPW; ++p) pin_vec(acc[p]);
#pragma unroll
        for (int p = 0; p < TPW; ++p)
#pragma unroll
          for (int r = 0; r < 4; ++r) rcv[p][r] = tanh_rc_scaled(acc[p][r]);
      }
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
#pragma unroll
        for (int r = 0; r < 4; ++r) hs[p][r] = fma_r(m2omf, rcv[p][r], fma_r(f, hs[p][r], omf));
        if constexpr (!RC) rr[ix + p * 64] = rcv[p];
        rs[ix + p * 64] = hs[p];
      }
      // the next step starts an interval: its state is that interval's checkpoint
      if (nck >= 0) {  // (once per interval: not prefetched, which would hold registers)
        load_ck(nck);
        take_ck();
      }
      if constexpr (!RC) publish(par);
    };

    // ---- fill of the LDS rings for the chunk the reverse role takes next:
    // S_{t+1} and rc_t of step t, loaded one phase ahead
    R4 fS[TPW], fR[TPW];
    auto load_fill = [&](int t, size_t ix) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < TPW; ++p) fS[p] = rs[ix + p * 64];
      if constexpr (RC) {
        const Real* src = rc_lane + (int64_t)(t < 0 ? 0 : (t < T32 ? t : T32 - 1)) * KV;
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          if (rc_vec) {
            const int c0 = col_of(p, 0);
            fR[p] = *(const R4*)(src + (FULL || c0 < V ? c0 : 0));
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int col = col_of(p, r);
              fR[p][r] = src[col < V ? col : 0];
            }
          }
        }
      } else {
#pragma unroll
        for (int p = 0; p < TPW; ++p) fR[p] = rr[ix + p * 64];
      }
    };

    // the sweep's first step: the last interval, from its checkpoint (published for
    // the first step's B operand as the previous step's state would be)
    load_sw(s_i * Ci, swc);
    load_ck(J - 1);
    take_ck();
    if constexpr (!RC) publish(1);

    __syncthreads();  // prologue staging by the side role

    auto sweep_phase = [&](int I, int jpar) __attribute__((always_inline)) {
      // step I of the cursor's chunk (if any chunk is left); the next step is the
      // following one in time, except after an interval's last step, where the
      // sweep goes on from the start of the interval before it
      if (s_left <= 0) return;
      const int x = s_i * Ci + s_pos + I;
      int nx = x + 1, nck = -1;
      const bool last = I + 1 == S && s_pos + S == s_len;
      if (last) {
        nck = s_i - 1;
        nx = nck >= 0 ? nck * Ci : 0;
      }
      s_next = nx;
      sweep_step(jpar, x, rix(s_i, s_pos + I), nck);
      if (I + 1 == S) {  // the chunk is done: advance the cursor
        --s_left;
        if (last) {
          --s_i;
          s_pos = 0;
          s_len = Ci;
        } else {
          s_pos += S;
        }
      }
    };
    // prologue: the last interval's sweep (and the following chunks up to P0)
    for (int kt = 0; kt < P0; ++kt) {
      for (int I = 0; I < S; ++I) {
        sweep_phase(I, (kt * S + I) & 1);
        if constexpr (!RC) load_sw(s_next, swc);
        __syncthreads();
      }
    }
    // Fill cursor: the interval f_i of the chunk filled in the period and that
    // chunk's first step within it (f_pos); the fill walks the chunks backward
    int f_i = J - 1, f_pos = (n_last - 1) * S;
    if (nch > 0) load_fill((nch - 1) * S, rix(f_i, f_pos));

    auto phase = [&](auto Ic, int k, int cF, bool rec, int slot, int hbase, int slotA, int slotB,
                     int slotC) {
      constexpr int I = decltype(Ic)::value;
      const int j = k * S + I;
      const int jp = j & 1;
      auto fill = [&]() __attribute__((always_inline)) {
        if (!rec) return;
        // the step t = cF S + I of the chunk: S_{t+1} and rc_t from the ring
        const Real* stp = &sm.st[slot][I * E];
        R4 s1[TPW], r1[TPW];
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          s1[p] = fS[p];
          r1[p] = fR[p];
          pin_vec(s1[p]);
          pin_vec(r1[p]);
          // padding rows and columns take rc = 1/2, as the recomputation gives them
#pragma unroll
          for (int r = 0; r < 4; ++r) r1[p][r] = colv[p][r] ? r1[p][r] : Real(0.5);
        }
        Real dqp = 0;
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          sm.hr[(hbase + I + 1) & (M - 1)][wr * TPW + p][lane] = s1[p];
          sm.zr[hbase + I][wr * TPW + p][lane] = r1[p];
          const R4 u = cols4(stp + OFF_U + (wr * TPW + p) * 16, g);
#pragma unroll
          for (int r = 0; r < 4; ++r) dqp = fma_r(s1[p][r], u[r], dqp);
        }
        dqp = cross_row_sum(dqp);
        if (g == 0) sm.rq[jp][li][wr] = dqp;
      };
      // the sweep, C / S chunks ahead of the fill.  Recomputing, the sweep goes
      // after the fill, from the stored rc before it (measured at V = 128: 6 % and
      // 11 % faster than the other order)
      if constexpr (RC) {
        sweep_phase(I, (P0 * S + j) & 1);
        fill();
      } else {
        fill();
        sweep_phase(I, (P0 * S + j) & 1);
      }
      // dq of the previous phase's step: the per-wave sums, added by wave 0
      if (wr == 0 && g == 0 && (FULL || row_ok) && j >= 1 && j <= nch * S) {
        const int tf = I > 0 ? cF * S + I - 1 : cF * S + 2 * S - 1;
        if (tf < T32) {
          Real sq = 0;
#pragma unroll
          for (int i = 0; i < NW; ++i) sq += sm.rq[jp ^ 1][li][i];
          dq_row[(int64_t)tf * NK] = sq;
        }
      }
      // dv of the reverse role's step of phase j - 1 (as in the recomputing role)
      if (ractive(j - 1)) {
        const int tp = (cF + 2) * S - I + 1;
        if (tp < T32) {
          constexpr int tq = (1 - I + S) % S;
          const Real* stq = &sm.st[S == 1 ? slotC : (I <= 1 ? slotB : slotA)][tq * E];
          const Real kq = stq[li];
          Real* dvp = dv_tok + (int64_t)tp * NV;
#pragma unroll
          for (int p = 0; p < TPW; ++p) {
            const R4 Dt = sm.xd[jp ^ 1][wr * TPW + p][lane];
            R4 sv = row16_sum_x4(Dt, kq);
            if (li == 0) {
              if (nslab == 1) {
                const R4 u = cols4(stq + OFF_U + (wr * TPW + p) * 16, g);
                const R4 w4 = cols4(&sm.wr[(wr * TPW + p) * 16], g);
#pragma unroll
                for (int r = 0; r < 4; ++r) sv[r] = fma_r(w4[r], u[r], sv[r]);
              }
              const int col0 = col_of(p, 0);
              if (dv_vec) {
                if (FULL || col0 < V) *(R4*)(dvp + col0) = sv;
              } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (col_of(p, r) < V) dvp[col_of(p, r)] = sv[r];
              }
            }
          }
        }
      }
      // S_0 (the initial state) for the reverse role's last step
      if (j == nch * S) {
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          R4 h0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int col = col_of(p, r);
            h0[r] = (a.H0 && row_ok && col < V) ? ((const Real*)a.H0)[state_base + col] : Real(0);
          }
          sm.hr[0][wr * TPW + p][lane] = h0;
        }
      }
      // the next phase's reads from memory, last and unconditionally (a harmless
      // in-ring address when there is nothing to fill): the fill's next step, then
      // the sweep's next inputs (when recomputing; the stored rc is loaded by the
      // sweep step itself)
      if constexpr (I + 1 < S) {
        load_fill(cF * S + I + 1, rix(f_i, f_pos + I + 1));
      } else {
        // the first step of the chunk before: the same interval, or the end of
        // the one before it
        load_fill((cF - 1) * S, f_pos > 0 ? rix(f_i, f_pos - S) : rix(f_i - 1, Ci - S));
      }
      if constexpr (!RC) load_sw(s_next, swc);
    };

    for (int k = 0; k < nper; ++k) {
      const int cF = nch - 1 - k;  // chunk filled in this period
      const bool rec = cF >= 0;
      const int slot = rec ? cF % NSLOT : 0;
      const int hbase = rec ? (cF & 1) * S : 0;  // ring position of S_{cF S}
      const int slotA = cF + 1 >= 0 ? (cF + 1) % NSLOT : 0;
      const int slotB = cF + 2 >= 0 ? (cF + 2) % NSLOT : 0;
      const int slotC = cF + 3 >= 0 ? (cF + 3) % NSLOT : 0;
      [&]<int... I>(std::integer_sequence<int, I...>) {
        ((phase(std::integral_constant<int, I>{}, k, cF, rec, slot, hbase, slotA, slotB, slotC),
          __syncthreads()),
         ...);
      }(std::make_integer_sequence<int, S>{});
      if (rec) {  // the fill moves to the chunk before
        if (f_pos > 0) {
          f_pos -= S;
        } else {
          --f_i;
          f_pos = Ci - S;
        }
      }
    }
    } else {
    // ================================================================ forward role
    // W^T as the A operand, rotated so this wave's own tiles come first and
    // scaled by 2 / ln 2, exactly as in the forward kernel
    Real wop[TPW][NS];
    if constexpr (!RC) {
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      const int col = (wr * TPW + p) * 16 + li;
#pragma unroll
      for (int s0 = 0; s0 < NS; ++s0) {
        const int s = (s0 + 4 * TPW * wr) % NS;
        const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
        wop[p][s0] = Wp[((int64_t)n * V + (l < V ? l : 0)) * V + (col < V ? col : 0)];
      }
    }
    // wait for these loads before the loop (a wait left for inside the loop
    // would also wait for the stores in flight there), all together, then
    // mask the padding (a guarded load would wait for itself at once)
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      const int col = (wr * TPW + p) * 16 + li;
#pragma unroll
      for (int s0 = 0; s0 < NS; s0 += 4) pin_values(wop[p][s0], wop[p][s0 + 1], wop[p][s0 + 2], wop[p][s0 + 3]);
#pragma unroll
      for (int s0 = 0; s0 < NS; ++s0) {
        const int s = (s0 + 4 * TPW * wr) % NS;
        const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
        wop[p][s0] = (col < V && l < V) ? kTanhScale<Real> * wop[p][s0] : Real(0);
      }
      // the final operands are held in registers (not recomputed in the loop)
#pragma unroll
      for (int s0 = 0; s0 < NS; s0 += 4) pin_values(wop[p][s0], wop[p][s0 + 1], wop[p][s0 + 2], wop[p][s0 + 3]);
    }
    }
    R4 h[TPW];
    Real hb[NS];
#pragma unroll
    for (int p = 0; p < TPW; ++p) h[p] = R4{0, 0, 0, 0};
    // w_r of this lane's dv columns (completed here, see above); where a lane's
    // four columns are consecutive (fp32) dv is written with one 16-byte store
    Real wrc[TPW][4];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = col_of(p, r);
        wrc[p][r] = col < V ? ((const Real*)a.w_r)[(int64_t)n * V + col] : Real(0);
      }
#pragma unroll
    for (int p = 0; p < TPW; ++p) pin_values(wrc[p][0], wrc[p][1], wrc[p][2], wrc[p][3]);
    const bool dv_vec = sizeof(Real) == 4 && (FULL || a.dv_vec);
    // output pointers at token (b, t = 0, n); step t adds t N rows
    Real* const dq_row = dq_base + tok0 * K + row;
    Real* const dv_tok = nslab == 1 ? (Real*)a.dv + tok0 * V
                                    : (Real*)a.ws + L.dv_part + ((int64_t)slab * B * T * N + tok0) * V;
    const int64_t NK = N * K, NV = N * V;
    // Stored rc (RC): this lane's values (row `row`, its tiles' columns) of the
    // step one phase ahead; steps past T read step T - 1 (f = 1 there, so rc
    // does not matter)
    R4 rcn[TPW];
    const Real* rc_lane = nullptr;
    const int64_t KV = K * V;
    const bool rc_vec = sizeof(Real) == 4 && (FULL || a.rc_vec);
    auto load_rc = [&](int t) {
      const int tt = t < T32 ? t : T32 - 1;
      const Real* src = rc_lane + (int64_t)tt * KV;
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        if (rc_vec) {
          const int c0 = col_of(p, 0);
          rcn[p] = *(const R4*)(src + (FULL || c0 < V ? c0 : 0));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int col = col_of(p, r);
            rcn[p][r] = src[col < V ? col : 0];
          }
        }
      }
    };
    if constexpr (RC) {
      rc_lane = (const Real*)a.rc + ((int64_t)bn * T * K + (row_ok ? row : 0)) * V;
      if (nch > 0) load_rc((nch - 1) * S);
    }

    __syncthreads();  // prologue staging by the side role

    auto phase = [&](auto Ic, int k, int cF, bool rec, int slot, int hbase, int slotA, int slotB,
                     int slotC) {
      constexpr int I = decltype(Ic)::value;
      const int j = k * S + I;
      const int jp = j & 1;
      if (RC && rec) {
        // the step t = cF S + I from state S_t, with the forward's stored rc:
        // S_{t+1} = (f S_t + (1 - f)) - 2 (1 - f) rc, as in the forward kernel
        const Real* stp = &sm.st[slot][I * E];
        R4 rcc[TPW];
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          rcc[p] = rcn[p];
          pin_vec(rcc[p]);
        }
        if (I + 1 < S || cF >= 1) load_rc(I + 1 < S ? cF * S + I + 1 : (cF - 1) * S);
        if constexpr (I == 0) {
          const int cb = (int)(cF & 1);
#pragma unroll
          for (int p = 0; p < TPW; ++p) h[p] = sm.ck[cb][wr * TPW + p][lane];
        }
        const Real f = stp[OFF_F];
        const Real omf = Real(1) - f;
        const Real m2omf = Real(-2) * omf;
        Real dqp = 0;
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          R4 rc;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // padding rows and columns keep S = 0: rc = 1/2 there, as recomputed
            rc[r] = (FULL || (row_ok && col_of(p, r) < V)) ? rcc[p][r] : Real(0.5);
            h[p][r] = fma_r(m2omf, rc[r], fma_r(f, h[p][r], omf));
          }
          sm.hr[(hbase + I + 1) & (M - 1)][wr * TPW + p][lane] = h[p];
          sm.zr[hbase + I][wr * TPW + p][lane] = rc;
          const R4 u = cols4(stp + OFF_U + (wr * TPW + p) * 16, g);
#pragma unroll
          for (int r = 0; r < 4; ++r) dqp = fma_r(h[p][r], u[r], dqp);
        }
        dqp = cross_row_sum(dqp);
        if (g == 0) sm.rq[jp][li][wr] = dqp;
      } else if (rec) {
        // the step t = cF S + I from state S_t
        const Real* stp = &sm.st[slot][I * E];
        if constexpr (I == 0) {
          const int cb = (int)(cF & 1);
#pragma unroll
          for (int q0 = 0; q0 < VT; ++q0) {
            const R4 t4 = sm.ck[cb][(q0 + TPW * wr) % VT][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
          }
#pragma unroll
          for (int p = 0; p < TPW; ++p)
#pragma unroll
            for (int r = 0; r < 4; ++r) h[p][r] = hb[4 * p + r];
        } else {
#pragma unroll
          for (int q0 = TPW; q0 < VT; ++q0) {
            const R4 t4 = sm.hr[hbase + I][(q0 + TPW * wr) % VT][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
          }
#pragma unroll
          for (int p = 0; p < TPW; ++p)
#pragma unroll
            for (int r = 0; r < 4; ++r) hb[4 * p + r] = h[p][r];
        }
        const Real f = stp[OFF_F];
        const Real omf = Real(1) - f;
        // the scaled rank-1 write k v^T starts the accumulators, as in the forward
        const Real ks = kTanhScale<Real> * stp[li];
        R4 acc[TPW];
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          const R4 vv = cols4(stp + OFF_V + (wr * TPW + p) * 16, g);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[p][r] = ks * vv[r];
        }
#pragma unroll
        for (int s0 = 0; s0 < NS; ++s0)
#pragma unroll
          for (int p = 0; p < TPW; ++p) acc[p] = mfma_16x16x4(wop[p][s0], hb[s0], acc[p]);
#pragma unroll
        for (int p = 0; p < TPW; ++p) pin_vec(acc[p]);
        const Real m2omf = Real(-2) * omf;
        Real dqp = 0;
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          R4 rc;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            rc[r] = tanh_rc_scaled(acc[p][r]);
            h[p][r] = fma_r(m2omf, rc[r], fma_r(f, h[p][r], omf));
          }
          sm.hr[(hbase + I + 1) & (M - 1)][wr * TPW + p][lane] = h[p];
          sm.zr[hbase + I][wr * TPW + p][lane] = rc;
          const R4 u = cols4(stp + OFF_U + (wr * TPW + p) * 16, g);
#pragma unroll
          for (int r = 0; r < 4; ++r) dqp = fma_r(h[p][r], u[r], dqp);
        }
        // this wave's columns of dq_t, summed over the four lane groups
        dqp = cross_row_sum(dqp);
        if (g == 0) sm.rq[jp][li][wr] = dqp;
      }
      // dq of the previous phase's step: the per-wave sums, added by wave 0
      // (by the side role when the reverse role reduces dv: with no store here
      // the role's only global accesses are its rc loads, and a wait for one
      // of them need not wait for a store issued after it)
      if (!kDvRev && wr == 0 && g == 0 && (FULL || row_ok) && j >= 1 && j <= nch * S) {
        const int tf = I > 0 ? cF * S + I - 1 : cF * S + 2 * S - 1;
        if (tf < T32) {
          Real sq = 0;
#pragma unroll
          for (int i = 0; i < NW; ++i) sq += sm.rq[jp ^ 1][li][i];
          dq_row[(int64_t)tf * NK] = sq;
        }
      }
      // dv_t' = D^T k over this slab's rows (+ w_r (.) u when the slab is the
      // whole head) for the reverse role's step t' = (cF + 2) S - I + 1 of
      // phase j - 1: this wave's D tiles, reduced over the 16 rows with DPP
      if (!kDvRev && ractive(j - 1)) {
        const int tp = (cF + 2) * S - I + 1;
        if (tp < T32) {
          constexpr int tq = (1 - I + S) % S;
          const Real* stq = &sm.st[S == 1 ? slotC : (I <= 1 ? slotB : slotA)][tq * E];
          const Real kq = stq[li];
          Real* dvp = dv_tok + (int64_t)tp * NV;
#pragma unroll
          for (int p = 0; p < TPW; ++p) {
            const R4 Dt = sm.xd[jp ^ 1][wr * TPW + p][lane];
            R4 sv = row16_sum_x4(Dt, kq);
            if (li == 0) {
              if (nslab == 1) {
                const R4 u = cols4(stq + OFF_U + (wr * TPW + p) * 16, g);
#pragma unroll
                for (int r = 0; r < 4; ++r) sv[r] = fma_r(wrc[p][r], u[r], sv[r]);
              }
              const int col0 = col_of(p, 0);
              if (dv_vec) {
                if (FULL || col0 < V) *(R4*)(dvp + col0) = sv;
              } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (col_of(p, r) < V) dvp[col_of(p, r)] = sv[r];
              }
            }
          }
        }
      }
      // S_0 (the initial state) for the reverse role's last step
      if (j == nch * S) {
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          R4 h0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int col = col_of(p, r);
            h0[r] = (a.H0 && row_ok && col < V) ? ((const Real*)a.H0)[state_base + col] : Real(0);
          }
          sm.hr[0][wr * TPW + p][lane] = h0;
        }
      }
    };

    for (int k = 0; k < nper; ++k) {
      const int cF = nch - 1 - k;  // chunk recomputed in this period
      const bool rec = cF >= 0;
      const int slot = rec ? cF % NSLOT : 0;
      const int hbase = rec ? (cF & 1) * S : 0;  // ring position of S_{cF S}
      const int slotA = cF + 1 >= 0 ? (cF + 1) % NSLOT : 0;
      const int slotB = cF + 2 >= 0 ? (cF + 2) % NSLOT : 0;
      const int slotC = cF + 3 >= 0 ? (cF + 3) % NSLOT : 0;
      [&]<int... I>(std::integer_sequence<int, I...>) {
        ((phase(std::integral_constant<int, I>{}, k, cF, rec, slot, hbase, slotA, slotB, slotC),
          __syncthreads()),
         ...);
      }(std::make_integer_sequence<int, S>{});
    }
    }  // SW
  } else if (role == 1) {
    // ================================================================ reverse role
    // W as the A operand of (D W^T)^T = W D^T, rotated like the forward role's
    Real wop[TPW][NS];
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      const int col = (wr * TPW + p) * 16 + li;
#pragma unroll
      for (int s0 = 0; s0 < NS; ++s0) {
        const int s = (s0 + 4 * TPW * wr) % NS;
        const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
        wop[p][s0] = Wp[((int64_t)n * V + (col < V ? col : 0)) * V + (l < V ? l : 0)];
      }
    }
    R4 fR[TPW], Dp[TPW], rcn[TPW];
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = col_of(p, r);
        fR[p][r] = (a.dHT && row_ok && col < V) ? ((const Real*)a.dHT)[state_base + col] : Real(0);
      }
      Dp[p] = R4{0, 0, 0, 0};
      rcn[p] = R4{0, 0, 0, 0};
    }
    // complete the loads made before the loop here (see the forward role),
    // then mask W's padding
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int s0 = 0; s0 < NS; s0 += 4) pin_values(wop[p][s0], wop[p][s0 + 1], wop[p][s0 + 2], wop[p][s0 + 3]);
      pin_vec(fR[p]);
      const int col = (wr * TPW + p) * 16 + li;
#pragma unroll
      for (int s0 = 0; s0 < NS; ++s0) {
        const int s = (s0 + 4 * TPW * wr) % NS;
        const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
        wop[p][s0] = (col < V && l < V) ? wop[p][s0] : Real(0);
      }
#pragma unroll
      for (int s0 = 0; s0 < NS; s0 += 4) pin_values(wop[p][s0], wop[p][s0 + 1], wop[p][s0 + 2], wop[p][s0 + 3]);
    }
    // transposed D: element (row li, column c) of a tile at [c][4 (li % 4) + li / 4]
    const int trow = 4 * (li & 3) + (li >> 2);
    // dv (kDvRev): w_r of this lane's columns, output row of token (b, t = 0, n)
    Real wrv[TPW][4];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = col_of(p, r);
        wrv[p][r] = (kDvRev && col < V) ? ((const Real*)a.w_r)[(int64_t)n * V + col] : Real(0);
      }
#pragma unroll
    for (int p = 0; p < TPW; ++p) pin_values(wrv[p][0], wrv[p][1], wrv[p][2], wrv[p][3]);
    const bool dv_vec_r = sizeof(Real) == 4 && (FULL || a.dv_vec);
    Real* const dv_tok_r = nslab == 1 ? (Real*)a.dv + tok0 * V
                                      : (Real*)a.ws + L.dv_part + ((int64_t)slab * B * T * N + tok0) * V;
    const int64_t NV_r = N * V;

    __syncthreads();  // prologue staging by the side role
    if constexpr (SW) {  // the forward role's sweep-only periods
      for (int i = 0; i < ((int)(a.C / S) + (S == 1 ? 1 : 0)) * S; ++i) __syncthreads();
    }

    auto phase = [&](auto Ic, int k, int slotA, int slotB, int par) {
      constexpr int I = decltype(Ic)::value;
      const int j = k * S + I;
      const int jp = j & 1;
      const int t = rstep(j);  // step reversed in this phase
      const bool act = ractive(j);
      const bool fin = j == jlast;
      if (act || fin) {
        // C = f R + D W^T of step t + 1 (other waves' D tiles from phase j - 1)
        Real db[NS];
#pragma unroll
        for (int q0 = 0; q0 < VT; ++q0) {
          const R4 t4 = q0 < TPW ? Dp[q0] : sm.xd[jp ^ 1][(q0 + TPW * wr) % VT][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) db[4 * q0 + r] = t4[r];
        }
        R4 acc[TPW];
#pragma unroll
        for (int p = 0; p < TPW; ++p) acc[p] = fR[p];
#pragma unroll
        for (int s0 = 0; s0 < NS; ++s0)
#pragma unroll
          for (int p = 0; p < TPW; ++p) acc[p] = mfma_16x16x4(wop[p][s0], db[s0], acc[p]);
        // read the accumulators before the branch below
#pragma unroll
        for (int p = 0; p < TPW; ++p) pin_vec(acc[p]);
        if (fin) {
          if (a.dH0 && row_ok) {
#pragma unroll
            for (int p = 0; p < TPW; ++p)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int col = col_of(p, r);
                if (col < V) ((Real*)a.dH0)[state_base + col] = acc[p][r];
              }
          }
        } else {
          // phase I >= 1 reverses step (cF + 1) S + S - I, phase 0 step (cF + 2) S
          constexpr int tt = I >= 1 ? S - I : 0;
          const Real* stp = &sm.st[I >= 1 ? slotA : slotB][tt * E];
          const Real f = stp[OFF_F];
          const Real omf = Real(1) - f;
          const Real qli = stp[OFF_Q + li];
          const int pos = (par * S - I) & (M - 1);  // ring position of t
          Real dfp = 0, dkp = 0;
#pragma unroll
          for (int p = 0; p < TPW; ++p) {
            const R4 hp = sm.hr[pos][wr * TPW + p][lane];
            const R4 u = cols4(stp + OFF_U + (wr * TPW + p) * 16, g);
            const R4 vv = cols4(stp + OFF_V + (wr * TPW + p) * 16, g);
            R4 D;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const Real rc = rcn[p][r];
              const Real z = fma_r(Real(-2), rc, Real(1));
              const Real sech2 = Real(4) * rc * (Real(1) - rc);
              const Real Rm = fma_r(qli, u[r], acc[p][r]);
              D[r] = omf * Rm * sech2;
              fR[p][r] = f * Rm;
              dfp = fma_r(Rm, hp[r] - z, dfp);
              dkp = fma_r(D[r], vv[r], dkp);
            }
            Dp[p] = D;
            sm.xd[jp][wr * TPW + p][lane] = D;
            if constexpr (Tr::kXdt) {
#pragma unroll
              for (int r = 0; r < 4; ++r) sm.xdT[jp][wr * TPW + p][acc_m<Real>(g, r)][trow] = D[r];
            }
          }
          sm.rk[jp][li][wr * 4 + g] = dkp;
          if constexpr (kDvRev) {
            // dv_t = D_t^T k_t over this slab's rows (+ w_r (.) u when the slab
            // is the whole head), reduced together with df's row sum
            static_assert(TPW == 1, "one tile per wave");
            const Real kq = stp[li];
            Real* dvp = dv_tok_r + (int64_t)t * NV_r;
            R4 sv = row16_sum_x4_e(Dp[0], kq, dfp);
            if (li == 0) sm.rf[jp][wr * 4 + g] = dfp;
            if (t < T32) {
#pragma unroll
              for (int p = 0; p < TPW; ++p) {
                if (li == 0) {
                  if (nslab == 1) {
                    const R4 u = cols4(stp + OFF_U + (wr * TPW + p) * 16, g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) sv[r] = fma_r(wrv[p][r], u[r], sv[r]);
                  }
                  const int col0 = col_of(p, 0);
                  if (dv_vec_r) {
                    if (FULL || col0 < V) *(R4*)(dvp + col0) = sv;
                  } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                      if (col_of(p, r) < V) dvp[col_of(p, r)] = sv[r];
                  }
                }
              }
            }
          } else {
            sm.rk[jp][li][wr * 4 + g] = dkp;
            dfp = row16_sum(dfp);
            if (li == 0) sm.rf[jp][wr * 4 + g] = dfp;
          }
          // rc of step t - 1, for the next phase
          if (t >= 1) {
#pragma unroll
            for (int p = 0; p < TPW; ++p) rcn[p] = sm.zr[(pos - 1) & (M - 1)][wr * TPW + p][lane];
          }
        }
      }
      if (j == S) {  // rc of the first reversed step
#pragma unroll
        for (int p = 0; p < TPW; ++p) rcn[p] = sm.zr[(nch * S - 1) & (M - 1)][wr * TPW + p][lane];
      }
    };

    for (int k = 0; k < nper; ++k) {
      const int cF = nch - 1 - k;  // chunk the forward role recomputes
      const int cA = cF + 1, cB = cF + 2;
      const int slotA = cA >= 0 ? cA % NSLOT : 0;
      const int slotB = cB >= 0 ? cB % NSLOT : 0;
      // step (cF + 1) S + S - I sits at ring position ((cF + 2) S - I) mod 2 S
      const int par = cB & 1;
      [&]<int... I>(std::integer_sequence<int, I...>) {
        ((phase(std::integral_constant<int, I>{}, k, slotA, slotB, par), __syncthreads()), ...);
      }(std::make_integer_sequence<int, S>{});
    }
  } else {
    // ================================================================ side role
    const int xt = tid - 2 * 64 * NW;  // thread index within the role
    const InT* __restrict__ kp = (const InT*)a.k;
    const InT* __restrict__ vp = (const InT*)a.v;
    const InT* __restrict__ qp = (const InT*)a.q;
    const Real* __restrict__ fp = (const Real*)a.f;
    const Real* __restrict__ dyp = (const Real*)a.dy;
    Real* __restrict__ ws = (Real*)a.ws;

    // ---- staging of one chunk's inputs.  Side thread xt owns the staged
    // values e = xt + m NX of a chunk (step e / E, field by e % E), each from
    // an InT array (k, q, v) or a Real array (dy, f); its source addresses for
    // chunk c are fixed pointers plus the step index times a stride, set up
    // once.  Steps past T are padding: f = 1 and dy = 0 make them exact
    // identities.  Raw values stay in registers until the LDS store at the
    // period's end, so nothing waits for the loads before then.
    const InT* ld_pin[NLD];
    const Real* ld_pre[NLD];
    int ld_ts[NLD], ld_tt[NLD];
    bool ld_in[NLD], ld_ok[NLD], ld_isf[NLD], ld_st[NLD];
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int e = xt + m * NX;
      const int tt = e / E, r = e % E;
      const InT* pin = kp;
      const Real* pre = fp;
      bool from_in = false, ok = false, isf = false;
      int ts = 0;
      if (e < S * E) {
        if (r < 32) {  // k (r < 16) or q, slab row r mod 16
          const int rr = slab * 16 + (r & 15);
          ok = rr < K;
          from_in = true;
          pin = (r < 16 ? kp : qp) + tokq0 * K + (ok ? rr : 0);
          ts = (int)(NQ * K);
        } else if (r < OFF_U) {  // v, column r - 32
          const int jj = r - OFF_V;
          ok = jj < V;
          from_in = true;
          pin = vp + tok0 * V + (ok ? jj : 0);
          ts = (int)(N * V);
        } else if (r < OFF_F) {  // dy, column r - 32 - VP
          const int jj = r - OFF_U;
          ok = jj < V;
          pre = dyp + tok0 * V + (ok ? jj : 0);
          ts = (int)(N * V);
        } else if (r == OFF_F) {  // f
          ok = true;
          isf = true;
          pre = fp + tok0;
          ts = (int)N;
        }
      }
      ld_pin[m] = pin;
      ld_pre[m] = pre;
      ld_ts[m] = ts;
      ld_tt[m] = e < S * E ? tt : 0;
      ld_in[m] = from_in;
      ld_ok[m] = ok;
      ld_isf[m] = isf;
      ld_st[m] = e < S * E;
    }
    InT stx_in[NLD];
    Real stx_re[NLD];
    bool stx_tv[NLD];
    auto stage_load = [&](int c) {
#pragma unroll
      for (int m = 0; m < NLD; ++m) {
        const int t = c * S + ld_tt[m];
        const bool tv = t < T32;
        const int64_t o = (int64_t)(tv ? t : T32 - 1) * ld_ts[m];
        stx_in[m] = ld_pin[m][ld_in[m] ? o : 0];
        stx_re[m] = ld_pre[m][ld_in[m] ? 0 : o];
        stx_tv[m] = tv;
      }
    };
    auto stage_store = [&](int c) {
      Real* dst = sm.st[c % NSLOT];
#pragma unroll
      for (int m = 0; m < NLD; ++m) {
        const Real x = ld_in[m] ? (Real)widen(stx_in[m]) : stx_re[m];
        const Real v = (ld_ok[m] && stx_tv[m]) ? x : (ld_isf[m] ? Real(1) : Real(0));
        if (ld_st[m]) dst[xt + m * NX] = v;
      }
    };
    // ---- start state of a chunk into register layout: element (row, col) of
    // the slab goes to tile col / 16, lane 16 acc_g(col % 16) + row, element
    // acc_r(col % 16).  Loads from clamped addresses; padding zeroed at the store.
    const Real* const cks_base = (const Real*)a.cks + (int64_t)bn * a.cks_count * K * V;
    const int64_t cks_stride = a.cks_step * K * V;
    int ck_src[NCK], ck_dst[NCK];
    bool ck_ok[NCK], ck_in[NCK];
#pragma unroll
    for (int m = 0; m < NCK; ++m) {
      const int e = xt + m * NX;
      const int rr = e / VP, col = e % VP, c16 = col & 15;
      const int grow = slab * 16 + rr;
      ck_in[m] = e < 16 * VP;
      ck_ok[m] = ck_in[m] && grow < K && col < V;
      ck_src[m] = ck_ok[m] ? grow * (int)V + col : 0;
      ck_dst[m] = ((col >> 4) * 64 + 16 * acc_g<Real>(c16) + rr) * 4 + acc_r<Real>(c16);
    }
    Real ckx[NCK];
    auto ck_load = [&](int c) {
      const Real* src = cks_base + c * cks_stride;
#pragma unroll
      for (int m = 0; m < NCK; ++m) ckx[m] = src[ck_src[m]];
    };
    auto ck_store = [&](int c) {
      Real* dst = (Real*)&sm.ck[c & 1][0][0];
#pragma unroll
      for (int m = 0; m < NCK; ++m)
        if (ck_in[m]) dst[ck_dst[m]] = ck_ok[m] ? ckx[m] : Real(0);
    };

    // ---- dW accumulators: this wave's row tiles wr * TPW + p, all column tiles
    R4 dWacc[TPW][VT];
    Real aop[TPW][4];
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) aop[p][kk] = Real(0);
#pragma unroll
      for (int jt = 0; jt < VT; ++jt) dWacc[p][jt] = R4{0, 0, 0, 0};
    }
    // transposed LDS element (row 4 kk + g, column li) of a state tile: lane
    // 16 acc_g(li) + 4 kk + g, element acc_r(li)
    auto tidx = [&](int kk) { return (16 * acc_g<Real>(li) + 4 * kk + g) * 4 + acc_r<Real>(li); };
    // output pointers at token (b, t = 0, n); step t adds t N rows
    Real* const dk_row = dk_base + tok0 * K + row;
    Real* const dq_row_s = dq_base + tok0 * K + row;
    Real* const df_tok = ws + L.df_part + (int64_t)slab * B * T * N + tok0;
    const int64_t NK = N * K;

    // both D buffers start at zero: the reverse role's first step reads the
    // (absent) later step's D, and dW multiplies zero A operands by the
    // transposed copy before the first D is written
    for (int i = xt; i < 2 * VT * 64; i += NX) (&sm.xd[0][0][0])[i] = R4{0, 0, 0, 0};
    for (int i = xt; i < (int)(sizeof(sm.xdT) / sizeof(Real)); i += NX) (&sm.xdT[0][0][0][0])[i] = Real(0);
    stage_load(nch - 1);
    if constexpr (!SW) ck_load(nch - 1);
    stage_store(nch - 1);
    if constexpr (!SW) ck_store(nch - 1);
    __syncthreads();
    if constexpr (SW) {  // the forward role's sweep-only periods
      for (int i = 0; i < ((int)(a.C / S) + (S == 1 ? 1 : 0)) * S; ++i) __syncthreads();
    }

    auto phase = [&](auto Ic, int k, int cF, int par) {
      constexpr int I = decltype(Ic)::value;
      const int j = k * S + I;
      const int jp = j & 1;
      // one wave per role: the reverse role's dk and df partials of phase j - 1,
      // read first so that their latency passes under the dW products
      R4 rkx = R4{0, 0, 0, 0}, rfx = R4{0, 0, 0, 0};
      Real rqx = 0;
      if constexpr (NW == 1) {
        rkx = *(const R4*)&sm.rk[jp ^ 1][li][0];
        rfx = *(const R4*)&sm.rf[jp ^ 1][0];
        rqx = sm.rq[jp ^ 1][li][0];
      }
      // dq of the forward role's step of phase j - 1 (kDvRev: one wave per
      // role, so its per-wave sum is the slab's)
      if constexpr (kDvRev) {
        if (g == 0 && (FULL || row_ok) && j >= 1 && j <= nch * S) {
          const int tf = I > 0 ? cF * S + I - 1 : cF * S + 2 * S - 1;
          if (tf < T32) dq_row_s[(int64_t)tf * NK] = rqx;
        }
      }
      // dW += S_t'^T D_t' for the reverse role's step t' of phase j - 1 (zero
      // A operands when it had none); B from the transposed D copy
      {
        R4 bop[VT];
#pragma unroll
        for (int jt = 0; jt < VT; ++jt) {
          if constexpr (Tr::kXdt) {
            bop[jt] = *(const R4*)&sm.xdT[jp ^ 1][jt][li][4 * g];
          } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) bop[jt][kk] = ((const Real*)&sm.xd[jp ^ 1][jt][0])[tidx(kk)];
          }
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int jt = 0; jt < VT; ++jt)
#pragma unroll
            for (int p = 0; p < TPW; ++p) dWacc[p][jt] = mfma_16x16x4(aop[p][kk], bop[jt][kk], dWacc[p][jt]);
      }
      // A operands for the reverse role's step of this phase, (cF + 2) S - I:
      // S_t transposed, or zeros when it takes none
      {
        const bool ra = ractive(j);
        const int pos = ra ? (par * S - I) & (M - 1) : 0;
#pragma unroll
        for (int p = 0; p < TPW; ++p)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const Real x = ((const Real*)&sm.hr[pos][wr * TPW + p][0])[tidx(kk)];
            aop[p][kk] = ra ? x : Real(0);
          }
      }
      // the reverse role's step of phase j - 1: tp = (cF + 2) S - I + 1
      if (!ractive(j - 1)) return;
      const int tp = (cF + 2) * S - I + 1;
      if (tp >= T32) return;
      // dk_t' and df_t' from the reverse role's partials: lane group q adds
      // entries 4 q .. 4 q + 3, then the four groups are added across lanes
      if constexpr (NW == 1) {
        // one wave: the four entries are the four lane groups' partials, so
        // every lane of group 0 holds its row's complete sum
        if (g == 0 && (FULL || row_ok)) dk_row[(int64_t)tp * NK] = (rkx[0] + rkx[1]) + (rkx[2] + rkx[3]);
        if (lane == 0) df_tok[(int64_t)tp * N] = (rfx[0] + rfx[1]) + (rfx[2] + rfx[3]);
        return;
      }
      if (wr == 0) {
        Real s4 = 0;
        if (4 * g < 4 * NW) {
          const R4 x = *(const R4*)&sm.rk[jp ^ 1][li][4 * g];
          s4 = (x[0] + x[1]) + (x[2] + x[3]);
        }
        s4 = cross_row_sum(s4);
        if (g == 0 && (FULL || row_ok)) dk_row[(int64_t)tp * NK] = s4;
      }
      if (wr == (1 % NW)) {
        Real s4 = 0;
        if (li == 0 && 4 * g < 4 * NW) {
          const R4 x = *(const R4*)&sm.rf[jp ^ 1][4 * g];
          s4 = (x[0] + x[1]) + (x[2] + x[3]);
        }
        s4 = cross_row_sum(s4);
        if (lane == 0) df_tok[(int64_t)tp * N] = s4;
      }
    };
    for (int k = 0; k < nper; ++k) {
      const int cF = nch - 1 - k;  // chunk the forward role recomputes
      const bool stage = cF >= 1;
      if (stage) {
        stage_load(cF - 1);
        if constexpr (!SW) ck_load(cF - 1);
      }
      const int par = (cF + 2) & 1;
      auto period_end = [&]() {
        if (stage) {
          stage_store(cF - 1);
          if constexpr (!SW) ck_store(cF - 1);
        }
      };
      [&]<int... I>(std::integer_sequence<int, I...>) {
        ((phase(std::integral_constant<int, I>{}, k, cF, par),
          (I == S - 1 ? period_end() : void()),
          __syncthreads()),
         ...);
      }(std::make_integer_sequence<int, S>{});
    }

    // this slab's share of dW: lane holds dW[16 c + m(g, r)][16 jt + li].
    // The last dW MFMAs sit in the loop; sleep before the accumulators are read.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_sleep(2);
    __builtin_amdgcn_sched_barrier(0);
    Real* dWp = ws + L.dW_part + (((size_t)b * nslab + slab) * N + n) * V * V;
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int jt = 0; jt < VT; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int l = col_of(p, r);
          const int jj = jt * 16 + li;
          if (l < V && jj < V) dWp[(int64_t)l * V + jj] = dWacc[p][jt][r];
        }
  }
}

// The same chunk-start states from the forward's stored rc: the
// interpolation S_{t+1} = (f S_t + (1 - f)) - 2 (1 - f) rc_t acts on every
// state element alone, so each thread carries four elements of one (b, n)
// through one checkpoint interval with no exchange and no matrix product
// (bit for bit the forward's arithmetic).  Workgroup id = (unit, interval,
// block of 1024 elements); elements are K V per unit.
template <typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_bwd_starts_rc_kernel(BwdArgs a, int S, int64_t nch, int64_t id0,
                               Real* __restrict__ out) {
  const int64_t T = a.T, N = a.N, KV = a.K * a.V, C = a.C;
  const int64_t eblocks = (KV + 1023) / 1024;
  const int64_t nck = (T + C - 1) / C;
  const int64_t id = id0 + blockIdx.x;
  const int64_t eb = id % eblocks;
  const int64_t c = (id / eblocks) % nck;  // checkpoint interval
  const int64_t bn = id / eblocks / nck;   // (b, n) unit
  const int64_t e0 = (eb * 256 + threadIdx.x) * 4;
  if (e0 >= KV) return;
  const int64_t t0 = c * C;
  const int64_t xmax = (nch - 1) * S;  // last chunk start
  if (t0 > xmax) return;
  const int64_t tend = (t0 + C < T ? t0 + C : T) < xmax ? (t0 + C < T ? t0 + C : T) : xmax;
  const int ne = KV - e0 < 4 ? (int)(KV - e0) : 4;  // elements of this thread
  const Real* ck = (const Real*)a.ckpt + (bn * nck + c) * KV + e0;
  const Real* rcp = (const Real*)a.rc + (bn * T + t0) * KV + e0;
  const Real* fp = (const Real*)a.f + (bn / N) * T * N + (bn % N);  // f of (b, t = 0, n)
  Real h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = i < ne ? ck[i] : Real(0);
  auto write_start = [&](int64_t x) {
    Real* dst = out + (bn * nch + x / S) * KV + e0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < ne) dst[i] = h[i];
  };
  if (t0 % S == 0) write_start(t0);
  if (sizeof(Real) == 4 && ne == 4 && (KV & 3) == 0 && a.rc_vec) {
    // four consecutive fp32 elements: one 16-byte load per step, eight steps'
    // loads issued ahead of their use
    using R4 = typename Vec4<Real>::type;
    int64_t t = t0;
    for (; t + 8 <= tend; t += 8) {
      R4 rv[8];
      Real fv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        rv[u] = *(const R4*)(rcp + (t - t0 + u) * KV);
        fv[u] = fp[(t + u) * N];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const Real omf = Real(1) - fv[u];
        const Real m2omf = Real(-2) * omf;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = fma_r(m2omf, rv[u][i], fma_r(fv[u], h[i], omf));
        if ((t + u + 1) % S == 0) write_start(t + u + 1);
      }
    }
    for (; t < tend; ++t) {
      const R4 rv = *(const R4*)(rcp + (t - t0) * KV);
      const Real f = fp[t * N];
      const Real omf = Real(1) - f;
      const Real m2omf = Real(-2) * omf;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = fma_r(m2omf, rv[i], fma_r(f, h[i], omf));
      if ((t + 1) % S == 0) write_start(t + 1);
    }
    return;
  }
  for (int64_t t = t0; t < tend; ++t, rcp += KV) {
    const Real f = fp[t * N];
    const Real omf = Real(1) - f;
    const Real m2omf = Real(-2) * omf;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < ne) h[i] = fma_r(m2omf, rcp[i], fma_r(f, h[i], omf));
    if ((t + 1) % S == 0) write_start(t + 1);
  }
}

// Chunk-start states at every multiple of S, recomputed from the forward's
// checkpoints when C does not divide S.  One workgroup per (slab, checkpoint
// interval): the intervals are independent, so they all run at once and the
// matrix units stay busy in spite of the step-to-step latency.  The step is
// the forward kernel's, operation for operation, so the states are bitwise
// the ones the forward produced.
template <typename InT, typename Real, int VT>
__global__ void __launch_bounds__((BwdShape<Real, VT>::NW * 64))
    m2rnn_bwd_starts_kernel(BwdArgs a, int64_t nch, int64_t id0, Real* __restrict__ out) {
  using Sh = BwdShape<Real, VT>;
  constexpr int S = BwdTraits<Real, VT>::S;
  using R4 = typename Vec4<Real>::type;
  constexpr int TPW = Sh::TPW, NS = Sh::NS;
  __shared__ R4 xb[2][VT][64];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int64_t units = a.B * a.N * a.nslab;
  const int64_t id = id0 + blockIdx.x;
  const int unit = (int)(id % units);
  const int64_t c = id / units;  // checkpoint interval
  const int nslab = a.nslab;
  const int slab = unit % nslab;
  const int bn = unit / nslab;
  const int64_t T = a.T, N = a.N, K = a.K, V = a.V, C = a.C;
  const int n = (int)(bn % N);
  const int b = (int)(bn / N);
  const int row = slab * 16 + li;
  const bool row_ok = row < K;
  const int64_t nck = (T + C - 1) / C;
  const int64_t t0 = c * C;
  const int64_t xmax = (nch - 1) * S;  // last chunk start
  if (t0 > xmax) return;               // uniform over the workgroup
  const int64_t tend = (t0 + C < T ? t0 + C : T) < xmax ? (t0 + C < T ? t0 + C : T) : xmax;
  const int64_t tok0 = (int64_t)b * T * N + n;
  const int64_t tokq0 = (int64_t)b * T * a.NQ + n / (int)(N / a.NQ);  // shared q/k head
  const InT* __restrict__ kp = (const InT*)a.k;
  const InT* __restrict__ vp = (const InT*)a.v;
  const Real* __restrict__ fp = (const Real*)a.f;
  const Real* __restrict__ Wp = (const Real*)a.W;

  // W^T (scaled) and the interval's start state: all loads from clamped
  // addresses first, completed together, then masked (a guarded load would be
  // a branch whose join waits for it, one load at a time)
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
  const Real* ck = (const Real*)a.ckpt + (((int64_t)bn * nck + c) * K + (row_ok ? row : 0)) * V;
  Real hb[NS];
  R4 h[TPW];
#pragma unroll
  for (int q0 = 0; q0 < VT; ++q0) {
    const int q = (q0 + TPW * w) % VT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = 16 * q + acc_m<Real>(g, r);
      hb[4 * q0 + r] = ck[col < V ? col : 0];
    }
  }
#pragma unroll
  for (int s0 = 0; s0 < NS; s0 += 4) {
#pragma unroll
    for (int p = 0; p < TPW; ++p) pin_values(wa[p][s0], wa[p][s0 + 1], wa[p][s0 + 2], wa[p][s0 + 3]);
    pin_values(hb[s0], hb[s0 + 1], hb[s0 + 2], hb[s0 + 3]);
  }
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
    const int col = (w * TPW + p) * 16 + li;
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) {
      const int s = (s0 + 4 * TPW * w) % NS;
      const int l = 16 * (s >> 2) + acc_m<Real>(g, s & 3);
      wa[p][s0] = (col < V && l < V) ? kTanhScale<Real> * wa[p][s0] : Real(0);
    }
#pragma unroll
    for (int s0 = 0; s0 < NS; s0 += 4) pin_values(wa[p][s0], wa[p][s0 + 1], wa[p][s0 + 2], wa[p][s0 + 3]);
  }
#pragma unroll
  for (int q0 = 0; q0 < VT; ++q0) {
    const int q = (q0 + TPW * w) % VT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = 16 * q + acc_m<Real>(g, r);
      hb[4 * q0 + r] = (row_ok && col < V) ? hb[4 * q0 + r] : Real(0);
    }
  }
#pragma unroll
  for (int p = 0; p < TPW; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) h[p][r] = hb[4 * p + r];
  auto write_start = [&](int64_t x) {
    if (!row_ok) return;
    Real* dst = out + (((int64_t)bn * nch + x / S) * K + row) * V;
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = (w * TPW + p) * 16 + acc_m<Real>(g, r);
        if (col < V) dst[col] = h[p][r];
      }
  };
  if ((t0 & (S - 1)) == 0) write_start(t0);
  // Inputs of a step, loaded raw one step ahead (from clamped addresses) so
  // that their latency hides behind the previous step's MFMA chain.
  InT kr, vr[TPW][4];
  Real fr;
  auto load_step = [&](int64_t t) {
    const int64_t tok = tok0 + t * N;
    fr = fp[tok];
    kr = kp[(tokq0 + t * a.NQ) * K + (row_ok ? row : 0)];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = (w * TPW + p) * 16 + acc_m<Real>(g, r);
        vr[p][r] = vp[tok * V + (col < V ? col : 0)];
      }
  };
  // a raw input converted in a register (kept there before any select)
  auto held = [&](auto x) -> Real {
    Real y = (Real)widen(x);
    asm volatile("" : "+v"(y));
    return y;
  };
  load_step(t0);
  for (int64_t t = t0; t < tend; ++t) {
    const Real f = held(fr);
    const Real kli = held(kr);
    Real vv[TPW][4];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) vv[p][r] = held(vr[p][r]);
    load_step(t + 1 < tend ? t + 1 : t);
    // the scaled rank-1 write k v^T starts the accumulators, as in the forward
    const Real ks = kTanhScale<Real> * (row_ok ? kli : Real(0));
    R4 acc[TPW];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = (w * TPW + p) * 16 + acc_m<Real>(g, r);
        acc[p][r] = ks * (col < V ? vv[p][r] : Real(0));
      }
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0)
#pragma unroll
      for (int p = 0; p < TPW; ++p) acc[p] = mfma_16x16x4(wa[p][s0], hb[s0], acc[p]);
    const Real omf = Real(1) - f;
    const Real m2omf = Real(-2) * omf;
    const int P = (int)(t & 1);
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        h[p][r] = fma_r(m2omf, tanh_rc_scaled(acc[p][r]), fma_r(f, h[p][r], omf));
      xb[P][w * TPW + p][lane] = h[p];
    }
    __syncthreads();
    if (((t + 1) & (S - 1)) == 0) write_start(t + 1);
#pragma unroll
    for (int q0 = TPW; q0 < VT; ++q0) {
      const R4 t4 = xb[P][(q0 + TPW * w) % VT][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) hb[4 * q0 + r] = t4[r];
    }
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) hb[4 * p + r] = h[p][r];
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

// dv = sum over slabs of the partials + w_r (.) dy (64-bit indices, for sizes beyond
// m2rnn_slab_sum_kernel's)
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

// Sum over groups of G consecutive heads (shared q and k: the gradient of a
// shared head is the sum of its value heads' gradients): out[r][i] =
// sum_{g < G} part[(r G + g) K + i] for the rows r of [B, T, NQ], in head order.
// `vec` (fp32, K % 4 == 0, both arrays 16-byte aligned): four columns per
// thread with 16-byte accesses, the group's loads issued four at a time and
// added in head order (the same sums, bit for bit).
template <typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_group_sum_kernel(int64_t total, int64_t K, int G, const Real* __restrict__ part,
                           Real* __restrict__ out, bool vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (sizeof(Real) == 4 && vec) {
    const int64_t total4 = total >> 2, K4 = K >> 2;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total4; e += stride) {
      const int64_t r = e / K4, i = e - r * K4;
      const f32x4* p = (const f32x4*)part + r * G * K4 + i;
      f32x4 s = p[0];
      int g = 1;
      for (; g + 3 < G; g += 4) {
        const f32x4 a0 = p[g * K4], a1 = p[(g + 1) * K4], a2 = p[(g + 2) * K4],
                    a3 = p[(g + 3) * K4];
        s += a0;
        s += a1;
        s += a2;
        s += a3;
      }
      for (; g < G; ++g) s += p[g * K4];
      ((f32x4*)out)[e] = s;
    }
    return;
  }
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int64_t r = e / K, i = e - r * K;
    const Real* p = part + r * G * K + i;
    Real s = p[0];
    for (int g = 1; g < G; ++g) s += p[(int64_t)g * K];
    out[e] = s;
  }
}

// Column sums over the B*T token rows, stage 1: one block per (row block of
// 256 rows, head).  Columns 0..V-1: dy (.) v (-> dw_r); V: -df softplus(x) f
// (-> dalpha); V+1: dlogit (-> dbeta).  The block's 256 threads are four row
// groups (rows r0 + g, r0 + g + 4, ...) of 64 column slots; the four group
// sums are added in a fixed order.
template <typename InT, typename Real>
__global__ void __launch_bounds__(256)
    m2rnn_bwd_colsum_kernel(int64_t rows, int64_t N, int64_t V, int kind,
                            const Real* __restrict__ dy, const InT* __restrict__ v,
                            const Real* __restrict__ df, const Real* __restrict__ f,
                            const Real* __restrict__ logit, const Real* __restrict__ alpha,
                            const Real* __restrict__ beta, const Real* __restrict__ dlogit,
                            Real* __restrict__ col_part) {
  constexpr int kMaxCols = 16 * kMaxValueTiles + 2;
  __shared__ Real red[16][kMaxCols];  // [wave x rows per load][column] partials
  __shared__ Real red2[2][256];       // the two per-head columns, one row per thread
  // one block per (row block, head), heads fastest, each XCD taking a
  // contiguous range: neighbouring heads of a row block share an L2, and with
  // V < 32 they share the 128-byte lines of dy and v
  const int64_t unit = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t rb = unit / N;
  const int64_t n = unit - rb * N;
  const int ncol = (int)V + 2;
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int64_t r0 = rb * 256;
  const int64_t r1 = (r0 + 256) < rows ? (r0 + 256) : rows;
  // value columns: with V < 64 one load covers rpl = min(4, 64 / V) rows (lane:
  // row offset lane / V, column lane % V), so narrow heads use most lanes
  const int rpl = V < 16 ? 4 : V < 64 ? (int)(64 / V) : 1;
  const int ro = V < 64 ? lane / (int)V : 0;
  const int64_t rstep = 4 * rpl * N * V;  // element step between a lane's rows
  for (int c0 = 0; c0 < (int)V; c0 += 64) {
    const int col = V < 64 ? lane % (int)V : c0 + lane;
    Real s = 0;
    if (ro < rpl && col < (int)V) {
      const int64_t rfirst = r0 + grp * rpl + ro;
      int64_t i = (rfirst * N + n) * V + col;
      for (int64_t r = rfirst; r < r1; r += 4 * rpl, i += rstep) s += dy[i] * load_as<Real>(v + i);
      red[grp * rpl + ro][col] = s;
    }
  }
  // the per-head columns (exp-softplus gate): dalpha and dbeta terms of row r0 + tid
  if (kind == kGateExpSoftplus) {
    const int64_t r = r0 + threadIdx.x;
    Real ta = 0, tb = 0;
    if (r < r1) {
      const int64_t i = r * N + n;
      ta = -df[i] * softplus_(logit[i] + beta[n]) * f[i];
      tb = dlogit[i];
    }
    red2[0][threadIdx.x] = ta;
    red2[1][threadIdx.x] = tb;
  }
  __syncthreads();
  // fixed-order sums: value columns over the 4 rpl partials, per-head columns
  // over the 256 rows by a tree
  for (int col = threadIdx.x; col < (int)V; col += blockDim.x) {
    Real s = 0;
    for (int k = 0; k < 4 * rpl; ++k) s += red[k][col];
    col_part[(rb * N + n) * ncol + col] = s;
  }
  if (kind == kGateExpSoftplus) {
    for (int h = 128; h >= 1; h >>= 1) {
      if ((int)threadIdx.x < 2 * h) {
        const int w = threadIdx.x / h, k = threadIdx.x % h;
        red2[w][k] += red2[w][k + h];
      }
      __syncthreads();
    }
    if (threadIdx.x < 2) col_part[(rb * N + n) * ncol + V + threadIdx.x] = red2[threadIdx.x][0];
  } else if (threadIdx.x < 2) {
    col_part[(rb * N + n) * ncol + V + threadIdx.x] = Real(0);
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
static hipError_t launch_bwd_vt(const BwdArgs& a0, hipStream_t stream) {
  using Tr = BwdTraits<Real, VT>;
  static_assert(sizeof(BwdSmem<Real, VT>) <= kLdsBytes, "LDS budget");
  BwdArgs a = a0;
  const BwdWorkspace L = bwd_workspace_layout(a.B, a.T, a.N, a.NQ, a.K, a.V, a.C,
                                              sizeof(Real) == 8 ? kF64 : kF32, a.rc != nullptr);
  Real* ws = (Real*)a.ws;
  const int64_t units = a.B * a.N * a.nslab;
  const int64_t nck = (a.T + a.C - 1) / a.C;
  hipError_t err;
  if (L.sweep) {
    // the main kernel sweeps each checkpoint interval itself
    a.ring_s = ws + L.ring_s;
    a.ring_r = a.rc ? nullptr : (void*)(ws + L.ring_r);
    a.cks = nullptr;
    a.cks_count = 0;
    a.cks_step = 0;
  } else if (L.subck_needed) {
    // one workgroup per (slab, checkpoint interval), in launches of at most 2^24 workgroups
    const int64_t total = units * nck;
    if (a.rc) {
      // from the stored rc: elementwise, one workgroup per (unit, interval, 1024 elements)
      const int64_t tot = a.B * a.N * nck * ((a.K * a.V + 1023) / 1024);
      for (int64_t id0 = 0; id0 < tot; id0 += (int64_t)1 << 24) {
        const int64_t cnt = tot - id0 < ((int64_t)1 << 24) ? tot - id0 : ((int64_t)1 << 24);
        hipLaunchKernelGGL((m2rnn_bwd_starts_rc_kernel<Real>), dim3((unsigned)cnt), dim3(256), 0,
                           stream, a, Tr::S, L.nch, id0, ws + L.subck);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
    } else {
      for (int64_t id0 = 0; id0 < total; id0 += (int64_t)1 << 24) {
        const int64_t cnt = total - id0 < ((int64_t)1 << 24) ? total - id0 : ((int64_t)1 << 24);
        hipLaunchKernelGGL((m2rnn_bwd_starts_kernel<InT, Real, VT>), dim3((unsigned)cnt),
                           dim3(Tr::NW * 64), 0, stream, a, L.nch, id0, ws + L.subck);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
    }
    a.cks = ws + L.subck;
    a.cks_count = L.nch;
    a.cks_step = 1;
  } else {
    a.cks = a.ckpt;
    a.cks_count = nck;
    a.cks_step = Tr::S / a.C;
  }
  // 16-byte rc loads and dv stores where fp32 columns come in fours and the
  // arrays are aligned for them (dv goes to the workspace partials when the
  // head has several slabs)
  const bool v4 = sizeof(Real) == 4 && (a.V & 3) == 0;
  a.rc_vec = v4 && aligned16(a.rc);
  a.dv_vec = v4 && aligned16(a.nslab == 1 ? a.dv : (const void*)(ws + L.dv_part));
  // every tile full: K rows in whole slabs, V columns in whole tiles, fp32 state,
  // rc and the dv destination 16-byte aligned
  const bool full = sizeof(Real) == 4 && a.K % 16 == 0 && a.V == Tr::VP && a.rc_vec && a.dv_vec;
  const dim3 grid((unsigned)units), block(Tr::NT);
  // variants: states from the stored rc (RC) or recomputed; every tile full (FULL);
  // intervals swept by the main kernel (SW)
  auto go = [&](auto rc_c, auto full_c, auto sw_c) {
    hipLaunchKernelGGL((m2rnn_bwd_kernel<InT, Real, VT, decltype(rc_c)::value,
                                         decltype(full_c)::value, decltype(sw_c)::value>),
                       grid, block, 0, stream, a, L);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto pick_sw = [&](auto rc_c, auto full_c) {
    if constexpr (Tr::S >= 2) {  // (the sweep needs chunks of two steps or more)
      if (L.sweep) {
        go(rc_c, full_c, T_{});
        return;
      }
    }
    go(rc_c, full_c, F_{});
  };
  auto pick_rc = [&](auto full_c) {
    if (a.rc) pick_sw(T_{}, full_c);
    else pick_sw(F_{}, full_c);
  };
  if constexpr (sizeof(Real) == 4) {
    if (full) pick_rc(T_{});
  }
  if (!full) pick_rc(F_{});
  if ((err = hipGetLastError()) != hipSuccess) return err;

  const int64_t tokens = a.B * a.T * a.N;
  hipLaunchKernelGGL((m2rnn_bwd_token_kernel<Real>), dim3(grid_for(tokens)), dim3(256), 0, stream,
                     tokens, a.N, a.nslab, a.gate_kind, ws + L.df_part, (const Real*)a.f,
                     (const Real*)a.logit, (const Real*)a.alpha, (const Real*)a.beta,
                     (Real*)a.dlogit);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.nslab > 1) {
    const int64_t total = tokens * a.V;
    if (total < ((int64_t)1 << 31)) {
      hipLaunchKernelGGL((m2rnn_slab_sum_kernel<Real, Real>), dim3(grid_for(total)), dim3(256), 0,
                         stream, (int)tokens, (int)a.N, (int)a.V, a.nslab, total, ws + L.dv_part,
                         (const Real*)a.dy, (const Real*)a.w_r, (Real*)a.dv,
                         slab_sum_vec<Real, Real>(a.V, ws + L.dv_part, a.dy, a.w_r, a.dv));
    } else {
      hipLaunchKernelGGL((m2rnn_bwd_dv_kernel<Real>), dim3(grid_for(total)), dim3(256), 0, stream,
                         total, a.N, a.V, a.nslab, ws + L.dv_part, (const Real*)a.dy,
                         (const Real*)a.w_r, (Real*)a.dv);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (a.NQ < a.N) {
    // shared q and k: dk and dq of a shared head are the sums over its group
    const int64_t out = a.B * a.T * a.NQ * a.K;
    const bool gv = sizeof(Real) == 4 && a.K % 4 == 0;  // the workspace partials are aligned
    const bool vk = gv && aligned16(a.dk), vq = gv && aligned16(a.dq);
    hipLaunchKernelGGL((m2rnn_group_sum_kernel<Real>), dim3(grid_for(vk ? out / 4 : out)), dim3(256),
                       0, stream, out, a.K, (int)(a.N / a.NQ), ws + L.dk_part, (Real*)a.dk, vk);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((m2rnn_group_sum_kernel<Real>), dim3(grid_for(vq ? out / 4 : out)), dim3(256),
                       0, stream, out, a.K, (int)(a.N / a.NQ), ws + L.dq_part, (Real*)a.dq, vq);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int64_t per = a.N * a.V * a.V;
  hipLaunchKernelGGL((m2rnn_bwd_dw_kernel<Real>), dim3(grid_for(per)), dim3(256), 0, stream, per,
                     a.B * a.nslab, ws + L.dW_part, (Real*)a.dW);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((m2rnn_bwd_colsum_kernel<InT, Real>),
                     dim3((unsigned)(L.row_blocks * a.N)), dim3(256), 0, stream,
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
