// Single-token step of the M²RNN recurrence (decoding) for gfx950.
//
// For a batch of sequences that each take one more token, every (b, n) unit
// applies one step of the recurrence of the M²RNN review (section 2.1,
// Eq. 10-12) to its state, in place, and reads it out:
//     H <- f H + (1 - f) tanh(H W_n + k v^T),   y = H^T q + w_r (.) v.
// This is the sequential cell step of the pararnn-torch "ParaM2RNN" page
// ("Reproduce (sequential)") with the review's readout.
//
// Work decomposition.  The state of a unit is read once and written once, so
// the step moves 2 K V state elements per (b, n) while doing 2 K V^2 flop of
// H W: about V / 4 flop per byte in fp32, near the MFMA-to-HBM balance point
// of the chip at V = 64 (157 TFLOP/s against 8 TB/s).  A wave owns one unit
// and walks its 16-row slabs; the four waves of a workgroup take batch rows
// of one head and share W^T, which is staged once in LDS in MFMA operand
// order.  The product is computed transposed, (H W)^T = W^T H^T, on the
// 16x16x4 MFMA with the contraction index of MFMA s enumerated as
// 16 (s / 4) + m(g, s % 4) (m the accumulator row map): then the lane that
// holds element r of output tile c also loaded H at exactly that position, so
// the interpolation with the old state, the store of the new one and the
// readout need no data movement between lanes: each lane accumulates its
// share of H^T q over the unit's slabs, and one DPP row sum per unit
// finishes the readout.  The grid is
// sized to what the device holds at once: each wave takes several batch rows
// in turn (the workgroup stages W once for all of them) and loads the next
// (row, slab) while computing the current one (16-byte loads in fp32).

#include <atomic>
#include <type_traits>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

template <typename InT, typename Real, int VT>
__global__ void __launch_bounds__(256, VT == 4 ? 3 : 1) m2rnn_step_kernel(StepArgs a) {
  using R4 = typename Vec4<Real>::type;
  constexpr int VP = 16 * VT;
  // W^T of the head in MFMA A-operand order: wl[c][j][lane][r] =
  // (2 / ln 2) W[16 j + m(g, r)][16 c + li], zero in the padding
  __shared__ R4 wl[VT][VT][64];
  __shared__ Real wrl[VP];  // w_r of the head (zero in the padding)

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int64_t B = a.B, N = a.N, K = a.K, V = a.V, NQ = a.NQ;
  const int64_t n = (int64_t)blockIdx.x % N;
  // the workgroup's batch rows: 4 upw of them from ((id / N) 4 upw), wave w
  // taking every fourth
  int64_t b = ((int64_t)blockIdx.x / N) * 4 * a.upw + w;

  const Real* __restrict__ Wp = (const Real*)a.W + n * V * V;
  for (int e = tid; e < VP * VP; e += 256) {
    const int l = e / VP, col = e % VP;  // W row (contraction) and column (output)
    const bool ok = l < V && col < V;
    Real x = Wp[(ok ? l : 0) * V + (ok ? col : 0)];
    pin_value(x);
    const int m = l & 15;
    ((Real*)&wl[col >> 4][l >> 4][16 * acc_g<Real>(m) + (col & 15)])[acc_r<Real>(m)] =
        ok ? kTanhScale<Real> * x : Real(0);
  }
  if (tid < VP) wrl[tid] = tid < V ? ((const Real*)a.w_r)[n * V + tid] : Real(0);
  __syncthreads();
  if (b >= B) return;  // a partial last group of batch rows

  const int64_t nq = n / (N / NQ);  // the q / k head this value head reads
  auto col_of = [&](int c, int r) { return 16 * c + acc_m<Real>(g, r); };
  const bool vec = sizeof(Real) == 4 && a.vec;
  const int nslab = (int)((K + 15) / 16);

  // Loaded k, v, q stay raw, one 32-bit register per bf16 value, until they
  // are used, so that no conversion (or packing) waits for a prefetch in flight.
  using Raw = std::conditional_t<std::is_same_v<InT, uint16_t>, uint32_t, InT>;
  auto raw_load = [](const InT* p) -> Raw { return (Raw)*p; };
  auto held = [](Raw x) -> Real {
    Real y;
    if constexpr (std::is_same_v<InT, uint16_t>)
      y = (Real)__builtin_bit_cast(float, x << 16);
    else
      y = (Real)x;
    asm volatile("" : "+v"(y));
    return y;
  };

  // Per unit: v at this lane's columns 16 c + m(g, r), and the gate.
  auto load_unit = [&](int64_t bb, Raw (&vr)[VT][4], Real& ff) {
    const InT* vp = (const InT*)a.v + (bb * N + n) * V;
#pragma unroll
    for (int c = 0; c < VT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = col_of(c, r);
        vr[c][r] = raw_load(vp + (col < V ? col : 0));
      }
    ff = ((const Real*)a.f)[bb * N + n];
  };
  auto mask_unit = [&](const Raw (&vr)[VT][4], Real (&vv)[VT][4]) {
#pragma unroll
    for (int c = 0; c < VT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const Real x = held(vr[c][r]);
        vv[c][r] = col_of(c, r) < V ? x : Real(0);
      }
  };
  // Per slab: the old state at this lane's positions (row 16 sl + li, columns
  // 16 j + m(g, r)) and k, q of the row; all from clamped addresses, masked
  // once the loads have completed.
  auto load_slab = [&](int64_t bb, int sl, R4 (&h)[VT], Raw& kr, Raw& qr) {
    const int row = sl * 16 + li;
    const int rr = row < K ? row : 0;
    const Real* src = (const Real*)a.H + ((bb * N + n) * K + rr) * V;
    if (vec) {
#pragma unroll
      for (int j = 0; j < VT; ++j) {
        const int c0 = 16 * j + 4 * g;
        h[j] = *(const R4*)(src + (c0 < V ? c0 : 0));
      }
    } else {
#pragma unroll
      for (int j = 0; j < VT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = col_of(j, r);
          h[j][r] = src[col < V ? col : 0];
        }
    }
    const int64_t kq = (bb * NQ + nq) * K + rr;
    kr = raw_load((const InT*)a.k + kq);
    qr = raw_load((const InT*)a.q + kq);
  };
  auto mask_slab = [&](int sl, R4 (&h)[VT], Raw kr, Raw qr, Real& kk, Real& qq) {
    const bool row_ok = sl * 16 + li < K;
#pragma unroll
    for (int j = 0; j < VT; ++j) {
      pin_vec(h[j]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!(row_ok && col_of(j, r) < V)) h[j][r] = Real(0);
    }
    const Real kx = held(kr), qx = held(qr);
    kk = row_ok ? kx : Real(0);
    qq = row_ok ? qx : Real(0);
  };

  // This wave's units: batch rows b, b + 4, ... below b_end (upw of them at
  // most), walked in groups of PD slabs; the next (unit, group) is loaded
  // while the current one is computed.  Narrow states take several slabs per
  // group so that a wave keeps a few KB of state loads in flight.
  constexpr int PD = VT >= 3 ? 1 : (VT == 2 ? 2 : 4);
  const int ngrp = (nslab + PD - 1) / PD;
  const int64_t b_end = ((int64_t)blockIdx.x / N + 1) * 4 * a.upw < B
                            ? ((int64_t)blockIdx.x / N + 1) * 4 * a.upw
                            : B;
  Real vcur[VT][4], fcur, fnx = 0, kk[PD], qq[PD];
  Raw vnx[VT][4], knx[PD], qnx[PD];
  R4 h[PD][VT], hnx[PD][VT];
#pragma unroll
  for (int p = 0; p < PD; ++p)
#pragma unroll
    for (int j = 0; j < VT; ++j) hnx[p][j] = R4{0, 0, 0, 0};
  auto load_group = [&](int64_t bb, int grp, R4 (&hh)[PD][VT], Raw (&kr)[PD], Raw (&qr)[PD]) {
#pragma unroll
    for (int p = 0; p < PD; ++p) load_slab(bb, grp * PD + p, hh[p], kr[p], qr[p]);
  };
  auto mask_group = [&](int grp, R4 (&hh)[PD][VT], Raw (&kr)[PD], Raw (&qr)[PD]) {
#pragma unroll
    for (int p = 0; p < PD; ++p) mask_slab(grp * PD + p, hh[p], kr[p], qr[p], kk[p], qq[p]);
  };
  load_unit(b, vnx, fcur);
  load_group(b, 0, h, knx, qnx);
  mask_unit(vnx, vcur);
  mask_group(0, h, knx, qnx);
  R4 yacc[VT];
#pragma unroll
  for (int c = 0; c < VT; ++c) yacc[c] = R4{0, 0, 0, 0};
  int grp = 0;
  while (true) {
    // the next (unit, group), if any
    const bool same_unit = grp + 1 < ngrp;
    const int64_t nb = same_unit ? b : b + 4;
    const int ngr = same_unit ? grp + 1 : 0;
    const bool has_next = nb < b_end;
    if (has_next) {
      load_group(nb, ngr, hnx, knx, qnx);
      if (!same_unit) load_unit(nb, vnx, fnx);
    }
    const Real omf = Real(1) - fcur, m2omf = Real(-2) * omf;
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int sl = grp * PD + p;
      if (PD > 1 && sl >= nslab) break;  // past the last slab (uniform)
      const bool row_ok = sl * 16 + li < K;
      const Real ks = kTanhScale<Real> * kk[p];
      Real* dst = (Real*)a.H + ((b * N + n) * K + (row_ok ? sl * 16 + li : 0)) * V;
#pragma unroll
      for (int c = 0; c < VT; ++c) {
        // the scaled rank-1 write starts the accumulators, then H W over all tiles
        R4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = ks * vcur[c][r];
#pragma unroll
        for (int j = 0; j < VT; ++j) {
          const R4 a4 = wl[c][j][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc = mfma_16x16x4(a4[r], h[p][j][r], acc);
        }
        pin_vec(acc);
        // H = f H + (1 - f) tanh(A) = (f H + (1 - f)) - 2 (1 - f) / (1 + e^{2A})
        R4 hn;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hn[r] = fma_r(m2omf, tanh_rc_scaled(acc[r]), fma_r(fcur, h[p][c][r], omf));
        if (vec) {
          if (row_ok && 16 * c + 4 * g < V) *(R4*)(dst + 16 * c + 4 * g) = hn;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (row_ok && col_of(c, r) < V) dst[col_of(c, r)] = hn[r];
        }
        // readout: this lane's share of sum_rows H q, reduced over the 16
        // lanes of each row once the unit is done
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[c][r] = fma_r(hn[r], qq[p], yacc[c][r]);
      }
    }
    if (!same_unit) {
      // y = H^T q + w_r (.) v of the finished unit: the lane shares summed
      // over each 16-lane row, written from lane 16 g
      R4 ys[VT];
#pragma unroll
      for (int c = 0; c < VT; ++c) ys[c] = row16_sum_x4(yacc[c], Real(1));
      if (li == 0) {
        Real* __restrict__ yp = (Real*)a.y + (b * N + n) * V;
#pragma unroll
        for (int c = 0; c < VT; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int col = col_of(c, r);
            if (col < V) yp[col] = ys[c][r] + wrl[col] * vcur[c][r];
          }
      }
#pragma unroll
      for (int c = 0; c < VT; ++c) yacc[c] = R4{0, 0, 0, 0};
    }
    if (!has_next) break;
    mask_group(ngr, hnx, knx, qnx);
#pragma unroll
    for (int p = 0; p < PD; ++p)
#pragma unroll
      for (int j = 0; j < VT; ++j) h[p][j] = hnx[p][j];
    if (!same_unit) {
      mask_unit(vnx, vcur);
      fcur = fnx;
    }
    b = nb;
    grp = ngr;
  }
}

// Full-tile step at V = 64: fp32 state, K a multiple of 16, the state and y
// 16-byte aligned, k, q, v and f 4-byte aligned (checked on the host).  (At
// V = 16 the step is bound by HBM alone and the general kernel, with four
// slabs per load group, reaches 70 % of its peak; this kernel is for the
// state that is as costly to compute as to move.)  The general kernel's arithmetic in the same order, with every access
// unguarded and W^T held in registers (VT^2 16-byte A operands per lane).
//
// The step reads each state element once, so at V = 64 it needs many bytes in
// flight per compute unit to keep HBM busy.  Each wave walks its (batch row,
// slab) sequence with two slabs ahead in flight, loaded straight into an LDS
// ring of two slots per wave (global_load_lds: no registers held while in
// flight): the slab's state tiles and, beside them, its rows' k and q, its
// unit's v and gate.  No load in the loop has a register destination, so the
// compiler inserts no wait there (it would wait for every ring load in
// flight); the ring is read with inline ds_read (each asm ends with its own
// wait), and each slot is awaited by an explicit vmcnt wait that counts only
// the operations issued after it, in a fixed order per iteration: the ring
// loads two slabs ahead, the VT state stores, at a unit's end its readout,
// pinned with scheduling barriers.
// The LDS offset of a pointer to shared memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// One 16-byte (4-byte) load per lane from global memory into LDS at
// dst + 16 lane (dst + 4 lane).
__device__ __forceinline__ void global_to_lds16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void global_to_lds4(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
}

template <typename InT, int VT>
__global__ void __launch_bounds__(256, 3) m2rnn_step_full_kernel(StepArgs a) {
  using R4 = f32x4;
  constexpr int VP = 16 * VT;
  constexpr bool kBf16 = std::is_same_v<InT, uint16_t>;
  constexpr int D = 2;                          // ring slots (slabs in flight) per wave
  constexpr int SIDE = VT * 1024;               // bytes: k, q, f, v blocks after the tiles
  constexpr int SLOT = SIDE + 1024;             // bytes per slot
  constexpr int RING = 4 * D * SLOT;            // the four waves' rings
  constexpr int WST = VT * VT * 1024;           // W^T staging (before the rings)
  __shared__ R4 lds[(RING > WST ? RING : WST) / 16];
  __shared__ float wrl[VP];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int64_t B = a.B, N = a.N, K = a.K, NQ = a.NQ;  // V = VP
  const int64_t n = (int64_t)blockIdx.x % N;
  const int64_t b0 = ((int64_t)blockIdx.x / N) * 4 * a.upw + w;

  // W^T of the head in MFMA A-operand order ([c][j][lane], as the general
  // kernel's), staged once, then held in registers
  const float* __restrict__ Wp = (const float*)a.W + n * VP * VP;
  for (int e = tid; e < VP * VP; e += 256) {
    const int l = e / VP, col = e % VP;
    const int m = l & 15;
    ((float*)&lds[((col >> 4) * VT + (l >> 4)) * 64 + 16 * acc_g<float>(m) + (col & 15)])
        [acc_r<float>(m)] = kTanhScale<float> * Wp[l * VP + col];
  }
  if (tid < VP) wrl[tid] = ((const float*)a.w_r)[n * VP + tid];
  __syncthreads();
  R4 wop[VT][VT];
#pragma unroll
  for (int c = 0; c < VT; ++c)
#pragma unroll
    for (int j = 0; j < VT; ++j) wop[c][j] = lds[(c * VT + j) * 64 + lane];
  __syncthreads();  // the staging area becomes the rings
  if (b0 >= B) return;

  const int64_t nq = n / (N / NQ);
  const int nslab = (int)(K / 16);
  const int64_t b_end = ((int64_t)blockIdx.x / N + 1) * 4 * a.upw < B
                            ? ((int64_t)blockIdx.x / N + 1) * 4 * a.upw
                            : B;
  // positions in the wave's sequence: batch row bb (b0, b0 + 4, ...), slab s
  struct Pos {
    int64_t bb;
    int s;
  };
  auto advance = [&](Pos p) -> Pos {
    if (p.s + 1 < nslab) return Pos{p.bb, p.s + 1};
    return Pos{p.bb + 4, 0};
  };
  // past the end, loads go to the last valid position (harmless re-reads)
  auto valid = [&](Pos p, Pos last) -> Pos { return p.bb < b_end ? p : last; };
  // this lane's state row (16 s + li, columns 16 j + 4 g .. + 3)
  auto hrow = [&](Pos p) -> float* {
    return (float*)a.H + ((p.bb * N + n) * K + p.s * 16 + li) * VP + 4 * g;
  };
  char* const ring = (char*)lds + w * D * SLOT;
  // dwords of a k (or q) slab and of a v row: lane l loads dword l mod their count
  constexpr int KDW = 16 * (int)sizeof(InT) / 4, VDW = VP * (int)sizeof(InT) / 4;
  // slab p into ring slot `slot`: VT state tiles, then k, q, the gate and v
  auto ring_load = [&](Pos p, int slot) {
    char* base = ring + slot * SLOT;
    const float* src = hrow(p);
#pragma unroll
    for (int j = 0; j < VT; ++j) global_to_lds16(src + 16 * j, base + j * 1024);
    const int64_t kq = (p.bb * NQ + nq) * K + p.s * 16;
    global_to_lds4((const uint32_t*)((const InT*)a.k + kq) + (lane % KDW), base + SIDE);
    global_to_lds4((const uint32_t*)((const InT*)a.q + kq) + (lane % KDW), base + SIDE + 256);
    global_to_lds4((const float*)a.f + p.bb * N + n, base + SIDE + 512);
    global_to_lds4((const uint32_t*)((const InT*)a.v + (p.bb * N + n) * VP) + (lane % VDW),
                     base + SIDE + 768);
  };
  // ring slot -> this lane's four state tiles, the k and q of its row and the
  // gate (raw 32-bit words), and, at a unit's first slab, its v at columns
  // 16 c + 4 g .. + 3: one asm of LDS reads that ends with their wait.  No
  // memory clobber: the compiler would take the asm for an LDS read and wait
  // for every ring load in flight; the order against the ring loads is kept by
  // the explicit waits and scheduling barriers.
  static_assert(VT == 4, "the ring kernel reads four tiles per slab");
  using VRaw = std::conditional_t<kBf16, uint2, R4>;
  auto ring_read = [&](int slot, R4 (&h)[VT], uint32_t& kr, uint32_t& qr, uint32_t& fr) {
    const char* base = ring + slot * SLOT;
    const uint32_t ah = lds_offset(base + 16 * lane);
    const uint32_t ak = lds_offset(base + SIDE + (kBf16 ? 2 : 4) * li);
    const uint32_t af = lds_offset(base + SIDE + 512);
    if constexpr (kBf16) {
      asm volatile(
          "ds_read_b128 %0, %7\n ds_read_b128 %1, %7 offset:1024\n"
          " ds_read_b128 %2, %7 offset:2048\n ds_read_b128 %3, %7 offset:3072\n"
          " ds_read_u16 %4, %8\n ds_read_u16 %5, %8 offset:256\n ds_read_b32 %6, %9\n"
          " s_waitcnt lgkmcnt(0)"
          : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]), "=&v"(kr), "=&v"(qr), "=&v"(fr)
          : "v"(ah), "v"(ak), "v"(af));
    } else {
      asm volatile(
          "ds_read_b128 %0, %7\n ds_read_b128 %1, %7 offset:1024\n"
          " ds_read_b128 %2, %7 offset:2048\n ds_read_b128 %3, %7 offset:3072\n"
          " ds_read_b32 %4, %8\n ds_read_b32 %5, %8 offset:256\n ds_read_b32 %6, %9\n"
          " s_waitcnt lgkmcnt(0)"
          : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]), "=&v"(kr), "=&v"(qr), "=&v"(fr)
          : "v"(ah), "v"(ak), "v"(af));
    }
  };
  auto v_read = [&](int slot, VRaw (&x)[VT]) {
    const uint32_t av = lds_offset(ring + slot * SLOT + SIDE + 768 + (kBf16 ? 8 : 16) * g);
    if constexpr (kBf16) {
      asm volatile("ds_read_b64 %0, %4\n ds_read_b64 %1, %4 offset:32\n"
                   " ds_read_b64 %2, %4 offset:64\n ds_read_b64 %3, %4 offset:96\n"
                   " s_waitcnt lgkmcnt(0)"
                   : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]) : "v"(av));
    } else {
      asm volatile("ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:64\n"
                   " ds_read_b128 %2, %4 offset:128\n ds_read_b128 %3, %4 offset:192\n"
                   " s_waitcnt lgkmcnt(0)"
                   : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]) : "v"(av));
    }
  };
  auto widen4 = [](VRaw x) -> R4 {
    if constexpr (kBf16) {
      return R4{__builtin_bit_cast(float, x.x << 16), __builtin_bit_cast(float, x.x & 0xffff0000u),
                __builtin_bit_cast(float, x.y << 16), __builtin_bit_cast(float, x.y & 0xffff0000u)};
    } else {
      return x;
    }
  };
  // w_r of this lane's readout columns, by the same route
  auto wr_read = [&](R4 (&x)[VT]) {
    const uint32_t ad = lds_offset(&wrl[4 * g]);
    asm volatile("ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:64\n"
                 " ds_read_b128 %2, %4 offset:128\n ds_read_b128 %3, %4 offset:192\n"
                 " s_waitcnt lgkmcnt(0)"
                 : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]) : "v"(ad));
  };

  // prologue: slabs 0 and 1 into slots 0 and 1
  Pos cur{b0, 0};
  Pos pr = valid(advance(cur), cur);  // the last ring load
  ring_load(cur, 0);
  ring_load(pr, 1);
  __builtin_amdgcn_sched_barrier(0);

  R4 yacc[VT], vv[VT];
#pragma unroll
  for (int c = 0; c < VT; ++c) yacc[c] = R4{0, 0, 0, 0};
  constexpr int kOps = VT + 4;  // memory operations of one ring load
  int slot = 0;
  for (int i = 0;; ++i) {
    // this slab's ring load is done once at most the ring loads and state
    // stores issued after it remain: one ring load in the first iteration, a
    // ring load and a slab's stores in the second, then a slab's stores, a
    // ring load and another slab's stores
    if (i == 0) {
      constexpr int m = kOps;
      __builtin_amdgcn_s_waitcnt((m & 15) | ((m >> 4) << 14) | (7 << 4) | (15 << 8));
    } else if (i == 1) {
      constexpr int m = kOps + VT;
      __builtin_amdgcn_s_waitcnt((m & 15) | ((m >> 4) << 14) | (7 << 4) | (15 << 8));
    } else {
      constexpr int m = kOps + 2 * VT;
      __builtin_amdgcn_s_waitcnt((m & 15) | ((m >> 4) << 14) | (7 << 4) | (15 << 8));
    }
    R4 h[VT];
    uint32_t kr, qr, fr;
    ring_read(slot, h, kr, qr, fr);
    if (cur.s == 0) {  // a unit's first slab: its v
      VRaw vx[VT];
      v_read(slot, vx);
#pragma unroll
      for (int c = 0; c < VT; ++c) vv[c] = widen4(vx[c]);
    }
    const float kk = __builtin_bit_cast(float, kBf16 ? kr << 16 : kr);
    const float qq = __builtin_bit_cast(float, kBf16 ? qr << 16 : qr);
    const float f = __builtin_bit_cast(float, fr);
    __builtin_amdgcn_sched_barrier(0);
    // the slab two ahead into the slot just read
    const Pos pn = valid(advance(pr), pr);
    ring_load(pn, slot);
    __builtin_amdgcn_sched_barrier(0);
    pr = pn;

    const float omf = 1.0f - f, m2omf = -2.0f * omf;
    const float ks = kTanhScale<float> * kk;
    float* dst = hrow(cur);
#pragma unroll
    for (int c = 0; c < VT; ++c) {
      R4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = ks * vv[c][r];
#pragma unroll
      for (int j = 0; j < VT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mfma_16x16x4(wop[c][j][r], h[j][r], acc);
      pin_vec(acc);
      R4 hn;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hn[r] = fma_r(m2omf, tanh_rc_scaled(acc[r]), fma_r(f, h[c][r], omf));
      *(R4*)(dst + 16 * c) = hn;
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[c][r] = fma_r(hn[r], qq, yacc[c][r]);
    }
    if (cur.s + 1 == nslab) {
      // y = H^T q + w_r (.) v of the finished unit, from lane 16 g of each row
      R4 ys[VT];
#pragma unroll
      for (int c = 0; c < VT; ++c) ys[c] = row16_sum_x4(yacc[c], 1.0f);
      if (li == 0) {
        float* yp = (float*)a.y + (cur.bb * N + n) * VP + 4 * g;
        R4 wr4[VT];
        wr_read(wr4);
#pragma unroll
        for (int c = 0; c < VT; ++c) {
          R4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = ys[c][r] + wr4[c][r] * vv[c][r];
          *(R4*)(yp + 16 * c) = o;
        }
      }
#pragma unroll
      for (int c = 0; c < VT; ++c) yacc[c] = R4{0, 0, 0, 0};
    }
    __builtin_amdgcn_sched_barrier(0);
    cur = advance(cur);
    if (cur.bb >= b_end) break;
    slot ^= 1;
  }
  // no ring load may still be writing LDS when the wave ends
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

template <typename InT, int VT>
static hipError_t launch_step_full(StepArgs a, hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> resident[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = kMaxDevices;
  int cap = dev < kMaxDevices ? resident[dev].load(std::memory_order_relaxed) : 0;
  if (cap <= 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, m2rnn_step_full_kernel<InT, VT>, 256,
                                                     0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      per_cu = 4;
      cus = 256;
    }
    cap = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    if (dev < kMaxDevices) resident[dev].store(cap, std::memory_order_relaxed);
  }
  const int64_t groups = (a.B + 3) / 4;
  int64_t upw = (a.N * groups + cap - 1) / cap;
  if (upw < 1) upw = 1;
  a.upw = upw;
  const int64_t wgs = a.N * ((groups + upw - 1) / upw);
  hipLaunchKernelGGL((m2rnn_step_full_kernel<InT, VT>), dim3((unsigned)wgs), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

template <typename InT, typename Real, int VT>
static hipError_t launch_step_vt(StepArgs a, hipStream_t stream) {
  static_assert(sizeof(typename Vec4<Real>::type) * VT * VT * 64 <= 160 * 1024, "LDS budget");
  // Workgroups the device holds at once (occupancy x compute units), per
  // device, found once.  Each wave takes enough units that the grid fits in
  // one round, so every workgroup stages W once for several batch rows.  The
  // cache is atomic: host threads may call concurrently, and all of them
  // compute and store the same value.
  constexpr int kMaxDevices = 64;
  static std::atomic<int> resident[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = kMaxDevices;
  int cap = dev < kMaxDevices ? resident[dev].load(std::memory_order_relaxed) : 0;
  if (cap <= 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, m2rnn_step_kernel<InT, Real, VT>,
                                                     256, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      per_cu = 4;
      cus = 256;
    }
    cap = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    if (dev < kMaxDevices) resident[dev].store(cap, std::memory_order_relaxed);
  }
  const int64_t groups = (a.B + 3) / 4;  // groups of four batch rows per head
  int64_t upw = (a.N * groups + cap - 1) / cap;
  if (upw < 1) upw = 1;
  a.upw = upw;
  const int64_t wgs = a.N * ((groups + upw - 1) / upw);
  hipLaunchKernelGGL((m2rnn_step_kernel<InT, Real, VT>), dim3((unsigned)wgs), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

template <typename InT, typename Real>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t stream) {
  if constexpr (std::is_same_v<Real, float>) {
    if (a.full) return launch_step_full<InT, 4>(a, stream);
  }
  switch (value_tiles(a.V)) {
    case 1: return launch_step_vt<InT, Real, 1>(a, stream);
    case 2: return launch_step_vt<InT, Real, 2>(a, stream);
    case 3: return launch_step_vt<InT, Real, 3>(a, stream);
    case 4: return launch_step_vt<InT, Real, 4>(a, stream);
    case 6: return launch_step_vt<InT, Real, 6>(a, stream);
    case 8: return launch_step_vt<InT, Real, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_step(const StepArgs& a, int in_dtype, int state_dtype, hipStream_t stream) {
  if (state_dtype == kF32) {
    if (in_dtype == kF32) return launch_step_t<float, float>(a, stream);
    if (in_dtype == kBF16) return launch_step_t<uint16_t, float>(a, stream);
  } else if (state_dtype == kF64) {
    if (in_dtype == kF64) return launch_step_t<double, double>(a, stream);
    if (in_dtype == kBF16) return launch_step_t<uint16_t, double>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace m2rnn
