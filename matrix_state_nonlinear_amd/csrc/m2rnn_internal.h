// Host-side interface between the C ABI (m2rnn_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m2rnn {

enum : int { kF32 = 0, kBF16 = 1, kF64 = 2 };
enum : int { kGateSigmoid = 0, kGateExpSoftplus = 1 };

// Rows of the K x V state handled by one workgroup.  The K rows of a head are
// independent recurrences that share W (W only mixes value columns), so a
// head splits into ceil(K / 16) slabs that run on different compute units.
constexpr int kSlabRows = 16;

inline int64_t num_slabs(int64_t K) { return (K + kSlabRows - 1) / kSlabRows; }

// Largest value width V the kernels take, in 16-column tiles.
constexpr int kMaxValueTiles = 8;

// Value columns padded to the kernels' tile count (multiples of 16, with the
// tile counts 5 and 7 rounded up to 6 and 8 so waves split them evenly).
inline int value_tiles(int64_t V) {
  int vt = (int)((V + 15) / 16);
  if (vt == 5) vt = 6;
  if (vt == 7) vt = 8;
  return vt;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct FwdArgs {
  const void* k;
  const void* v;
  const void* q;
  const void* f;
  const void* W;
  const void* w_r;
  const void* H0;    // may be null
  void* y;
  void* ypart;       // [nslab, B, T, N, V] partial readouts when nslab > 1
  void* HT;          // may be null
  void* ckpt;        // may be null
  void* rc;          // [B, N, T, K, V] per-step 1 / (1 + e^{2A}), or null
  int64_t B, T, N, K, V, C;
  int64_t NQ;        // heads of q and k; value head n reads q/k head n / (N / NQ)
  int nslab;
  int st_vec;        // fp32, V % 4 == 0 and ckpt, HT, rc 16-byte aligned: 16-byte state stores
};

struct BwdArgs {
  const void* k;
  const void* v;
  const void* q;
  const void* logit;
  const void* alpha;
  const void* beta;
  const void* f;
  const void* W;
  const void* w_r;
  const void* H0;    // may be null
  const void* ckpt;
  const void* rc;    // [B, N, T, K, V] from the forward, or null (recompute)
  const void* dy;
  const void* dHT;   // may be null
  void* dk;
  void* dv;
  void* dq;
  void* dlogit;
  void* dW;
  void* dw_r;
  void* dalpha;      // may be null
  void* dbeta;       // may be null
  void* dH0;         // may be null
  void* ws;          // workspace base
  // Chunk-start states of the reverse sweep, [B, N, cks_count, K, V]: chunk c
  // (steps [cS, cS + S)) starts from entry c * cks_step.  Either the forward's
  // checkpoints (when C divides S) or states recomputed into the workspace.
  const void* cks;
  int64_t cks_count, cks_step;
  // Interval sweep (BwdWorkspace::sweep): per unit, two checkpoint intervals of
  // states S_{t+1} (ring_s) and, when the states are recomputed, rc_t (ring_r),
  // each [2][C][ceil(V / 16) tiles][64 lanes][4] in the kernels' register layout.
  void* ring_s;
  void* ring_r;
  int64_t B, T, N, K, V, C;
  int64_t NQ;        // heads of q and k; value head n reads q/k head n / (N / NQ)
  int nslab;
  int gate_kind;
  int rc_vec;        // fp32, V % 4 == 0 and rc 16-byte aligned: 16-byte rc loads
  int dv_vec;        // fp32, V % 4 == 0 and the dv destination 16-byte aligned: 16-byte stores
};

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Workspace layout of the backward: offsets in elements of the state type,
// each region aligned to 64 elements.
struct BwdWorkspace {
  int period;         // S: steps per chunk of the reverse sweep (depends on V and dtype)
  int64_t nch;        // ceil(T / S)
  bool subck_needed;  // C does not divide S: chunk starts are recomputed first
  bool sweep;         // the main kernel sweeps each checkpoint interval itself instead
                      // (C a multiple of S, larger, and at most kMaxSweepInterval)
  size_t subck;       // [B, N, nch, K, V] chunk-start states (subck_needed only)
  size_t ring_s;      // [units, 2, C, 16 VP] states of two intervals (sweep only)
  size_t ring_r;      // [units, 2, C, 16 VP] rc of two intervals (sweep, recomputing only)
  size_t dv_part;     // [nslab, B, T, N, V]  (nslab > 1 only)
  size_t df_part;     // [nslab, B, T, N]
  size_t dW_part;     // [B * nslab, N, V, V]
  size_t col_part;    // [row_blocks, N, V + 2] column-sum partials (dw_r, dalpha, dbeta)
  size_t dk_part;     // [B, T, N, K] per-value-head dk (NQ < N only; summed over groups)
  size_t dq_part;     // [B, T, N, K] per-value-head dq (NQ < N only)
  int64_t row_blocks;
  size_t total_elems;
};
// Checkpoint intervals up to this length are swept inside the backward's main
// kernel (two intervals of states per 16-row slab in the workspace); longer
// ones get their chunk starts from a separate recomputing pass.
constexpr int64_t kMaxSweepInterval = 1024;

BwdWorkspace bwd_workspace_layout(int64_t B, int64_t T, int64_t N, int64_t NQ, int64_t K,
                                  int64_t V, int64_t C, int state_dtype, bool stored_rc);

struct StepArgs {
  const void* k;     // [B, NQ, K]
  const void* v;     // [B, N, V]
  const void* q;     // [B, NQ, K]
  const void* f;     // [B, N]
  const void* W;
  const void* w_r;
  void* H;           // [B, N, K, V], updated in place
  void* y;           // [B, N, V]
  int64_t B, N, NQ, K, V;
  int vec;           // fp32 state, V % 4 == 0 and H 16-byte aligned: 16-byte state accesses
  int full;          // fp32 state, K % 16 == 0, V = 64, H and y 16-byte aligned, k, q, v, f
                     // 4-byte aligned: the full-tile kernel with its LDS ring
  int64_t upw;       // batch rows (units) per wave, set by the launcher
};

// Block prologue (causal conv + SiLU) and epilogue (gate + RMSNorm).
struct BlockConvArgs {
  int64_t B, T, C;
  const void* x;     // [B, T, C] io dtype
  const void* w;     // [C, 4]
  const void* bias;  // [C] or null
  void* out;         // [B, T, C] io dtype (forward)
  const void* dout;  // [B, T, C] (backward)
  void* dx;          // [B, T, C] (backward)
  void* dw;          // [C, 4] (backward)
  void* dbias;       // [C] or null (backward)
  void* ws;          // backward partials
};
struct BlockNormArgs {
  int64_t rows, D;
  double eps;
  const void* y;      // [rows, D]
  const void* g_pre;  // [rows, D] io dtype
  const void* gamma;  // [D]
  void* out;          // [rows, D] io dtype (forward)
  const void* dout;   // [rows, D] (backward)
  void* dy;           // (backward)
  void* dg_pre;       // (backward)
  void* dgamma;       // [D] (backward)
  void* ws;           // backward: per-row 1/rms and dgamma partials
};
size_t conv_bwd_workspace_elems(int64_t B, int64_t T, int64_t C);
size_t rmsnorm_bwd_workspace_elems(int64_t rows, int64_t D);
hipError_t launch_conv_silu(const BlockConvArgs& a, int io_dtype, int param_dtype, bool bwd,
                            hipStream_t stream);
hipError_t launch_gate_rmsnorm(const BlockNormArgs& a, int io_dtype, int param_dtype, bool bwd,
                               hipStream_t stream);

hipError_t launch_gates(int64_t B, int64_t T, int64_t N, int gate_kind, int dtype,
                        const void* logit, const void* alpha, const void* beta, void* f,
                        hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, int in_dtype, int state_dtype, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int in_dtype, int state_dtype, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, int in_dtype, int state_dtype, hipStream_t stream);

}  // namespace m2rnn
