// C ABI of libm2rnn.so: argument checks, workspace sizing, kernel dispatch.
// Declarations and the contract of every entry point are in include/m2rnn.h.

#include <limits.h>

#include <atomic>

#include "../../include/m2rnn.h"
#include "m2rnn_internal.h"
#include "m2rnn_newton_internal.h"

using namespace m2rnn;

namespace {

// B, T or n_heads may be 0 (an empty batch or sequence: nothing to recompute;
// the per-head and state outputs still get their values); K and V may not.
bool sizes_ok(int64_t B, int64_t T, int64_t N, int64_t K, int64_t V) {
  if (B < 0 || T < 0 || N < 0 || K < 1 || V < 1) return false;
  // every element count the kernels index must stay far from int64 overflow
  const double elems = (double)B * (double)T * (double)N * (double)(K > V ? K : V);
  return elems < 4.0e18;
}

// q and k have NQ heads shared by groups of N / NQ value heads: NQ divides N
// (NQ = N is one q/k head per value head); with no heads both are 0.
bool qk_heads_ok(int64_t N, int64_t NQ) {
  return N > 0 ? (NQ >= 1 && NQ <= N && N % NQ == 0) : NQ == 0;
}

bool sizes_supported(int64_t B, int64_t T, int64_t N, int64_t K, int64_t V) {
  if (K > 256 || V > 128) return false;
  if (T >= ((int64_t)1 << 30)) return false;  // step indices are 32-bit in the kernels
  // one workgroup (at most 1024 threads) per slab: the grid stays below 2^32 threads
  return (double)B * (double)N * (double)num_slabs(K) < (double)(1 << 22);
}

// The block kernels' one-dimensional grids: at most (tokens / 16 + B) x
// ceil(C / 256) and tokens / 4 workgroups, below 2^31.
bool block_grid_ok(int64_t B, int64_t T, int64_t C) {
  const double tok = (double)B * (double)T;
  const double cb = (double)((C + 255) / 256);
  return (tok / 16.0 + (double)B) * cb < 2147483647.0 && tok / 4.0 < 2147483647.0 &&
         C < ((int64_t)1 << 40);
}

size_t real_size(int state_dtype) { return state_dtype == M2RNN_F64 ? 8 : 4; }

bool dtypes_ok(int in_dtype, int state_dtype) {
  if (state_dtype == M2RNN_F32) return in_dtype == M2RNN_F32 || in_dtype == M2RNN_BF16;
  if (state_dtype == M2RNN_F64) return in_dtype == M2RNN_F64 || in_dtype == M2RNN_BF16;
  return false;
}

bool state_dtype_known(int state_dtype) {
  return state_dtype == M2RNN_F32 || state_dtype == M2RNN_F64;
}

bool in_dtype_known(int in_dtype) {
  return in_dtype == M2RNN_F32 || in_dtype == M2RNN_BF16 || in_dtype == M2RNN_F64;
}

size_t fwd_ws_bytes(int64_t B, int64_t T, int64_t N, int64_t K, int64_t V, int state_dtype) {
  const int64_t ns = num_slabs(K);
  if (ns <= 1) return 0;
  return align_up((size_t)ns * (size_t)B * (size_t)T * (size_t)N * (size_t)V *
                      real_size(state_dtype),
                  256);
}

// The larger of the two backward modes' layouts (recomputing needs the rc ring
// as well when the main kernel sweeps the intervals), so one size serves both.
size_t bwd_ws_bytes(int64_t B, int64_t T, int64_t N, int64_t NQ, int64_t K, int64_t V,
                    int64_t C, int state_dtype) {
  const BwdWorkspace L = bwd_workspace_layout(B, T, N, NQ, K, V, C, state_dtype, false);
  return align_up(L.total_elems * real_size(state_dtype), 256);
}

int status_of(hipError_t e) { return e == hipSuccess ? M2RNN_OK : M2RNN_ERR_HIP; }

// dst[0..n) = src[0..n), or zeros when src is NULL (outputs of empty calls)
template <typename Real>
__global__ void __launch_bounds__(256) fill_kernel(Real* __restrict__ dst,
                                                   const Real* __restrict__ src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : Real(0);
}

hipError_t fill(void* dst, const void* src, int64_t n, int state_dtype, hipStream_t stream) {
  if (!dst || n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (state_dtype == M2RNN_F64)
    hipLaunchKernelGGL(fill_kernel<double>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (double*)dst, (const double*)src, n);
  else
    hipLaunchKernelGGL(fill_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (float*)dst, (const float*)src, n);
  return hipGetLastError();
}

// The Newton forward's shapes: V a multiple of 16 up to 64, and wave counts of
// its kernels within 32-bit wave indices.
bool newton_supported(int64_t B, int64_t T, int64_t N, int64_t K, int64_t V) {
  if (!(V == 16 || V == 32 || V == 48 || V == 64) || K > 256 || T >= ((int64_t)1 << 30))
    return false;
  if (B * T * N == 0) return true;
  const NewtonLayout L = newton_layout(B, T, N, K, V, true);
  const double U = (double)B * (double)N;
  const double waves = U * (double)num_slabs(K) * (double)L.NTB;
  const double map_waves = U * (double)L.P * (double)K * (double)(V / 16);
  return waves < 2.0e9 && map_waves < 2.0e9 && U * (double)T * (double)K * (double)V < 4.0e18;
}

// The argument checks of m2rnn_bwd and m2rnn_bwd_noalloc, before any
// workspace: M2RNN_OK or the status to return.
int bwd_check(int64_t B, int64_t T, int64_t n_heads, int64_t qk_heads, int64_t K, int64_t V,
              int in_dtype, int state_dtype, const void* k, const void* v, const void* q,
              int gate_kind, const void* logit, const void* alpha, const void* beta,
              const void* f, const void* W, const void* w_r, const void* ckpt, int64_t C,
              const void* dy, const void* dk, const void* dv, const void* dq, const void* dlogit,
              const void* dW, const void* dw_r, const void* dalpha, const void* dbeta) {
  if (!sizes_ok(B, T, n_heads, K, V) || !qk_heads_ok(n_heads, qk_heads))
    return M2RNN_ERR_INVALID_ARG;
  if (!in_dtype_known(in_dtype) || !state_dtype_known(state_dtype)) return M2RNN_ERR_INVALID_ARG;
  const bool empty = B * T * n_heads == 0;
  const bool heads = n_heads > 0;  // per-head outputs exist
  if (!empty && (!k || !v || !q || !logit || !f || !W || !w_r || !ckpt || !dy))
    return M2RNN_ERR_INVALID_ARG;
  if (!empty && (!dk || !dv || !dq || !dlogit)) return M2RNN_ERR_INVALID_ARG;
  if (heads && (!dW || !dw_r)) return M2RNN_ERR_INVALID_ARG;
  if (C < 1) return M2RNN_ERR_INVALID_ARG;
  if (gate_kind == M2RNN_GATE_SIGMOID) {
    if (alpha || beta || dalpha || dbeta) return M2RNN_ERR_INVALID_ARG;
  } else if (gate_kind == M2RNN_GATE_EXP_SOFTPLUS) {
    if (heads && (!dalpha || !dbeta)) return M2RNN_ERR_INVALID_ARG;
    if (!empty && (!alpha || !beta)) return M2RNN_ERR_INVALID_ARG;
  } else {
    return M2RNN_ERR_INVALID_ARG;
  }
  if (!sizes_supported(B, T, n_heads, K, V) || !dtypes_ok(in_dtype, state_dtype))
    return M2RNN_ERR_UNSUPPORTED;
  return M2RNN_OK;
}

// Workspace of m2rnn_bwd_noalloc: one fixed array per device, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it names a stand-in): the device address comes from
// hipGetSymbolAddress, once per device, and is passed to the kernels like any
// workspace.
constexpr size_t kScratchBytes = M2RNN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) __attribute__((used)) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::atomic<void*> scratch_ptr[kScratchDevices];

// Device address of `scratch` on device `dev` (the current device), looked
// up on the first call there.  Concurrent first calls look it up alike and
// store the same address.
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* m2rnn_status_string(int status) {
  switch (status) {
    case M2RNN_OK: return "M2RNN_OK";
    case M2RNN_ERR_INVALID_ARG: return "M2RNN_ERR_INVALID_ARG: invalid size, pointer or enum";
    case M2RNN_ERR_UNSUPPORTED: return "M2RNN_ERR_UNSUPPORTED: K > 256, V > 128 or dtype pairing";
    case M2RNN_ERR_WORKSPACE: return "M2RNN_ERR_WORKSPACE: workspace missing or too small";
    case M2RNN_ERR_HIP: return "M2RNN_ERR_HIP: kernel launch failed";
    case M2RNN_ERR_SCRATCH:
      return "M2RNN_ERR_SCRATCH: the call needs more workspace than the static scratch holds";
    default: return "M2RNN: unknown status";
  }
}

size_t m2rnn_workspace_bytes(int is_bwd, int64_t B, int64_t T, int64_t n_heads,
                             int64_t qk_heads, int64_t K, int64_t V, int64_t C,
                             int state_dtype) {
  if (!sizes_ok(B, T, n_heads, K, V) || !sizes_supported(B, T, n_heads, K, V) ||
      !qk_heads_ok(n_heads, qk_heads) || !state_dtype_known(state_dtype) || (is_bwd && C < 1))
    return 0;
  if (B * T * n_heads == 0) return 0;  // empty calls run no kernel that needs one
  return is_bwd ? bwd_ws_bytes(B, T, n_heads, qk_heads, K, V, C, state_dtype)
                : fwd_ws_bytes(B, T, n_heads, K, V, state_dtype);
}

int m2rnn_gates(int64_t B, int64_t T, int64_t n_heads, int gate_kind, int dtype,
                const void* logit, const void* alpha, const void* beta, void* f, void* stream) {
  if (B < 0 || T < 0 || n_heads < 0) return M2RNN_ERR_INVALID_ARG;
  if (dtype != M2RNN_F32 && dtype != M2RNN_F64) return M2RNN_ERR_INVALID_ARG;
  const bool empty = B * T * n_heads == 0;
  if (!empty && (!logit || !f)) return M2RNN_ERR_INVALID_ARG;
  if (gate_kind == M2RNN_GATE_SIGMOID) {
    if (alpha || beta) return M2RNN_ERR_INVALID_ARG;
  } else if (gate_kind == M2RNN_GATE_EXP_SOFTPLUS) {
    if (!empty && (!alpha || !beta)) return M2RNN_ERR_INVALID_ARG;
  } else {
    return M2RNN_ERR_INVALID_ARG;
  }
  if (empty) return M2RNN_OK;
  return status_of(launch_gates(B, T, n_heads, gate_kind, dtype, logit, alpha, beta, f,
                                (hipStream_t)stream));
}

int m2rnn_fwd(int64_t B, int64_t T, int64_t n_heads, int64_t qk_heads, int64_t K, int64_t V,
              int in_dtype, int state_dtype, const void* k, const void* v, const void* q,
              const void* f, const void* W, const void* w_r, const void* H0, void* y, void* HT,
              void* ckpt, int64_t C, void* rc, void* workspace, size_t workspace_bytes,
              void* stream) {
  if (!sizes_ok(B, T, n_heads, K, V) || !qk_heads_ok(n_heads, qk_heads))
    return M2RNN_ERR_INVALID_ARG;
  if (!in_dtype_known(in_dtype) || !state_dtype_known(state_dtype)) return M2RNN_ERR_INVALID_ARG;
  const bool empty = B * T * n_heads == 0;
  if (!empty && (!k || !v || !q || !f || !W || !w_r || !y)) return M2RNN_ERR_INVALID_ARG;
  if (ckpt && C < 1) return M2RNN_ERR_INVALID_ARG;
  if (!sizes_supported(B, T, n_heads, K, V) || !dtypes_ok(in_dtype, state_dtype))
    return M2RNN_ERR_UNSUPPORTED;
  if (empty)  // no step: H_T = H_0 (zero when NULL); y and the checkpoints are empty
    return status_of(fill(HT, H0, B * n_heads * K * V, state_dtype, (hipStream_t)stream));
  const size_t need = fwd_ws_bytes(B, T, n_heads, K, V, state_dtype);
  if (need && (!workspace || workspace_bytes < need)) return M2RNN_ERR_WORKSPACE;
  FwdArgs a{};
  a.k = k; a.v = v; a.q = q; a.f = f; a.W = W; a.w_r = w_r; a.H0 = H0;
  a.y = y; a.ypart = workspace; a.HT = HT; a.ckpt = ckpt; a.rc = rc;
  a.B = B; a.T = T; a.N = n_heads; a.K = K; a.V = V; a.C = ckpt ? C : 1;
  a.NQ = qk_heads;
  a.nslab = (int)num_slabs(K);
  return status_of(launch_fwd(a, in_dtype, state_dtype, (hipStream_t)stream));
}

int m2rnn_bwd(int64_t B, int64_t T, int64_t n_heads, int64_t qk_heads, int64_t K, int64_t V,
              int in_dtype, int state_dtype, const void* k, const void* v, const void* q,
              int gate_kind, const void* logit, const void* alpha, const void* beta,
              const void* f, const void* W, const void* w_r, const void* H0, const void* ckpt,
              int64_t C, const void* rc, const void* dy, const void* dHT, void* dk, void* dv,
              void* dq,
              void* dlogit, void* dW, void* dw_r, void* dalpha, void* dbeta, void* dH0,
              void* workspace, size_t workspace_bytes, void* stream) {
  const int chk = bwd_check(B, T, n_heads, qk_heads, K, V, in_dtype, state_dtype, k, v, q,
                            gate_kind, logit, alpha, beta, f, W, w_r, ckpt, C, dy, dk, dv, dq,
                            dlogit, dW, dw_r, dalpha, dbeta);
  if (chk != M2RNN_OK) return chk;
  const bool empty = B * T * n_heads == 0;
  if (empty) {
    // no step: dH_0 = dH_T (zero when NULL); dW, dw_r (and dalpha, dbeta) are
    // sums over no tokens; the per-token gradients are empty
    const hipStream_t st = (hipStream_t)stream;
    hipError_t e = fill(dH0, dHT, B * n_heads * K * V, state_dtype, st);
    if (e == hipSuccess) e = fill(dW, nullptr, n_heads * V * V, state_dtype, st);
    if (e == hipSuccess) e = fill(dw_r, nullptr, n_heads * V, state_dtype, st);
    if (e == hipSuccess) e = fill(dalpha, nullptr, n_heads, state_dtype, st);
    if (e == hipSuccess) e = fill(dbeta, nullptr, n_heads, state_dtype, st);
    return status_of(e);
  }
  const size_t need = bwd_ws_bytes(B, T, n_heads, qk_heads, K, V, C, state_dtype);
  if (need && (!workspace || workspace_bytes < need)) return M2RNN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return M2RNN_ERR_INVALID_ARG;
  BwdArgs a{};
  a.k = k; a.v = v; a.q = q; a.logit = logit; a.alpha = alpha; a.beta = beta; a.f = f;
  a.W = W; a.w_r = w_r; a.H0 = H0; a.ckpt = ckpt; a.rc = rc; a.dy = dy; a.dHT = dHT;
  a.dk = dk; a.dv = dv; a.dq = dq; a.dlogit = dlogit; a.dW = dW; a.dw_r = dw_r;
  a.dalpha = dalpha; a.dbeta = dbeta; a.dH0 = dH0; a.ws = workspace;
  a.B = B; a.T = T; a.N = n_heads; a.K = K; a.V = V; a.C = C;
  a.NQ = qk_heads;
  a.nslab = (int)num_slabs(K);
  a.gate_kind = gate_kind;
  return status_of(launch_bwd(a, in_dtype, state_dtype, (hipStream_t)stream));
}

int m2rnn_bwd_noalloc(int64_t B, int64_t T, int64_t n_heads, int64_t qk_heads, int64_t K,
                      int64_t V, int in_dtype, int state_dtype, const void* k, const void* v,
                      const void* q, int gate_kind, const void* logit, const void* alpha,
                      const void* beta, const void* f, const void* W, const void* w_r,
                      const void* H0, const void* ckpt, int64_t C, const void* rc,
                      const void* dy, const void* dHT, void* dk, void* dv, void* dq,
                      void* dlogit, void* dW, void* dw_r, void* dalpha, void* dbeta, void* dH0,
                      void* stream) {
  const int chk = bwd_check(B, T, n_heads, qk_heads, K, V, in_dtype, state_dtype, k, v, q,
                            gate_kind, logit, alpha, beta, f, W, w_r, ckpt, C, dy, dk, dv, dq,
                            dlogit, dW, dw_r, dalpha, dbeta);
  if (chk != M2RNN_OK) return chk;
  const size_t need = bwd_ws_bytes(B, T, n_heads, qk_heads, K, V, C, state_dtype);
  if (B * T * n_heads != 0 && need > kScratchBytes) return M2RNN_ERR_SCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return M2RNN_ERR_HIP;
  if (stream) {  // the scratch address is the current device's
    int sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return M2RNN_ERR_HIP;
    if (sdev != dev) return M2RNN_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  if (scratch_address(dev, &ws) != hipSuccess) return M2RNN_ERR_HIP;
  return m2rnn_bwd(B, T, n_heads, qk_heads, K, V, in_dtype, state_dtype, k, v, q, gate_kind,
                   logit, alpha, beta, f, W, w_r, H0, ckpt, C, rc, dy, dHT, dk, dv, dq, dlogit,
                   dW, dw_r, dalpha, dbeta, dH0, ws, kScratchBytes, stream);
}

size_t m2rnn_newton_workspace_bytes(int64_t B, int64_t T, int64_t n_heads, int64_t K, int64_t V,
                                    int states_given) {
  if (!sizes_ok(B, T, n_heads, K, V) || !newton_supported(B, T, n_heads, K, V)) return 0;
  if (B * T * n_heads == 0) return 0;
  return align_up(newton_layout(B, T, n_heads, K, V, states_given != 0).total_floats * 4, 256);
}

int m2rnn_newton_fwd(int64_t B, int64_t T, int64_t n_heads, int64_t qk_heads, int64_t K,
                     int64_t V, int in_dtype, const void* k, const void* v, const void* q,
                     const void* f, const void* W, const void* w_r, const void* H0, int iters,
                     void* y, void* HT, void* states, void* residual, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!sizes_ok(B, T, n_heads, K, V) || !qk_heads_ok(n_heads, qk_heads))
    return M2RNN_ERR_INVALID_ARG;
  if (in_dtype != M2RNN_F32 && in_dtype != M2RNN_BF16) {
    return in_dtype_known(in_dtype) ? M2RNN_ERR_UNSUPPORTED : M2RNN_ERR_INVALID_ARG;
  }
  if (iters < 0 || iters > 64) return M2RNN_ERR_INVALID_ARG;
  const bool empty = B * T * n_heads == 0;
  if (!empty && (!k || !v || !q || !f || !W || !w_r || !y)) return M2RNN_ERR_INVALID_ARG;
  if (!aligned16(v) || !aligned16(H0) || !aligned16(y) || !aligned16(HT) || !aligned16(states) ||
      !aligned16(workspace))
    return M2RNN_ERR_INVALID_ARG;
  if (!newton_supported(B, T, n_heads, K, V)) return M2RNN_ERR_UNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  if (empty) {
    hipError_t e = fill(HT, H0, B * n_heads * K * V, M2RNN_F32, st);
    if (e == hipSuccess) e = fill(residual, nullptr, iters + 1, M2RNN_F32, st);
    return status_of(e);
  }
  const NewtonLayout L = newton_layout(B, T, n_heads, K, V, states != nullptr);
  const size_t need = align_up(L.total_floats * 4, 256);
  if (!workspace || workspace_bytes < need) return M2RNN_ERR_WORKSPACE;
  float* ws = (float*)workspace;
  NewtonArgs a{};
  a.k = k; a.v = v; a.q = q;
  a.f = (const float*)f; a.W = (const float*)W; a.w_r = (const float*)w_r;
  a.H0 = (const float*)H0;
  a.y = (float*)y; a.HT = (float*)HT;
  a.X = states ? (float*)states : ws + L.X;
  a.Xn = ws + L.X2;
  a.S = ws + L.S; a.R = ws + L.R;
  a.M = ws + L.M; a.E = ws + L.E; a.D = ws + L.D;
  a.res = (unsigned*)residual;
  a.B = B; a.T = T; a.N = n_heads; a.NQ = qk_heads; a.K = K; a.V = V;
  a.iters = iters;
  a.L = L.L; a.P = L.P; a.TL = L.TL; a.NTB = L.NTB;
  return status_of(launch_newton(a, in_dtype, st));
}

int m2rnn_step(int64_t B, int64_t n_heads, int64_t qk_heads, int64_t K, int64_t V, int in_dtype,
               int state_dtype, const void* k, const void* v, const void* q, const void* f,
               const void* W, const void* w_r, void* H, void* y, void* stream) {
  if (!sizes_ok(B, 1, n_heads, K, V) || !qk_heads_ok(n_heads, qk_heads))
    return M2RNN_ERR_INVALID_ARG;
  if (!in_dtype_known(in_dtype) || !state_dtype_known(state_dtype)) return M2RNN_ERR_INVALID_ARG;
  const bool empty = B * n_heads == 0;
  if (!empty && (!k || !v || !q || !f || !W || !w_r || !H || !y)) return M2RNN_ERR_INVALID_ARG;
  // one workgroup per head and group of four batch rows
  if (K > 256 || V > 128 || (double)n_heads * (double)((B + 3) / 4) >= 2147483648.0 ||
      !dtypes_ok(in_dtype, state_dtype))
    return M2RNN_ERR_UNSUPPORTED;
  if (empty) return M2RNN_OK;  // no unit: nothing is read or written
  StepArgs a{};
  a.k = k; a.v = v; a.q = q; a.f = f; a.W = W; a.w_r = w_r; a.H = H; a.y = y;
  a.B = B; a.N = n_heads; a.NQ = qk_heads; a.K = K; a.V = V;
  a.vec = state_dtype == M2RNN_F32 && (V & 3) == 0 && ((uintptr_t)H & 15) == 0;
  a.full = a.vec && K % 16 == 0 && V == 64 && ((uintptr_t)y & 15) == 0 &&
           ((uintptr_t)v & 3) == 0 && ((uintptr_t)k & 3) == 0 && ((uintptr_t)q & 3) == 0 &&
           ((uintptr_t)f & 3) == 0;
  return status_of(launch_step(a, in_dtype, state_dtype, (hipStream_t)stream));
}

size_t m2rnn_block_workspace_bytes(int op, int64_t B, int64_t T, int64_t C, int param_dtype) {
  if (B < 0 || T < 0 || C < 1 || !state_dtype_known(param_dtype)) return 0;
  if (B * T == 0) return 0;
  size_t elems;
  if (op == 0) elems = conv_bwd_workspace_elems(B, T, C);
  else if (op == 1) elems = rmsnorm_bwd_workspace_elems(B * T, C);
  else return 0;
  return align_up(elems * real_size(param_dtype), 256);
}

int m2rnn_conv_silu(int64_t B, int64_t T, int64_t C, int io_dtype, int param_dtype,
                    const void* x, const void* w, const void* bias, void* out, void* stream) {
  if (B < 0 || T < 0 || C < 1 || !in_dtype_known(io_dtype) || !state_dtype_known(param_dtype))
    return M2RNN_ERR_INVALID_ARG;
  const bool empty = B * T == 0;
  if (!empty && (!x || !w || !out)) return M2RNN_ERR_INVALID_ARG;
  if (!dtypes_ok(io_dtype, param_dtype) || !block_grid_ok(B, T, C)) return M2RNN_ERR_UNSUPPORTED;
  if (empty) return M2RNN_OK;
  BlockConvArgs a{};
  a.B = B; a.T = T; a.C = C; a.x = x; a.w = w; a.bias = bias; a.out = out;
  return status_of(launch_conv_silu(a, io_dtype, param_dtype, false, (hipStream_t)stream));
}

int m2rnn_conv_silu_bwd(int64_t B, int64_t T, int64_t C, int io_dtype, int param_dtype,
                        const void* x, const void* w, const void* bias, const void* dout, void* dx,
                        void* dw, void* dbias, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (B < 0 || T < 0 || C < 1 || !in_dtype_known(io_dtype) || !state_dtype_known(param_dtype))
    return M2RNN_ERR_INVALID_ARG;
  const bool empty = B * T == 0;
  if (!w || !dw || (bias == nullptr) != (dbias == nullptr)) return M2RNN_ERR_INVALID_ARG;
  if (!empty && (!x || !dout || !dx)) return M2RNN_ERR_INVALID_ARG;
  if (!dtypes_ok(io_dtype, param_dtype) || !block_grid_ok(B, T, C)) return M2RNN_ERR_UNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  if (empty) {  // sums over no tokens
    hipError_t e = fill(dw, nullptr, C * 4, param_dtype, st);
    if (e == hipSuccess) e = fill(dbias, nullptr, C, param_dtype, st);
    return status_of(e);
  }
  const size_t need = m2rnn_block_workspace_bytes(0, B, T, C, param_dtype);
  if (!workspace || workspace_bytes < need) return M2RNN_ERR_WORKSPACE;
  BlockConvArgs a{};
  a.B = B; a.T = T; a.C = C; a.x = x; a.w = w; a.bias = bias; a.dout = dout; a.dx = dx;
  a.dw = dw; a.dbias = dbias; a.ws = workspace;
  return status_of(launch_conv_silu(a, io_dtype, param_dtype, true, st));
}

int m2rnn_gate_rmsnorm(int64_t rows, int64_t D, int io_dtype, int param_dtype, double eps,
                       const void* y, const void* g_pre, const void* gamma, void* out,
                       void* stream) {
  if (rows < 0 || D < 1 || !(eps >= 0.0) || eps > 1e30 || !in_dtype_known(io_dtype) ||
      !state_dtype_known(param_dtype))
    return M2RNN_ERR_INVALID_ARG;
  const bool empty = rows == 0;
  if (!empty && (!y || !g_pre || !gamma || !out)) return M2RNN_ERR_INVALID_ARG;
  if (!dtypes_ok(io_dtype, param_dtype) || !block_grid_ok(rows, 1, D))
    return M2RNN_ERR_UNSUPPORTED;
  if (empty) return M2RNN_OK;
  BlockNormArgs a{};
  a.rows = rows; a.D = D; a.eps = eps; a.y = y; a.g_pre = g_pre; a.gamma = gamma; a.out = out;
  return status_of(launch_gate_rmsnorm(a, io_dtype, param_dtype, false, (hipStream_t)stream));
}

int m2rnn_gate_rmsnorm_bwd(int64_t rows, int64_t D, int io_dtype, int param_dtype, double eps,
                           const void* y, const void* g_pre, const void* gamma, const void* dout,
                           void* dy, void* dg_pre, void* dgamma, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (rows < 0 || D < 1 || !(eps >= 0.0) || eps > 1e30 || !in_dtype_known(io_dtype) ||
      !state_dtype_known(param_dtype))
    return M2RNN_ERR_INVALID_ARG;
  const bool empty = rows == 0;
  if (!dgamma) return M2RNN_ERR_INVALID_ARG;
  if (!empty && (!y || !g_pre || !gamma || !dout || !dy || !dg_pre)) return M2RNN_ERR_INVALID_ARG;
  if (!dtypes_ok(io_dtype, param_dtype) || !block_grid_ok(rows, 1, D))
    return M2RNN_ERR_UNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  if (empty) return status_of(fill(dgamma, nullptr, D, param_dtype, st));
  const size_t need = m2rnn_block_workspace_bytes(1, rows, 1, D, param_dtype);
  if (!workspace || workspace_bytes < need) return M2RNN_ERR_WORKSPACE;
  BlockNormArgs a{};
  a.rows = rows; a.D = D; a.eps = eps; a.y = y; a.g_pre = g_pre; a.gamma = gamma;
  a.dout = dout; a.dy = dy; a.dg_pre = dg_pre; a.dgamma = dgamma; a.ws = workspace;
  return status_of(launch_gate_rmsnorm(a, io_dtype, param_dtype, true, st));
}

}  // extern "C"
