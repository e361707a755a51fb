// Host-side interface of the parallel-in-time Newton forward (m2rnn_newton.hip)
// for the C ABI (m2rnn_api.hip).
#pragma once

#include "m2rnn_internal.h"

namespace m2rnn {

// Parallel-in-time Newton forward (fp32 state, V in {16, 32, 48, 64}).
struct NewtonArgs {
  const void* k;     // [B, T, NQ, K] in dtype
  const void* v;     // [B, T, N, V]
  const void* q;     // [B, T, NQ, K]
  const float* f;    // [B, T, N]
  const float* W;    // [N, V, V]
  const float* w_r;  // [N, V]
  const float* H0;   // [B, N, K, V] or null
  float* y;          // [B, T, N, V]
  float* HT;         // [B, N, K, V] or null
  float* X;          // [B N, T, K, V] iterate: X[u][t] is the state after step t
  float* Xn;         // [B N, T, K, V] the next iterate (the two buffers alternate)
  float* S;          // [B N, T, K, V] (1 - f_t)(1 - Z_t^2) at the linearisation
  float* R;          // [B N, T, K, V] residual X_t - F(X_{t-1})
  float* M;          // [B N, P, K, V, V] chunk maps (P > 1)
  float* E;          // [B N, P, K, V] chunk updates from a zero start (P > 1)
  float* D;          // [B N, P, K, V] chunk starting updates (P > 1)
  unsigned* res;     // [iters + 1] largest |residual| per iterate (float bits), or null
  int64_t B, T, N, NQ, K, V;
  int iters;
  int64_t L, P;      // chunk length and count
  int64_t TL, NTB;   // linearisation: steps per wave and blocks of steps
};
// Workspace layout (offsets in floats, 64-float aligned) and schedule sizes.
struct NewtonLayout {
  int64_t L, P, TL, NTB;
  size_t X, X2, S, R, M, E, D;  // X unused when the caller's states buffer holds the iterate
  size_t total_floats;
};
NewtonLayout newton_layout(int64_t B, int64_t T, int64_t N, int64_t K, int64_t V,
                           bool states_given);
hipError_t launch_newton(const NewtonArgs& a, int in_dtype, hipStream_t stream);

}  // namespace m2rnn
