"""float64 reference of the parallel-in-time Newton solve of the M²RNN state
sequence.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: the pararnn-torch "ParaM2RNN" page ("Jacobian class": factorized
Newton for the matrix recurrence; "Parallel path": Newton on the matrix
residual) and the "ParaGRU" page ("Parallel path": Newton + scan, default
initial guess h_t^(0) = f(0, x_t), a typical budget of three iterations).

The unknowns are the states X_1 .. X_T of every (b, n) unit (X_0 = H_0 given);
the residual of step t is X_t - F(X_{t-1}, x_t) with F the recurrence of the
review's section 2.1:  F(X, x_t) = f X + (1 - f) tanh(X W + k v^T).  One Newton
iteration linearises F at the current iterate X^old and solves the linear
recurrence exactly:

    X_t^new = F(X_{t-1}^old) + J_t (X_{t-1}^new - X_{t-1}^old),
    J_t h = f h + (1 - f) (h W) (.) (1 - Z_t^2),   Z_t = tanh(X_{t-1}^old W + k v^T),

acting on every state row h (1 x V) alone.  Written as an affine recurrence:
X_t^new = J_t X_{t-1}^new + c_t with c_t = (1 - f)(Z_t - (X_{t-1}^old W) (.) (1 - Z_t^2)).
Here that recurrence is solved by a plain loop over t; a parallel scan gives
the same values up to rounding.  Readings: the initial guess F(0, x_t) is
X_t^(0) = (1 - f_t) tanh(k_t v_t^T); a causal system is solved exactly by at
most T iterations (after i iterations X_1 .. X_i are exact).
"""
from __future__ import annotations

import numpy as np

from .m2rnn_oracle import _expand_qk

_f64 = np.float64


def _a(x):
    return None if x is None else np.asarray(x, dtype=_f64)


def newton_linearize(X_prev, k_t, v_t, f_t, W):
    """For one step t over all units: (F_t, s_t, c_t) at X_prev = X_{t-1}^old,
    with s_t = 1 - Z_t^2 the diagonal factor of J_t and c_t its affine term."""
    XW = np.matmul(X_prev, W[None])
    Z = np.tanh(XW + k_t[..., :, None] * v_t[..., None, :])
    fb = f_t[..., None, None]
    F = fb * X_prev + (1.0 - fb) * Z
    s = 1.0 - Z * Z
    c = (1.0 - fb) * (Z - XW * s)
    return F, s, c


def newton_forward(k, v, q, f, W, w_r, H0=None, iters=3, X_init=None):
    """Newton iterations from the initial guess X_t^(0) = F(0, x_t) (or X_init
    [T + 1, B, N, K, V] with X_init[0] = H_0).  Returns a dict with the final
    states X [T + 1, B, N, K, V] (X[0] = H_0), the readouts y [B, T, N, V] of
    X, and res[i] = max_t |X_t^(i) - F(X_{t-1}^(i))| for the iterates i = 0 .. iters."""
    k, v, q, f, W, w_r = map(_a, (k, v, q, f, W, w_r))
    k, q = _expand_qk(k, v.shape[2]), _expand_qk(q, v.shape[2])
    B, T, N, K = k.shape
    V = v.shape[-1]
    H0 = np.zeros((B, N, K, V), _f64) if H0 is None else _a(H0)
    if X_init is None:
        X = np.empty((T + 1, B, N, K, V), _f64)
        X[0] = H0
        for t in range(T):
            X[t + 1] = (1.0 - f[:, t, :, None, None]) * np.tanh(
                k[:, t, :, :, None] * v[:, t, :, None, :])
    else:
        X = _a(X_init).copy()
    res = []

    def residual(X):
        r = 0.0
        for t in range(T):
            F, _, _ = newton_linearize(X[t], k[:, t], v[:, t], f[:, t], W)
            r = max(r, float(np.max(np.abs(X[t + 1] - F))) if X[t + 1].size else 0.0)
        return r

    res.append(residual(X))
    for _ in range(iters):
        Xn = np.empty_like(X)
        Xn[0] = H0
        for t in range(T):
            _, s, c = newton_linearize(X[t], k[:, t], v[:, t], f[:, t], W)
            fb = f[:, t, :, None, None]
            h = Xn[t]
            Xn[t + 1] = fb * h + (1.0 - fb) * np.matmul(h, W[None]) * s + c
        X = Xn
        res.append(residual(X))
    y = np.empty((B, T, N, V), _f64)
    for t in range(T):
        y[:, t] = np.matmul(q[:, t, :, None, :], X[t + 1])[:, :, 0, :] + w_r[None] * v[:, t]
    return {"X": X, "y": y, "res": np.asarray(res)}
