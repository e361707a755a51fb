"""float64 reference of the M²RNN recurrence: gates, forward, backward.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Slow and plain on
purpose: a time loop in Python, vectorised over the independent (b, n) units
with numpy float64 matmuls, no blocking, fusion or reordering beyond what the
equations state.

Sources (cited by title and section):
  [R] review of "M²RNN: Non-Linear RNNs with Matrix-Valued States for Scalable
      Language Modeling" (arXiv:2603.14360v2): section 2.1 Eq. (10)-(12)
      (recurrence and readout), section 2.2 Eq. (13)/(17) (exp-softplus gate),
      section 2.5 / Theorem 1 (vector-RNN embedding), section 2.6 (recompute
      then reverse-scan backward), section 2.7 (corrected BPTT chain rule).
  [P] pararnn-torch documentation, "ParaM2RNN": "Recurrence (library core)"
      (sigmoid gate, right-multiplied W) and "Jacobian class" (dense (KV)^2
      Jacobian, used as an oracle only).

Layouts (token-major, C-contiguous):
  k, q  [B, T, N, K]      v, dy, y  [B, T, N, V]      f, logit  [B, T, N]
        or [B, T, NQ, K] with NQ dividing N: q and k shared by groups of
        N / NQ consecutive value heads ([R] section 2.4 shares one q and one k
        across all value heads, NQ = 1)
  W     [N, V, V]  with (H W)[i, j] = sum_l H[i, l] W[l, j]
  w_r   [N, V]            H0, HT, dHT  [B, N, K, V]
  ckpt  [B, N, ceil(T / C), K, V], ckpt[:, :, c] = H_{cC} (H_0 = H0)
"""
from __future__ import annotations

import math

import numpy as np

GATE_SIGMOID = 0
GATE_EXP_SOFTPLUS = 1

_f64 = np.float64


def _a(x):
    return np.asarray(x, dtype=_f64)


def softplus(x):
    """softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(e^{-|x|}) so
    that neither branch overflows ([R] section 2.2 writes the gate through it)."""
    x = _a(x)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """Logistic function 1 / (1 + e^{-x}), split at 0 so exp never overflows."""
    x = _a(x)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def gates(kind, logit, alpha=None, beta=None):
    """Forget gate f for every (b, t, n); it never reads the state, so the whole
    sequence is computed up front ([R] section 2.2, last paragraph).

    kind GATE_SIGMOID:      f = sigmoid(logit)            ([P] "Recurrence")
    kind GATE_EXP_SOFTPLUS: f = (1 + e^{a + beta_n})^{-alpha_n}
                              = exp(-alpha_n * softplus(a + beta_n))
                                                          ([R] Eq. 13 / 17)
    logit: [B, T, N]; alpha, beta: [N] (exp-softplus only; alpha >= 0 keeps f
    in [0, 1], a precondition that is not enforced here).
    """
    logit = _a(logit)
    if kind == GATE_SIGMOID:
        return sigmoid(logit)
    if kind == GATE_EXP_SOFTPLUS:
        x = logit + _a(beta)
        return np.exp(-_a(alpha) * softplus(x))
    raise ValueError(f"unknown gate kind {kind}")


def gate_partials(kind, logit, alpha=None, beta=None):
    """f and its partial derivatives (df/dlogit, df/dalpha, df/dbeta) per element.

    sigmoid:       df/dg = f (1 - f)
    exp-softplus:  with x = a + beta, f = exp(-alpha softplus(x)) and
                   softplus'(x) = sigmoid(x):
                   df/da = df/dbeta = -alpha sigmoid(x) f,  df/dalpha = -softplus(x) f
    """
    f = gates(kind, logit, alpha, beta)
    if kind == GATE_SIGMOID:
        return f, f * (1.0 - f), None, None
    x = _a(logit) + _a(beta)
    dfa = -_a(alpha) * sigmoid(x) * f
    return f, dfa, -softplus(x) * f, dfa


def _expand_qk(x, N):
    """Shared q / k ([R] section 2.4): value head n reads q/k head n // (N / NQ).
    Returns the per-value-head array [B, T, N, K]."""
    NQ = x.shape[2]
    if NQ == N:
        return x
    assert NQ > 0 and N % NQ == 0, (NQ, N)
    return np.repeat(x, N // NQ, axis=2)


def _reduce_qk(g, NQ):
    """Gradient of a shared q / k: the sum over the value heads that read it
    (chain rule), in head order."""
    B, T, N, K = g.shape
    if NQ == N:
        return g
    return g.reshape(B, T, NQ, N // NQ, K).sum(axis=3)


def forward(k, v, q, f, W, w_r, H0=None, C=0, keep_states=False):
    """M²RNN forward, [R] section 2.1 Eq. (10)-(12), [P] "Recurrence":

        Z_t = tanh(H_{t-1} W + k_t v_t^T)
        H_t = f_t H_{t-1} + (1 - f_t) Z_t
        y_t = H_t^T q_t + w_r (.) v_t          (readout of the updated state)

    starting from H_0 = H0 (zero when None).  Returns a dict with y, HT, and
    ckpt when C > 0; with keep_states also H [T+1, B, N, K, V] (H[0] = H_0)
    and Z [T, B, N, K, V].
    """
    k, v, q, f, W, w_r = map(_a, (k, v, q, f, W, w_r))
    k, q = _expand_qk(k, v.shape[2]), _expand_qk(q, v.shape[2])
    B, T, N, K = k.shape
    V = v.shape[-1]
    H = np.zeros((B, N, K, V), _f64) if H0 is None else _a(H0).copy()
    y = np.empty((B, T, N, V), _f64)
    ckpt = None
    if C and C > 0:
        ckpt = np.empty((B, N, math.ceil(T / C), K, V), _f64)
    Hs = Zs = None
    if keep_states:
        Hs = np.empty((T + 1, B, N, K, V), _f64)
        Zs = np.empty((T, B, N, K, V), _f64)
        Hs[0] = H
    for t in range(T):
        if ckpt is not None and t % C == 0:
            ckpt[:, :, t // C] = H
        A = np.matmul(H, W[None]) + k[:, t, :, :, None] * v[:, t, :, None, :]
        Z = np.tanh(A)
        ft = f[:, t, :, None, None]
        H = ft * H + (1.0 - ft) * Z
        y[:, t] = np.matmul(q[:, t, :, None, :], H)[:, :, 0, :] + w_r[None] * v[:, t]
        if keep_states:
            Hs[t + 1] = H
            Zs[t] = Z
    out = {"y": y, "HT": H}
    if ckpt is not None:
        out["ckpt"] = ckpt
    if keep_states:
        out["H"] = Hs
        out["Z"] = Zs
    return out


def decode_step(H, k, v, q, f, W, w_r):
    """One step of the recurrence for a batch of single tokens (decoding), the
    sequential cell step of [P] "Reproduce (sequential)" with the readout of
    [R] section 2.1 Eq. (10)-(12):

        H_t = f H_{t-1} + (1 - f) tanh(H_{t-1} W + k v^T),   y = H_t^T q + w_r (.) v

    H [B, N, K, V] is H_{t-1}; k, q [B, NQ, K] (NQ dividing N, shared as in
    forward); v [B, N, V]; f [B, N].  Returns (H_t, y) with y [B, N, V].
    """
    H, k, v, q, f, W, w_r = map(_a, (H, k, v, q, f, W, w_r))
    N = v.shape[1]
    k = _expand_qk(k[:, None], N)[:, 0]
    q = _expand_qk(q[:, None], N)[:, 0]
    Z = np.tanh(np.matmul(H, W[None]) + k[:, :, :, None] * v[:, :, None, :])
    fb = f[:, :, None, None]
    Hn = fb * H + (1.0 - fb) * Z
    y = np.matmul(q[:, :, None, :], Hn)[:, :, 0, :] + w_r[None] * v
    return Hn, y


def backward(k, v, q, f, W, w_r, dy, H0=None, dHT=None, gate_kind=None,
             logit=None, alpha=None, beta=None, b_group=None):
    """Reverse-time BPTT of the forward above for the loss L with dL/dy = dy
    and dL/dH_T = dHT (zero when None).

    Follows [R] section 2.6 (rerun the recurrence, keep every step's state,
    scan backwards) and the corrected chain rule of [R] section 2.7, with the
    value-residual branch restored.  With u_t = dy_t and C_t the state
    gradient arriving from later steps (C_T = dHT):

        R_t     = C_t + q_t u_t^T
        D_t     = ((1 - f_t) R_t) (.) (1 - Z_t (.) Z_t)
        C_{t-1} = f_t R_t + D_t W^T
        df_t    = <R_t, H_{t-1} - Z_t>_F
        dW     += H_{t-1}^T D_t              (summed over batch and time)
        dk_t    = D_t v_t,   dv_t = D_t^T k_t + w_r (.) u_t,   dq_t = H_t u_t
        dw_r   += u_t (.) v_t                (summed over batch and time)

    dH0 = C_0.  When gate_kind is given, the gate chain rule maps df to
    d(logit) (and d(alpha), d(beta) summed over batch and time for the
    exp-softplus gate).  ``b_group`` bounds memory by processing that many
    batch rows at a time (per-row results are independent; only the
    parameter gradients are summed across the groups).
    """
    k, v, q, f, W, w_r, dy = map(_a, (k, v, q, f, W, w_r, dy))
    NQ = k.shape[2]
    k, q = _expand_qk(k, v.shape[2]), _expand_qk(q, v.shape[2])
    B, T, N, K = k.shape
    V = v.shape[-1]
    dk = np.empty((B, T, N, K), _f64)
    dq = np.empty((B, T, N, K), _f64)
    dv = np.empty((B, T, N, V), _f64)
    df = np.empty((B, T, N), _f64)
    dH0 = np.empty((B, N, K, V), _f64)
    dW = np.zeros((N, V, V), _f64)
    WT = np.swapaxes(W, -1, -2)[None]
    step = max(1, B if not b_group else b_group)  # an empty batch has no groups
    for b0 in range(0, B, step):
        sl = slice(b0, min(B, b0 + step))
        st = forward(k[sl], v[sl], q[sl], f[sl], W, w_r,
                     None if H0 is None else _a(H0)[sl], keep_states=True)
        Hs, Zs = st["H"], st["Z"]
        Cst = (np.zeros_like(Hs[0]) if dHT is None else _a(dHT)[sl].copy())
        for t in range(T - 1, -1, -1):
            u = dy[sl, t]                                         # [b, N, V]
            R = Cst + q[sl, t, :, :, None] * u[:, :, None, :]
            dq[sl, t] = np.matmul(Hs[t + 1], u[..., None])[..., 0]
            Zt = Zs[t]
            Hp = Hs[t]
            ft = f[sl, t, :, None, None]
            D = (1.0 - ft) * R * (1.0 - Zt * Zt)
            df[sl, t] = np.sum(R * (Hp - Zt), axis=(-2, -1))
            dk[sl, t] = np.matmul(D, v[sl, t, :, :, None])[..., 0]
            dv[sl, t] = (np.matmul(np.swapaxes(D, -1, -2), k[sl, t, :, :, None])[..., 0]
                         + w_r[None] * u)
            dW += np.sum(np.matmul(np.swapaxes(Hp, -1, -2), D), axis=0)
            Cst = ft * R + np.matmul(D, WT)
        dH0[sl] = Cst
        del Hs, Zs, st
    out = {"dk": _reduce_qk(dk, NQ), "dv": dv, "dq": _reduce_qk(dq, NQ), "df": df, "dW": dW,
           "dw_r": np.sum(dy * v, axis=(0, 1)), "dH0": dH0}
    if gate_kind is not None:
        _, dfl, dfa, dfb = gate_partials(gate_kind, logit, alpha, beta)
        out["dlogit"] = df * dfl
        if gate_kind == GATE_EXP_SOFTPLUS:
            out["dalpha"] = np.sum(df * dfa, axis=(0, 1))
            out["dbeta"] = np.sum(df * dfb, axis=(0, 1))
    return out


def step_jacobian_dense(H_prev, Z, f_t, W):
    """Dense one-step Jacobian d vec(H_t) / d vec(H_{t-1}) of one (b, n) unit,
    the (KV) x (KV) matrix that [P] "Jacobian class" keeps as an oracle only.

    vec is row-major (index i*V + j).  From Eq. (10)-(11),
    dH_t[i,j] / dH_{t-1}[i',l] = delta_ii' (f delta_jl + (1 - f)(1 - Z_ij^2) W[l, j]),
    i.e. J = f I + (1 - f) diag(vec(1 - Z^2)) (I_K kron W^T).
    H_prev enters only through Z; it is accepted to keep the call explicit.
    """
    Z = _a(Z)
    K, V = Z.shape
    W = _a(W)
    eye = np.eye(K * V)
    return f_t * eye + (1.0 - f_t) * (1.0 - Z * Z).reshape(-1, 1) * np.kron(np.eye(K), W.T)


def tangent_growth(k, v, q, f, W, H0=None, seed=0):
    """Sensitivity of the exact dynamics: push a random tangent dH through the
    linearisation of Eq. (10)-(11) along the float64 trajectory,

        dH_t = f_t dH_{t-1} + (1 - f_t) (1 - Z_t^2) (.) (dH_{t-1} W),

    i.e. J_t applied to vec(dH) without forming J_t.  Each row of the state is
    a recurrence of its own (W right-multiplies, so it mixes the value columns
    of one row; the rank-1 write and the gate act row by row), and J_t is block
    diagonal over the K rows: a perturbation of one row is amplified by that
    row's blocks alone.  So the amplification is measured per row (max-abs
    norm over the row's V entries; one norm over the whole state would hide a
    row whose tangent stays smaller than another's), and the result per
    (b, n) is the largest over the rows of max_{s <= t} |dH_t[i]| / |dH_s[i]|.
    Values near or below 1 mean rounding errors do not grow; large values
    mean the trajectory is not reproducible in finite precision.
    """
    k, v, q, f, W = map(_a, (k, v, q, f, W))
    B, T, N, K = k.shape
    V = v.shape[-1]
    rng = np.random.Generator(np.random.PCG64(seed))
    H = np.zeros((B, N, K, V), _f64) if H0 is None else _a(H0).copy()
    dH = rng.standard_normal((B, N, K, V))
    dH /= np.abs(dH).max(axis=-1)[..., None]
    logn = np.zeros((B, N, K))       # log of each row's true max-abs norm
    run_min = np.zeros((B, N, K))
    best = np.zeros((B, N, K))
    for t in range(T):
        A = np.matmul(H, W[None]) + k[:, t, :, :, None] * v[:, t, :, None, :]
        Z = np.tanh(A)
        ft = f[:, t, :, None, None]
        dH = ft * dH + (1.0 - ft) * (1.0 - Z * Z) * np.matmul(dH, W[None])
        H = ft * H + (1.0 - ft) * Z
        m = np.abs(dH).max(axis=-1)
        dH = dH / m[..., None]           # renormalise each row; the log keeps the scale
        logn = logn + np.log(m)
        best = np.maximum(best, logn - run_min)
        run_min = np.minimum(run_min, logn)
    return np.exp(best.max(axis=-1))
