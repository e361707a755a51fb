"""float64 reference of the elementwise parts of the M²RNN block around the
recurrence: the short causal convolution with SiLU on q, k, v before it, and
the output gate with RMSNorm after it, each with its backward.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Plain numpy, written
from the definitions, no blocking or reordering.

Source: review of "M²RNN: Non-Linear RNNs with Matrix-Valued States for
Scalable Language Modeling" (arXiv:2603.14360v2), section 2.3 (the full block,
Eq. 14-23): q, k, v each pass a linear projection, a depthwise causal Conv1D of
kernel size 4 and SiLU; the output gate g = SiLU(W_g x) has no convolution; the
recurrence's readout y is multiplied by g and then RMS-normalised
(gate first, then RMSNorm) before the output projection W_o.

Readings of what the section leaves open:
  * the convolution has a per-channel bias (optional: None means none) and
    zero history before the first token of the sequence;
  * tap i of the kernel weights the input 3 - i steps back,
    u_t = bias + sum_{i=0}^{3} w[i] x_{t-3+i}: the cross-correlation layout of
    a depthwise torch Conv1d with left padding 3;
  * RMSNorm normalises over all channels of a token (every head's V values,
    D = N V), with a learned per-channel scale gamma and
    rms = sqrt(mean(z^2) + eps); eps is an argument (the section gives none).

Layouts: x, u, dx [B, T, C] (channels last); w [C, 4]; bias [C];
y, g_pre, out [B, T, D]; gamma [D].
"""
from __future__ import annotations

import numpy as np

_f64 = np.float64


def _a(x):
    return None if x is None else np.asarray(x, dtype=_f64)


def _sigmoid(x):
    # split at 0 so that neither branch overflows
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(x):
    """SiLU(x) = x sigmoid(x)."""
    x = _a(x)
    return x * _sigmoid(x)


def silu_grad(x):
    """d SiLU / dx = sigmoid(x) (1 + x (1 - sigmoid(x)))."""
    x = _a(x)
    s = _sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def causal_conv(x, w, bias=None):
    """u_t[c] = bias[c] + sum_{i=0}^{3} w[c, i] x_{t-3+i}[c], x_{<0} = 0
    (depthwise, per sequence: [R] section 2.3, step 1)."""
    x, w, bias = _a(x), _a(w), _a(bias)
    B, T, C = x.shape
    taps = w.shape[1]
    u = np.zeros((B, T, C), _f64) if bias is None else np.broadcast_to(bias, (B, T, C)).copy()
    for i in range(taps):
        lag = taps - 1 - i  # tap i reads the input lag steps back
        u[:, lag:] += w[None, None, :, i] * x[:, :T - lag]
    return u


def conv_silu(x, w, bias=None):
    """The prologue applied to each of q, k, v: SiLU(causal_conv(x))."""
    return silu(causal_conv(x, w, bias))


def conv_silu_backward(x, w, bias, dout):
    """Gradients of sum(dout * conv_silu(x, w, bias)): (dx, dw, dbias).

    du = dout silu'(u);  dx_s = sum_i w[i] du_{s+3-i};  dw[i] = sum_{b,t} du_t x_{t-3+i};
    dbias = sum_{b,t} du_t (dbias is None when bias is None)."""
    x, w, dout = _a(x), _a(w), _a(dout)
    B, T, C = x.shape
    taps = w.shape[1]
    du = dout * silu_grad(causal_conv(x, w, bias))
    dx = np.zeros((B, T, C), _f64)
    dw = np.zeros((C, taps), _f64)
    for i in range(taps):
        lag = taps - 1 - i
        dx[:, :T - lag] += w[None, None, :, i] * du[:, lag:]
        dw[:, i] = np.sum(du[:, lag:] * x[:, :T - lag], axis=(0, 1))
    dbias = None if bias is None else np.sum(du, axis=(0, 1))
    return dx, dw, dbias


def gate_rmsnorm(y, g_pre, gamma, eps):
    """Epilogue: z = y SiLU(g_pre); out = gamma z / sqrt(mean_D(z^2) + eps)
    ([R] section 2.3, step 4: gate first, then RMSNorm over the token's D
    channels)."""
    y, g_pre, gamma = _a(y), _a(g_pre), _a(gamma)
    z = y * silu(g_pre)
    rms = np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)
    return gamma * z / rms


def gate_rmsnorm_backward(y, g_pre, gamma, eps, dout):
    """Gradients of sum(dout * gate_rmsnorm(...)): (dy, dg_pre, dgamma).

    With r = 1 / sqrt(mean(z^2) + eps) and zh = z r: dgamma = sum_{b,t} dout zh;
    dzh = dout gamma; dz = r (dzh - zh mean_D(dzh zh)); dy = dz SiLU(g_pre);
    dg_pre = dz y silu'(g_pre)."""
    y, g_pre, gamma, dout = _a(y), _a(g_pre), _a(gamma), _a(dout)
    g = silu(g_pre)
    z = y * g
    r = 1.0 / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)
    zh = z * r
    dgamma = np.sum(dout * zh, axis=tuple(range(dout.ndim - 1)))
    dzh = dout * gamma
    dz = r * (dzh - zh * np.mean(dzh * zh, axis=-1, keepdims=True))
    return dz * g, dz * y * silu_grad(g_pre), dgamma
