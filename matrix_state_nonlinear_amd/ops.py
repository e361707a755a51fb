"""Python entry points with the C ABI's names: argument marshalling only.

Each function checks that the torch tensors it is given are on one GPU,
contiguous and of the shapes/dtypes the C ABI documents, allocates outputs and
workspace with torch (device memory is the only thing torch provides here),
and calls the library on torch's current stream.  All arithmetic happens in
the HIP kernels.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import check

_DT = {torch.float32: _lib.M2RNN_F32, torch.bfloat16: _lib.M2RNN_BF16,
       torch.float64: _lib.M2RNN_F64}


def _ptr(t):
    return None if t is None else ctypes_ptr(t)


def ctypes_ptr(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("tensors passed to libm2rnn must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libm2rnn must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _opt(t, shape, dtype, name):
    if t is not None:
        _need(t, shape, dtype, name)


def m2rnn_status_string(status: int) -> str:
    return _lib.status_string(status)


def m2rnn_workspace_bytes(is_bwd: bool, B: int, T: int, n_heads: int, qk_heads: int, K: int,
                          V: int, C: int, state_dtype=torch.float32) -> int:
    return int(_lib.lib().m2rnn_workspace_bytes(int(bool(is_bwd)), B, T, n_heads, qk_heads, K,
                                                V, C, _DT[state_dtype]))


def _heads(k, v):
    """(N, NQ): value heads from v, q/k heads from k (NQ divides N; value head
    n reads q/k head n // (N // NQ))."""
    if k.dim() != 4 or v.dim() != 4:
        raise ValueError("k, q must be [B, T, qk_heads, K] and v [B, T, n_heads, V]")
    N, NQ = v.shape[2], k.shape[2]
    if (NQ < 1 or NQ > N or N % NQ) if N > 0 else NQ != 0:
        raise ValueError(f"qk_heads = {NQ} must divide n_heads = {N}")
    return N, NQ


def _workspace(nbytes: int, device, given=None):
    if nbytes == 0:
        return None, 0
    if given is not None:
        if given.numel() * given.element_size() < nbytes:
            raise ValueError(f"workspace holds {given.numel() * given.element_size()} bytes, "
                             f"{nbytes} needed")
        return given, given.numel() * given.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def m2rnn_gates(logit: torch.Tensor, gate_kind: int, alpha=None, beta=None, out=None):
    """f[B, T, N] from the gate logits (sigmoid or exp-softplus form)."""
    if logit.dim() != 3:
        raise ValueError("logit must be [B, T, n_heads]")
    B, T, N = logit.shape
    dt = logit.dtype
    if dt not in (torch.float32, torch.float64):
        raise ValueError("logit must be float32 or float64")
    _opt(alpha, (N,), dt, "alpha")
    _opt(beta, (N,), dt, "beta")
    f = torch.empty_like(logit) if out is None else out
    _need(f, (B, T, N), dt, "out")
    st = _lib.lib().m2rnn_gates(B, T, N, int(gate_kind), _DT[dt], _ptr(logit), _ptr(alpha),
                                _ptr(beta), _ptr(f), _stream(logit.device))
    check(st, "m2rnn_gates")
    return f


def m2rnn_fwd(k, v, q, f, W, w_r, H0=None, C: int = 0, want_ht: bool = True,
              out=None, workspace=None, rc_out=None):
    """Forward recurrence.  Returns (y, HT or None, ckpt or None).

    k, q [B, T, NQ, K] and v [B, T, N, V] in float32 / bfloat16 (float32 state)
    or float64 / bfloat16 (float64 state), where NQ divides N and value head n
    reads q/k head n // (N // NQ); f [B, T, N], W [N, V, V], w_r [N, V],
    H0 [B, N, K, V] in the state dtype (taken from f).  C > 0 also writes the
    checkpoints ckpt[B, N, ceil(T / C), K, V] with ckpt[:, :, c] = H_{cC}.
    ``out`` may hold preallocated (y, HT, ckpt).  ``rc_out`` [B, N, T, K, V] (state
    dtype), when given, receives every step's rc = 1 / (1 + e^{2A}) for m2rnn_bwd.
    """
    N, NQ = _heads(k, v)
    B, T, _, K = k.shape
    V = v.shape[-1]
    sd = f.dtype
    _need(v, (B, T, N, V), k.dtype, "v")
    _need(q, (B, T, NQ, K), k.dtype, "q")
    _need(f, (B, T, N), sd, "f")
    _need(W, (N, V, V), sd, "W")
    _need(w_r, (N, V), sd, "w_r")
    _opt(H0, (B, N, K, V), sd, "H0")
    dev = k.device
    if out is not None:
        y, HT, ckpt = out
    else:
        y = torch.empty((B, T, N, V), dtype=sd, device=dev)
        HT = torch.empty((B, N, K, V), dtype=sd, device=dev) if want_ht else None
        ckpt = (torch.empty((B, N, math.ceil(T / C), K, V), dtype=sd, device=dev)
                if C and C > 0 else None)
    _need(y, (B, T, N, V), sd, "y")
    _opt(HT, (B, N, K, V), sd, "HT")
    if ckpt is not None:
        if not C or C < 1:
            raise ValueError("a checkpoint buffer needs C >= 1")
        _need(ckpt, (B, N, math.ceil(T / C), K, V), sd, "ckpt")
    _opt(rc_out, (B, N, T, K, V), sd, "rc_out")
    ws, wsb = _workspace(m2rnn_workspace_bytes(False, B, T, N, NQ, K, V, max(C, 1), sd), dev,
                         workspace)
    st = _lib.lib().m2rnn_fwd(B, T, N, NQ, K, V, _DT[k.dtype], _DT[sd], _ptr(k), _ptr(v), _ptr(q),
                              _ptr(f), _ptr(W), _ptr(w_r), _ptr(H0), _ptr(y), _ptr(HT),
                              _ptr(ckpt), int(C) if ckpt is not None else 0, _ptr(rc_out),
                              _ptr(ws), wsb, _stream(dev))
    check(st, "m2rnn_fwd")
    return y, HT, ckpt


def _bwd_outputs(k, v, q, gate_kind, logit, alpha, beta, f, W, w_r, H0, ckpt, C, dy, dHT,
                 want_dh0, rc, out):
    """Checks the backward's inputs and returns (B, T, N, NQ, K, V, state dtype,
    output dict) with the given or newly allocated gradient buffers."""
    N, NQ = _heads(k, v)
    B, T, _, K = k.shape
    V = v.shape[-1]
    sd = f.dtype
    _need(v, (B, T, N, V), k.dtype, "v")
    _need(q, (B, T, NQ, K), k.dtype, "q")
    _need(logit, (B, T, N), sd, "logit")
    _need(f, (B, T, N), sd, "f")
    _need(W, (N, V, V), sd, "W")
    _need(w_r, (N, V), sd, "w_r")
    _opt(H0, (B, N, K, V), sd, "H0")
    _need(ckpt, (B, N, math.ceil(T / C), K, V), sd, "ckpt")
    _need(dy, (B, T, N, V), sd, "dy")
    _opt(dHT, (B, N, K, V), sd, "dHT")
    _opt(rc, (B, N, T, K, V), sd, "rc")
    dev = k.device
    exp_gate = gate_kind == _lib.M2RNN_GATE_EXP_SOFTPLUS
    shapes = {"dk": (B, T, NQ, K), "dv": (B, T, N, V), "dq": (B, T, NQ, K), "dlogit": (B, T, N),
              "dW": (N, V, V), "dw_r": (N, V), "dalpha": (N,) if exp_gate else None,
              "dbeta": (N,) if exp_gate else None, "dH0": (B, N, K, V) if want_dh0 else None}
    given = dict(out) if out is not None else {}
    res = {}
    for name, shape in shapes.items():
        if name in given:
            res[name] = given[name]
            if shape is None:
                if res[name] is not None:
                    raise ValueError(f"{name} is not an output of this gate")
            else:
                (_opt if name == "dH0" else _need)(res[name], shape, sd, name)
        else:
            res[name] = None if shape is None else torch.empty(shape, dtype=sd, device=dev)
    return B, T, N, NQ, K, V, sd, res


def _bwd_args(k, v, q, gate_kind, logit, alpha, beta, f, W, w_r, H0, ckpt, C, rc, dy, dHT, o):
    """The pointer arguments shared by m2rnn_bwd and m2rnn_bwd_noalloc, in ABI order
    from k to dH0."""
    return (_ptr(k), _ptr(v), _ptr(q), int(gate_kind), _ptr(logit), _ptr(alpha), _ptr(beta),
            _ptr(f), _ptr(W), _ptr(w_r), _ptr(H0), _ptr(ckpt), int(C), _ptr(rc), _ptr(dy),
            _ptr(dHT), _ptr(o["dk"]), _ptr(o["dv"]), _ptr(o["dq"]), _ptr(o["dlogit"]),
            _ptr(o["dW"]), _ptr(o["dw_r"]), _ptr(o["dalpha"]), _ptr(o["dbeta"]), _ptr(o["dH0"]))


def m2rnn_bwd(k, v, q, gate_kind: int, logit, alpha, beta, f, W, w_r, H0, ckpt, C: int, dy,
              dHT=None, want_dh0: bool = True, workspace=None, rc=None, out=None):
    """Backward of m2rnn_fwd.  Returns a dict with dk, dv, dq, dlogit, dW, dw_r,
    dalpha and dbeta (exp-softplus gate only, else None) and dH0 (or None).
    dk and dq have the shape of k and q: with shared heads (NQ < N) each is
    the sum over the value heads that read it.  ``rc`` (from m2rnn_fwd's rc_out)
    replaces the recomputation of the states; the results are the same.
    ``out`` may hold preallocated gradient buffers under those names (any
    missing one is allocated; dH0 = None there skips it)."""
    B, T, N, NQ, K, V, sd, o = _bwd_outputs(k, v, q, gate_kind, logit, alpha, beta, f, W, w_r,
                                            H0, ckpt, C, dy, dHT, want_dh0, rc, out)
    dev = k.device
    ws, wsb = _workspace(m2rnn_workspace_bytes(True, B, T, N, NQ, K, V, C, sd), dev, workspace)
    st = _lib.lib().m2rnn_bwd(
        B, T, N, NQ, K, V, _DT[k.dtype], _DT[sd],
        *_bwd_args(k, v, q, gate_kind, logit, alpha, beta, f, W, w_r, H0, ckpt, C, rc, dy, dHT, o),
        _ptr(ws), wsb, _stream(dev))
    check(st, "m2rnn_bwd")
    return o


def m2rnn_bwd_noalloc(k, v, q, gate_kind: int, logit, alpha, beta, f, W, w_r, H0, ckpt, C: int,
                      dy, dHT=None, want_dh0: bool = True, rc=None, out=None):
    """m2rnn_bwd without a workspace: the library's static per-device scratch
    (NOALLOC_SCRATCH_BYTES) holds the partial sums.  With every gradient buffer
    given in ``out``, nothing is allocated.  Calls that may overlap on one
    device share the scratch and race."""
    B, T, N, NQ, K, V, sd, o = _bwd_outputs(k, v, q, gate_kind, logit, alpha, beta, f, W, w_r,
                                            H0, ckpt, C, dy, dHT, want_dh0, rc, out)
    st = _lib.lib().m2rnn_bwd_noalloc(
        B, T, N, NQ, K, V, _DT[k.dtype], _DT[sd],
        *_bwd_args(k, v, q, gate_kind, logit, alpha, beta, f, W, w_r, H0, ckpt, C, rc, dy, dHT, o),
        _stream(k.device))
    check(st, "m2rnn_bwd_noalloc")
    return o


def m2rnn_newton_workspace_bytes(B: int, T: int, n_heads: int, K: int, V: int,
                                 states_given: bool) -> int:
    return int(_lib.lib().m2rnn_newton_workspace_bytes(B, T, n_heads, K, V,
                                                       int(bool(states_given))))


def m2rnn_newton_fwd(k, v, q, f, W, w_r, H0=None, iters: int = 3, want_ht: bool = True,
                     want_states: bool = False, want_residual: bool = False, out=None,
                     workspace=None):
    """Parallel-in-time forward by Newton's method (fp32 state, V in 16/32/48/64).

    Arguments as for m2rnn_fwd (k, q, v in float32 or bfloat16; f, W, w_r, H0
    float32).  Returns (y, HT or None, states [B, N, T, K, V] or None,
    residual [iters + 1] or None); ``out`` may hold preallocated
    (y, HT, states, residual).
    """
    N, NQ = _heads(k, v)
    B, T, _, K = k.shape
    V = v.shape[-1]
    sd = torch.float32
    _need(v, (B, T, N, V), k.dtype, "v")
    _need(q, (B, T, NQ, K), k.dtype, "q")
    _need(f, (B, T, N), sd, "f")
    _need(W, (N, V, V), sd, "W")
    _need(w_r, (N, V), sd, "w_r")
    _opt(H0, (B, N, K, V), sd, "H0")
    dev = k.device
    if out is not None:
        y, HT, states, res = out
    else:
        y = torch.empty((B, T, N, V), dtype=sd, device=dev)
        HT = torch.empty((B, N, K, V), dtype=sd, device=dev) if want_ht else None
        states = torch.empty((B, N, T, K, V), dtype=sd, device=dev) if want_states else None
        res = torch.empty((iters + 1,), dtype=sd, device=dev) if want_residual else None
    _need(y, (B, T, N, V), sd, "y")
    _opt(HT, (B, N, K, V), sd, "HT")
    _opt(states, (B, N, T, K, V), sd, "states")
    _opt(res, (iters + 1,), sd, "residual")
    ws, wsb = _workspace(m2rnn_newton_workspace_bytes(B, T, N, K, V, states is not None), dev,
                         workspace)
    st = _lib.lib().m2rnn_newton_fwd(B, T, N, NQ, K, V, _DT[k.dtype], _ptr(k), _ptr(v), _ptr(q),
                                     _ptr(f), _ptr(W), _ptr(w_r), _ptr(H0), int(iters), _ptr(y),
                                     _ptr(HT), _ptr(states), _ptr(res), _ptr(ws), wsb,
                                     _stream(dev))
    check(st, "m2rnn_newton_fwd")
    return y, HT, states, res


def m2rnn_step(H, k, v, q, f, W, w_r, out=None):
    """One token of every sequence (decoding): H [B, N, K, V] (state dtype) is
    updated in place from H_{t-1} to H_t, and y [B, N, V] is returned.  k, q
    [B, NQ, K] and v [B, N, V] in the input dtype, f [B, N], W [N, V, V] and
    w_r [N, V] in the state dtype (taken from H)."""
    if H.dim() != 4 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("H must be [B, N, K, V], k and q [B, qk_heads, K], v [B, n_heads, V]")
    B, N, K, V = H.shape
    NQ = k.shape[1]
    if (NQ < 1 or NQ > N or N % NQ) if N > 0 else NQ != 0:
        raise ValueError(f"qk_heads = {NQ} must divide n_heads = {N}")
    sd = H.dtype
    _need(H, (B, N, K, V), sd, "H")
    _need(k, (B, NQ, K), k.dtype, "k")
    _need(q, (B, NQ, K), k.dtype, "q")
    _need(v, (B, N, V), k.dtype, "v")
    _need(f, (B, N), sd, "f")
    _need(W, (N, V, V), sd, "W")
    _need(w_r, (N, V), sd, "w_r")
    y = torch.empty((B, N, V), dtype=sd, device=H.device) if out is None else out
    _need(y, (B, N, V), sd, "out")
    st = _lib.lib().m2rnn_step(B, N, NQ, K, V, _DT[k.dtype], _DT[sd], _ptr(k), _ptr(v), _ptr(q),
                               _ptr(f), _ptr(W), _ptr(w_r), _ptr(H), _ptr(y), _stream(H.device))
    check(st, "m2rnn_step")
    return y


def _io_param(x, param):
    """(io dtype code, param dtype code) of a block call; param from the parameters."""
    if param.dtype not in (torch.float32, torch.float64):
        raise ValueError("parameters must be float32 or float64")
    return _DT[x.dtype], _DT[param.dtype]


def m2rnn_conv_silu(x, w, bias=None, out=None):
    """Block prologue on one projected tensor x [B, T, C] (float32 / bfloat16, or
    float64 / bfloat16): SiLU of the depthwise causal convolution with w [C, 4]
    (+ bias [C]); returns [B, T, C] in x's dtype."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, C]")
    B, T, C = x.shape
    io, pd = _io_param(x, w)
    _need(w, (C, 4), w.dtype, "w")
    _opt(bias, (C,), w.dtype, "bias")
    y = torch.empty_like(x) if out is None else out
    _need(y, (B, T, C), x.dtype, "out")
    st = _lib.lib().m2rnn_conv_silu(B, T, C, io, pd, _ptr(x), _ptr(w), _ptr(bias), _ptr(y),
                                    _stream(x.device))
    check(st, "m2rnn_conv_silu")
    return y


def m2rnn_conv_silu_bwd(x, w, bias, dout, workspace=None):
    """Gradients of sum(dout * m2rnn_conv_silu(x, w, bias)): (dx, dw, dbias or None),
    in the parameters' dtype."""
    B, T, C = x.shape
    io, pd = _io_param(x, w)
    _need(w, (C, 4), w.dtype, "w")
    _opt(bias, (C,), w.dtype, "bias")
    _need(dout, (B, T, C), w.dtype, "dout")
    dx = torch.empty((B, T, C), dtype=w.dtype, device=x.device)
    dw = torch.empty((C, 4), dtype=w.dtype, device=x.device)
    dbias = torch.empty((C,), dtype=w.dtype, device=x.device) if bias is not None else None
    nb = int(_lib.lib().m2rnn_block_workspace_bytes(0, B, T, C, pd))
    ws, wsb = _workspace(nb, x.device, workspace)
    st = _lib.lib().m2rnn_conv_silu_bwd(B, T, C, io, pd, _ptr(x), _ptr(w), _ptr(bias),
                                        _ptr(dout), _ptr(dx), _ptr(dw), _ptr(dbias), _ptr(ws),
                                        wsb, _stream(x.device))
    check(st, "m2rnn_conv_silu_bwd")
    return dx, dw, dbias


def m2rnn_gate_rmsnorm(y, g_pre, gamma, eps: float = 1e-6, out=None):
    """Block epilogue: gamma * z / sqrt(mean(z^2) + eps), z = y * SiLU(g_pre), over the
    last dimension D.  y [..., D] and gamma [D] in the state dtype, g_pre [..., D] in the
    input dtype; returns [..., D] in g_pre's dtype."""
    D = y.shape[-1]
    rows = y.numel() // D if D else 0
    io, pd = _io_param(g_pre, y)
    _need(g_pre, tuple(y.shape), g_pre.dtype, "g_pre")
    _need(gamma, (D,), y.dtype, "gamma")
    o = torch.empty(tuple(y.shape), dtype=g_pre.dtype, device=y.device) if out is None else out
    _need(o, tuple(y.shape), g_pre.dtype, "out")
    st = _lib.lib().m2rnn_gate_rmsnorm(rows, D, io, pd, float(eps), _ptr(y), _ptr(g_pre),
                                       _ptr(gamma), _ptr(o), _stream(y.device))
    check(st, "m2rnn_gate_rmsnorm")
    return o


def m2rnn_gate_rmsnorm_bwd(y, g_pre, gamma, dout, eps: float = 1e-6, workspace=None):
    """Gradients of sum(dout * m2rnn_gate_rmsnorm(y, g_pre, gamma, eps)):
    (dy, dg_pre, dgamma) in the state dtype."""
    D = y.shape[-1]
    rows = y.numel() // D if D else 0
    io, pd = _io_param(g_pre, y)
    _need(g_pre, tuple(y.shape), g_pre.dtype, "g_pre")
    _need(gamma, (D,), y.dtype, "gamma")
    _need(dout, tuple(y.shape), y.dtype, "dout")
    dy = torch.empty_like(y)
    dg = torch.empty_like(y)
    dgamma = torch.empty((D,), dtype=y.dtype, device=y.device)
    nb = int(_lib.lib().m2rnn_block_workspace_bytes(1, rows, 1, D, pd))
    ws, wsb = _workspace(nb, y.device, workspace)
    st = _lib.lib().m2rnn_gate_rmsnorm_bwd(rows, D, io, pd, float(eps), _ptr(y), _ptr(g_pre),
                                           _ptr(gamma), _ptr(dout), _ptr(dy), _ptr(dg),
                                           _ptr(dgamma), _ptr(ws), wsb, _stream(y.device))
    check(st, "m2rnn_gate_rmsnorm_bwd")
    return dy, dg, dgamma
