"""Seeded synthetic inputs for the M²RNN recurrence workloads.

This module only draws random numbers and rounds them to the storage type the
kernels read (bf16 round-to-nearest-even).  It holds none of the recurrence's
arithmetic: both the float64 oracle and the HIP path consume what it returns,
so the two sides always see bit-identical inputs.

The named workloads follow the shapes and distributions of the M²RNN
layer described in the review of "M²RNN: Non-Linear RNNs with Matrix-Valued
States for Scalable Language Modeling" (section 2.1, Eq. 10-12; section 2.2,
Eq. 13/17 for the exp-softplus gate; section 2.4 for the paper's own K=64,
V=16 head shape with one q and one k shared by all value heads).  "N(0, s)"
is read as standard deviation s.

Draw order inside one workload is fixed: k, v, q, gate logit, alpha, beta,
W, w_r, dy.  Every array is drawn at its full shape, so a workload with the
same seed and shape always reproduces the same values.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GATE_SIGMOID = 0
GATE_EXP_SOFTPLUS = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    N: int
    K: int
    V: int
    bf16: bool            # k, v, q stored as bf16 (else fp32)
    gate: int             # GATE_SIGMOID or GATE_EXP_SOFTPLUS
    kq_scale: float       # std of k and q
    v_scale: float        # std of v
    g_mean: float         # mean of the sigmoid-gate logit (sigmoid gate only)
    w_kind: str           # "ident" (I + w_eps*N(0,1)*w_scale) or "orth" (0.9*Q)
    w_eps: float
    w_scale: float
    C: int = 0            # checkpoint interval for the backward workload (0: forward only)
    seed: int = 1
    NQ: int = 0           # heads of q and k, dividing N (0: one per value head)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def qk_heads(self) -> int:
        return self.NQ if self.NQ else self.N

    @property
    def tokens_heads(self) -> int:
        return self.B * self.T * self.N


# The workloads.  Sizes are the full ones; tests shrink B/T through
# Workload.replace while keeping the recipe.  The first five are the
# benchmark's configurations; the last is the paper's multi-value layout
# (K=64, V=16, q and k shared by all heads) at the same state size per
# sequence as the long-context one (64 heads x 64 x 16).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", B=2, T=64, N=1, K=8, V=8, bf16=False,
                          gate=GATE_SIGMOID, kq_scale=1 / math.sqrt(8),
                          v_scale=1 / math.sqrt(8), g_mean=0.0, w_kind="ident",
                          w_eps=0.1, w_scale=1 / math.sqrt(8), seed=1),
    "fp32_k64": Workload("fp32_k64", B=8, T=2048, N=8, K=64, V=64, bf16=False,
                         gate=GATE_SIGMOID, kq_scale=1 / 8, v_scale=1 / 8,
                         g_mean=1.0, w_kind="ident", w_eps=0.05, w_scale=1 / 8,
                         seed=2),
    "long_t16k_k64": Workload("long_t16k_k64", B=4, T=16384, N=16, K=64, V=64,
                              bf16=True, gate=GATE_EXP_SOFTPLUS, kq_scale=1 / 8,
                              v_scale=1 / 8, g_mean=0.0, w_kind="ident",
                              w_eps=0.05, w_scale=1 / 8, seed=3),
    "big_state_k128": Workload("big_state_k128", B=1, T=16384, N=32, K=128,
                               V=128, bf16=True, gate=GATE_SIGMOID,
                               kq_scale=1 / math.sqrt(128),
                               v_scale=1 / math.sqrt(128), g_mean=0.0,
                               w_kind="orth", w_eps=0.0, w_scale=0.0, seed=4),
    "fwd_bwd_k32_v128": Workload("fwd_bwd_k32_v128", B=16, T=4096, N=16, K=32,
                                 V=128, bf16=True, gate=GATE_EXP_SOFTPLUS,
                                 kq_scale=1 / math.sqrt(32),
                                 v_scale=1 / math.sqrt(128), g_mean=0.0,
                                 w_kind="ident", w_eps=0.05,
                                 w_scale=1 / math.sqrt(128), C=64, seed=5),
    "multi_value_k64_v16": Workload("multi_value_k64_v16", B=4, T=16384, N=64, K=64, V=16,
                                    bf16=True, gate=GATE_EXP_SOFTPLUS, kq_scale=1 / 8,
                                    v_scale=1 / 4, g_mean=0.0, w_kind="ident", w_eps=0.05,
                                    w_scale=1 / 4, C=4, seed=6, NQ=1),
}
# Decoding: one token for each of B sequences (T = 1), the state updated in
# place.  The recipes of the long-context workload (K = V = 64) and of the
# multi-value one (K = 64, V = 16, shared q/k), with 512 sequences: the state
# read and written per step is 128 MiB (512 x 16 heads x 64 x 64 fp32), so the
# step's HBM traffic, not its launch, sets its time.
DECODE_WORKLOADS = {
    "decode_k64": WORKLOADS["long_t16k_k64"].replace(name="decode_k64", B=512, T=1, seed=7),
    "decode_multi_value": WORKLOADS["multi_value_k64_v16"].replace(
        name="decode_multi_value", B=512, T=1, C=0, seed=8),
}

# The parallel-in-time Newton forward's workload: few units (one sequence of
# four value heads with the paper's K = 64, V = 16 and shared q/k), so that the
# sequential forward leaves most of the device idle, and a contractive
# transition W = 0.9 Q (Q orthogonal), under which every step map contracts and
# Newton converges in about three iterations.
NEWTON_WORKLOADS = {
    "newton_k64_v16": WORKLOADS["multi_value_k64_v16"].replace(
        name="newton_k64_v16", B=1, N=4, C=0, w_kind="orth", w_eps=0.0, w_scale=0.0, seed=9),
}

WORKLOAD_ORDER = ["tiny_fp32", "fp32_k64", "long_t16k_k64", "big_state_k128",
                  "fwd_bwd_k32_v128"]


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((bits >> 16) & 1)
    return ((bits + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """Host arrays of one workload.

    k, v, q are float32 arrays holding exactly the values the kernels read
    (already bf16-rounded when ``wl.bf16``); ``*_bits`` hold the bf16 bit
    patterns in that case.  Layouts: k, q [B,T,NQ,K] (NQ = wl.qk_heads); v [B,T,N,V];
    logit [B,T,N]; alpha, beta [N]; W [N,V,V] with (H W)[i,j] = sum_l H[i,l] W[l,j];
    w_r [N,V]; H0 [B,N,K,V] or None; dy [B,T,N,V] or None.
    """
    wl: Workload
    k: np.ndarray
    v: np.ndarray
    q: np.ndarray
    logit: np.ndarray
    alpha: np.ndarray | None
    beta: np.ndarray | None
    W: np.ndarray
    w_r: np.ndarray
    H0: np.ndarray | None = None
    dy: np.ndarray | None = None
    dHT: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    q_bits: np.ndarray | None = None


def _rounded(x: np.ndarray, bf16: bool):
    if not bf16:
        return x.astype(np.float32), None
    bits = round_to_bf16_bits(x)
    return bf16_bits_to_f32(bits), bits


def make_inputs(wl: Workload, seed: int | None = None, with_dy: bool | None = None,
                with_h0: bool = False, with_dht: bool = False) -> Inputs:
    """Draw one workload's inputs with numpy's PCG64 generator.

    ``with_h0`` / ``with_dht`` add a non-zero initial state / final-state
    gradient (drawn after everything else, so the other arrays do not change).
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B, T, N, K, V, NQ = wl.B, wl.T, wl.N, wl.K, wl.V, wl.qk_heads
    f32 = np.float32
    k = rng.standard_normal((B, T, NQ, K), dtype=f32) * f32(wl.kq_scale)
    v = rng.standard_normal((B, T, N, V), dtype=f32) * f32(wl.v_scale)
    q = rng.standard_normal((B, T, NQ, K), dtype=f32) * f32(wl.kq_scale)
    logit = rng.standard_normal((B, T, N), dtype=f32)
    if wl.gate == GATE_SIGMOID:
        logit = logit + f32(wl.g_mean)
        alpha = beta = None
    else:
        # alpha log-uniform on [0.1, 2]; beta uniform on [-2, 2]
        alpha = np.exp(rng.uniform(math.log(0.1), math.log(2.0), size=N)).astype(f32)
        beta = rng.uniform(-2.0, 2.0, size=N).astype(f32)
    if wl.w_kind == "ident":
        W = (np.eye(V, dtype=f32)[None]
             + f32(wl.w_eps) * rng.standard_normal((N, V, V), dtype=f32) * f32(wl.w_scale))
    elif wl.w_kind == "orth":
        G = rng.standard_normal((N, V, V)).astype(np.float64)
        W = np.empty((N, V, V), dtype=f32)
        for n in range(N):
            Q, R = np.linalg.qr(G[n])
            Q = Q * np.sign(np.diag(R))[None, :]
            W[n] = (0.9 * Q).astype(f32)
    else:
        raise ValueError(wl.w_kind)
    w_r = (rng.standard_normal((N, V), dtype=f32) * f32(0.1)).astype(f32)
    if with_dy is None:
        with_dy = wl.C > 0
    dy = rng.standard_normal((B, T, N, V), dtype=f32) if with_dy else None
    H0 = None
    dHT = None
    if with_h0:
        H0 = rng.uniform(-0.5, 0.5, size=(B, N, K, V)).astype(f32)
    if with_dht:
        dHT = rng.standard_normal((B, N, K, V), dtype=f32)
    k, kb = _rounded(k, wl.bf16)
    v, vb = _rounded(v, wl.bf16)
    q, qb = _rounded(q, wl.bf16)
    return Inputs(wl=wl, k=k, v=v, q=q, logit=logit, alpha=alpha, beta=beta,
                  W=W.astype(f32), w_r=w_r, H0=H0, dy=dy, dHT=dHT,
                  k_bits=kb, v_bits=vb, q_bits=qb)


def to_device(inp: Inputs, state_dtype="float32", device="cuda:0") -> dict:
    """torch tensors of one workload on `device` (no arithmetic: dtype casts only).

    k, v, q are bf16 (from the stored bit patterns) for bf16 workloads, else in
    the state dtype; every other array is in the state dtype.
    """
    import torch

    sd = {"float32": torch.float32, "float64": torch.float64}[state_dtype]
    nd = {"float32": np.float32, "float64": np.float64}[state_dtype]

    def t(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=nd)).to(device)

    if inp.wl.bf16:
        kv = {n: torch.from_numpy(getattr(inp, n + "_bits").view(np.int16)).view(torch.bfloat16)
              .to(device) for n in ("k", "v", "q")}
    else:
        kv = {n: t(getattr(inp, n)) for n in ("k", "v", "q")}
    out = dict(kv)
    for name in ("logit", "alpha", "beta", "W", "w_r", "H0", "dy", "dHT"):
        out[name] = t(getattr(inp, name))
    return out


# ---------------------------------------------------------------- block around the recurrence

@dataclasses.dataclass
class ConvInputs:
    """Prologue inputs: x [B, T, C] (exact bf16 values when bf16; x_bits the
    patterns), w [C, 4], bias [C], dout [B, T, C]."""
    x: np.ndarray
    w: np.ndarray
    bias: np.ndarray
    dout: np.ndarray
    x_bits: np.ndarray | None = None


def make_conv_inputs(B: int, T: int, C: int, seed: int = 11, bf16: bool = True) -> ConvInputs:
    """x ~ N(0, 1) (a projection output), w ~ N(0, 1/4) per tap (fan-in 4),
    bias ~ N(0, 0.1), dout ~ N(0, 1); draw order x, w, bias, dout."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f32 = np.float32
    x = rng.standard_normal((B, T, C), dtype=f32)
    w = rng.standard_normal((C, 4), dtype=f32) * f32(0.5)
    bias = rng.standard_normal(C, dtype=f32) * f32(0.1)
    dout = rng.standard_normal((B, T, C), dtype=f32)
    x, xb = _rounded(x, bf16)
    return ConvInputs(x=x, w=w, bias=bias, dout=dout, x_bits=xb)


@dataclasses.dataclass
class NormInputs:
    """Epilogue inputs: y [rows, D] (a readout), g_pre [rows, D] (exact bf16
    values when bf16), gamma [D], dout [rows, D]."""
    y: np.ndarray
    g_pre: np.ndarray
    gamma: np.ndarray
    dout: np.ndarray
    g_bits: np.ndarray | None = None


def make_norm_inputs(rows: int, D: int, seed: int = 12, bf16: bool = True) -> NormInputs:
    """y ~ N(0, 0.5), g_pre ~ N(0, 1), gamma ~ U(0.5, 1.5), dout ~ N(0, 1);
    draw order y, g_pre, gamma, dout."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f32 = np.float32
    y = rng.standard_normal((rows, D), dtype=f32) * f32(0.5)
    g = rng.standard_normal((rows, D), dtype=f32)
    gamma = rng.uniform(0.5, 1.5, D).astype(f32)
    dout = rng.standard_normal((rows, D), dtype=f32)
    g, gb = _rounded(g, bf16)
    return NormInputs(y=y, g_pre=g, gamma=gamma, dout=dout, g_bits=gb)
