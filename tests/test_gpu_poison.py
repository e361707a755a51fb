"""Race and coverage check: every output and workspace is filled with NaN
before the call, then the results are compared with the float64 oracle.

An output element the kernels never write, or a workspace element read before
it is written (a partial sum, a chunk-start state, a staging slot), would
carry the NaN into the results and fail the comparison.  The cases reach the
edges where such gaps hide: K and V that leave a ragged last slab and tile, T
that leaves ragged staging chunks and checkpoint intervals, a checkpoint
interval C that does not divide the backward's chunk length (chunk starts
recomputed into the workspace), q/k shared across value heads (dk, dq summed
from workspace partials), the decode step, and the Newton forward.

Tolerances are those of the small-shape parity tests: 2e-5 max-abs on fp32
forward outputs, tau = 1e-4 of max(1, |ref|) on fp32 gradients, 1e-11 / 1e-10
for the fp64 state.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from m2rnn_inputs import WORKLOADS, make_inputs, to_device
from matrix_state_nonlinear_amd import (m2rnn_bwd, m2rnn_fwd, m2rnn_gates, m2rnn_newton_fwd,
                                        m2rnn_step, m2rnn_workspace_bytes,
                                        m2rnn_newton_workspace_bytes)

pytestmark = pytest.mark.gpu

TOL_Y = {"float32": 2e-5, "float64": 1e-11}
TAU_G = {"float32": 1e-4, "float64": 1e-10}
DT = {"float32": torch.float32, "float64": torch.float64}


def np_(t):
    return t.detach().cpu().numpy().astype(np.float64)


def maxerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def nan_tensor(shape, dtype, dev="cuda:0"):
    return torch.full(shape, float("nan"), dtype=dtype, device=dev)


def nan_workspace(nbytes, dev="cuda:0"):
    """A byte workspace whose every float (and double) reads as NaN (0xFF bytes)."""
    return torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=dev)


def case(K, V, T, NQ=0, N=2, B=2, seed=5):
    wl = WORKLOADS["fwd_bwd_k32_v128"].replace(B=B, T=T, N=N, K=K, V=V, NQ=NQ,
                                               kq_scale=1 / math.sqrt(K), v_scale=1 / math.sqrt(V),
                                               w_scale=1 / math.sqrt(V), seed=seed)
    return wl, make_inputs(wl, with_dy=True, with_h0=True, with_dht=True)


def poisoned_fwd_bwd(wl, inp, sd, C, stored_rc):
    d = to_device(inp, sd)
    dt = DT[sd]
    B, T, N, K, V, NQ = wl.B, wl.T, wl.N, wl.K, wl.V, wl.qk_heads
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"], out=nan_tensor((B, T, N), dt))
    y = nan_tensor((B, T, N, V), dt)
    HT = nan_tensor((B, N, K, V), dt)
    ck = nan_tensor((B, N, math.ceil(T / C), K, V), dt)
    rc = nan_tensor((B, N, T, K, V), dt) if stored_rc else None
    wsf = nan_workspace(m2rnn_workspace_bytes(False, B, T, N, NQ, K, V, C, dt))
    m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"], C, out=(y, HT, ck),
              workspace=wsf, rc_out=rc)
    names = {"dk": (B, T, NQ, K), "dv": (B, T, N, V), "dq": (B, T, NQ, K), "dlogit": (B, T, N),
             "dW": (N, V, V), "dw_r": (N, V), "dalpha": (N,), "dbeta": (N,), "dH0": (B, N, K, V)}
    out = {k_: nan_tensor(s, dt) for k_, s in names.items()}
    wsb = nan_workspace(m2rnn_workspace_bytes(True, B, T, N, NQ, K, V, C, dt))
    g = m2rnn_bwd(d["k"], d["v"], d["q"], wl.gate, d["logit"], d["alpha"], d["beta"], f, d["W"],
                  d["w_r"], d["H0"], ck, C, d["dy"], d["dHT"], workspace=wsb, rc=rc, out=out)
    torch.cuda.synchronize()
    return f, y, HT, ck, rc, g


def check_against_oracle(wl, inp, sd, C, f, y, HT, ck, rc, g, label):
    fo = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
    o = oracle.forward(inp.k, inp.v, inp.q, fo, inp.W, inp.w_r, inp.H0, C=C, keep_states=True)
    assert maxerr(np_(f), fo) <= (2e-7 if sd == "float32" else 1e-15), label
    errs = {"y": maxerr(np_(y), o["y"]), "HT": maxerr(np_(HT), o["HT"]),
            "ckpt": maxerr(np_(ck), o["ckpt"])}
    if rc is not None:
        errs["rc"] = maxerr(np_(rc), np.transpose((1.0 - o["Z"]) / 2.0, (1, 2, 0, 3, 4)))
    ref = oracle.backward(inp.k, inp.v, inp.q, fo, inp.W, inp.w_r, inp.dy, inp.H0, inp.dHT,
                          gate_kind=wl.gate, logit=inp.logit, alpha=inp.alpha, beta=inp.beta)
    gerr = {}
    for name, r in ref.items():
        if name == "df":
            continue
        gerr[name] = maxerr(np_(g[name]), r) / max(1.0, float(np.max(np.abs(r))))
    print(label, {k_: f"{v_:.1e}" for k_, v_ in {**errs, **gerr}.items()})
    # NaN compares false, so an unwritten element fails these bounds
    assert all(v_ <= TOL_Y[sd] for v_ in errs.values()), errs
    assert all(v_ <= TAU_G[sd] for v_ in gerr.values()), gerr


# (K, V, T, NQ, C): ragged slab/tile/chunk edges; C not dividing the backward's
# chunk length (4 steps for V <= 96, 2 at V = 128) or dividing it; shared q/k;
# at V > 112 intervals swept by the main kernel (C = 4, 6: its ring workspace)
CASES = [
    (17, 40, 45, 0, 7),
    (33, 100, 29, 0, 5),
    (40, 72, 70, 0, 3),
    (48, 128, 37, 0, 3),
    (16, 16, 33, 0, 4),
    (24, 20, 23, 1, 6),
    (64, 16, 41, 1, 2),
    (20, 24, 19, 2, 1),
    (9, 10, 27, 0, 3),
    (40, 128, 45, 0, 4),
    (24, 120, 70, 1, 6),
]


@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("K,V,T,NQ,C", CASES)
def test_poisoned_outputs_and_workspace_forward_backward(K, V, T, NQ, C, sd):
    wl, inp = case(K, V, T, NQ=NQ, N=4 if NQ else 2)
    for stored_rc in (False, True):
        f, y, HT, ck, rc, g = poisoned_fwd_bwd(wl, inp, sd, C, stored_rc)
        check_against_oracle(wl, inp, sd, C, f, y, HT, ck, rc, g,
                             f"K{K} V{V} T{T} NQ{NQ} C{C} {sd} rc={stored_rc}")


@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("K,V,NQ,B", [(17, 40, 0, 5), (64, 64, 1, 9), (33, 100, 0, 3),
                                      (64, 16, 1, 13)])
def test_poisoned_decode_step(K, V, NQ, B, sd):
    wl, inp = case(K, V, 1, NQ=NQ, N=4 if NQ else 2, B=B)
    d = to_device(inp, sd)
    dt = DT[sd]
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])[:, 0].contiguous()
    H = d["H0"].clone()
    y = nan_tensor((B, wl.N, V), dt)
    m2rnn_step(H, d["k"][:, 0].contiguous(), d["v"][:, 0].contiguous(), d["q"][:, 0].contiguous(),
               f, d["W"], d["w_r"], out=y)
    torch.cuda.synchronize()
    fo = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)[:, 0]
    Hn, yo = oracle.decode_step(inp.H0, inp.k[:, 0], inp.v[:, 0], inp.q[:, 0], fo, inp.W, inp.w_r)
    ey, eh = maxerr(np_(y), yo), maxerr(np_(H), Hn)
    print(f"decode K{K} V{V} NQ{NQ} B{B} {sd}: y {ey:.1e} H {eh:.1e}")
    assert ey <= TOL_Y[sd] and eh <= TOL_Y[sd]


@pytest.mark.parametrize("K,V,T,NQ", [(20, 16, 37, 1), (64, 48, 50, 0), (33, 32, 70, 2)])
def test_poisoned_newton(K, V, T, NQ):
    N = 4 if NQ else 2
    wl = WORKLOADS["multi_value_k64_v16"].replace(
        B=2, T=T, N=N, K=K, V=V, NQ=NQ, bf16=True, C=0, w_kind="orth", w_eps=0.0, w_scale=0.0,
        kq_scale=1 / math.sqrt(K), v_scale=1 / math.sqrt(V), seed=13)
    inp = make_inputs(wl, with_h0=True)
    d = to_device(inp, "float32")
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
    iters = 3
    B = wl.B
    y = nan_tensor((B, T, N, V), torch.float32)
    HT = nan_tensor((B, N, K, V), torch.float32)
    X = nan_tensor((B, N, T, K, V), torch.float32)
    res = nan_tensor((iters + 1,), torch.float32)
    ws = nan_workspace(m2rnn_newton_workspace_bytes(B, T, N, K, V, True))
    m2rnn_newton_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"], iters=iters,
                     out=(y, HT, X, res), workspace=ws)
    torch.cuda.synchronize()
    fo = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
    o = oracle.newton_forward(inp.k, inp.v, inp.q, fo, inp.W, inp.w_r, inp.H0, iters=iters)
    errs = {"y": maxerr(np_(y), o["y"]), "HT": maxerr(np_(HT), o["X"][-1]),
            "states": maxerr(np_(X), np.moveaxis(o["X"][1:], 0, 2))}
    rr = np_(res)
    ok_res = bool(np.all(np.abs(rr - o["res"]) <= 1e-5 + 1e-3 * np.abs(o["res"])))
    print(f"newton K{K} V{V} T{T} NQ{NQ}:", {k_: f"{v_:.1e}" for k_, v_ in errs.items()}, rr)
    assert all(v_ <= 1e-5 for v_ in errs.values()), errs
    assert ok_res, (rr, o["res"])
