"""GPU parity of the parallel-in-time Newton forward (m2rnn_newton_fwd) through
the C ABI, against the float64 Newton oracle iterate by iterate and against the
sequential recurrence once converged (pararnn-torch "ParaM2RNN" page,
"Parallel path" and "Agreement").

Inputs follow the workload recipes with a contractive transition W = 0.9 Q
(Q orthogonal), under which Newton converges quadratically; one case keeps the
near-identity W of the other workloads, where the pages' caveat applies and
the first iteration's residual grows instead.

Tolerances.  The GPU iterates are fp32: the guess is within ~1e-7 of the
oracle's, and each iteration adds the rounding of a linear recurrence whose
step maps contract, so the states stay within a few 1e-6; the readout sums K
rows.  Bounds: 1e-5 absolute on states, H_T and y (observed: below 1e-6),
and 1e-5 + 1e-3 |ref| on each iterate's residual (a converged fp32 residual
bottoms out near 1e-7, the float64 one near 1e-16).  Shapes cover V = 16,
32, 48, 64; K with a ragged last slab; shared and per-head q/k; a given H_0; bf16 and fp32 inputs; chunks of one
step and of many steps; a single chunk (no scan); the linearisation fused into
the applying solve and separate; and the full Newton workload.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from m2rnn_inputs import NEWTON_WORKLOADS, WORKLOADS, make_inputs, to_device
from matrix_state_nonlinear_amd import m2rnn_fwd, m2rnn_gates, m2rnn_newton_fwd

pytestmark = pytest.mark.gpu

TOL = 1e-5


def np_(t):
    return t.detach().cpu().numpy().astype(np.float64)


def maxerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def orth_case(B, T, N, K, V, NQ, bf16=True, seed=11, with_h0=False):
    wl = WORKLOADS["multi_value_k64_v16"].replace(
        B=B, T=T, N=N, K=K, V=V, NQ=NQ, bf16=bf16, C=0, w_kind="orth", w_eps=0.0, w_scale=0.0,
        kq_scale=1 / math.sqrt(K), v_scale=1 / math.sqrt(V), seed=seed)
    return wl, make_inputs(wl, with_h0=with_h0)


def run(wl, inp, iters, sd="float32"):
    d = to_device(inp, sd)
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
    out = m2rnn_newton_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d.get("H0"), iters=iters,
                           want_states=True, want_residual=True)
    torch.cuda.synchronize()
    return d, f, out


def oracle_newton(wl, inp, iters):
    fo = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
    return oracle.newton_forward(inp.k, inp.v, inp.q, fo, inp.W, inp.w_r, inp.H0, iters=iters)


def check_against_oracle(wl, inp, iters, out, tag):
    y, HT, states, res = out
    o = oracle_newton(wl, inp, iters)
    X = np.moveaxis(o["X"][1:], 0, 2)          # [B, N, T, K, V]
    ex, ey = maxerr(np_(states), X), maxerr(np_(y), o["y"])
    eh = maxerr(np_(HT), o["X"][-1])
    r = np_(res)
    er = float(np.max(np.abs(r - o["res"]) - 1e-3 * np.abs(o["res"])))
    print(f"{tag} iters={iters}: states {ex:.1e} y {ey:.1e} HT {eh:.1e} "
          f"res gpu {r[-1]:.1e} oracle {o['res'][-1]:.1e}")
    assert ex <= TOL and ey <= TOL and eh <= TOL, (ex, ey, eh)
    assert er <= TOL, (r, o["res"])
    return o


@pytest.mark.parametrize("V", [16, 32, 48, 64])
@pytest.mark.parametrize("K,NQ", [(20, 1), (33, 2)])
def test_newton_iterates_match_oracle(V, K, NQ):
    # B N = 4 units: chunks of a single step (a long scan over 70 chunks)
    wl, inp = orth_case(B=2, T=70, N=2, K=K, V=V, NQ=NQ)
    for iters in (0, 1, 3):
        _, _, out = run(wl, inp, iters)
        check_against_oracle(wl, inp, iters, out, f"K={K} V={V} NQ={NQ}")


@pytest.mark.parametrize("bf16", [True, False])
def test_newton_long_chunks_with_h0(bf16):
    # 4 units of 64 rows, V = 16: 55 chunks of 55 steps (the last one of 30)
    wl, inp = orth_case(B=1, T=3000, N=4, K=64, V=16, NQ=1, bf16=bf16, with_h0=True)
    _, _, out = run(wl, inp, 3)
    check_against_oracle(wl, inp, 3, out, f"T=3000 bf16={bf16}")


@pytest.mark.parametrize("V", [16, 64])
def test_newton_fused_linearisation_matches_oracle(V):
    # 16 units of 64 rows: the applying solve has B N P ceil(K / 16) >= 1024
    # waves, so it linearises each new iterate itself (the separate pass is
    # used below that); iterates and residuals against the oracle
    wl, inp = orth_case(B=4, T=400, N=4, K=64, V=V, NQ=2, with_h0=True)
    for iters in (1, 3):
        _, _, out = run(wl, inp, iters)
        check_against_oracle(wl, inp, iters, out, f"fused V={V}")


@pytest.mark.parametrize("B,T,N,K,V", [(1, 1, 1, 1, 16), (2, 2, 1, 3, 48), (1, 5, 2, 17, 32)])
def test_newton_small_edges(B, T, N, K, V):
    # one step, one state row, sequences shorter than a prefetch group
    wl, inp = orth_case(B=B, T=T, N=N, K=K, V=V, NQ=1, with_h0=True)
    for iters in (0, 1, 2):
        _, _, out = run(wl, inp, iters)
        check_against_oracle(wl, inp, iters, out, f"B={B} T={T} N={N} K={K} V={V}")


def test_newton_single_chunk_fused():
    # 256 units x 64 rows: a single chunk, and the applying solve's waves cover
    # the device, so the fused linearisation runs from H_0 with no scan
    wl, inp = orth_case(B=4, T=20, N=64, K=64, V=16, NQ=1, with_h0=True)
    _, _, out = run(wl, inp, 2)
    check_against_oracle(wl, inp, 2, out, "one chunk, fused")


def test_newton_single_chunk():
    # 128 units x 64 rows fill the device: one chunk, the update solved directly
    wl, inp = orth_case(B=4, T=40, N=32, K=64, V=16, NQ=1)
    _, _, out = run(wl, inp, 2)
    check_against_oracle(wl, inp, 2, out, "one chunk")


@pytest.mark.parametrize("V", [16, 64])
def test_newton_converged_equals_the_sequential_forward(V):
    wl, inp = orth_case(B=2, T=500, N=2, K=40, V=V, NQ=2, with_h0=True)
    d, f, (y, HT, states, res) = run(wl, inp, 4)
    y_seq, HT_seq, _ = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"])
    torch.cuda.synchronize()
    fo = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
    o = oracle.forward(inp.k, inp.v, inp.q, fo, inp.W, inp.w_r, inp.H0)
    e_seq = max(maxerr(np_(y), np_(y_seq)), maxerr(np_(HT), np_(HT_seq)))
    e_or = max(maxerr(np_(y), o["y"]), maxerr(np_(HT), o["HT"]))
    print(f"V={V}: vs sequential kernel {e_seq:.1e}, vs oracle {e_or:.1e}, residual {np_(res)}")
    assert e_seq <= TOL and e_or <= TOL
    assert float(np_(res)[-1]) < 1e-5


def test_newton_reports_divergence_of_an_expanding_linearisation():
    # the near-identity W of the long-context workload: the first linear solve
    # grows over the sequence and the residual jumps (the oracle's does too)
    wl = WORKLOADS["long_t16k_k64"].replace(B=1, T=2048, N=2)
    inp = make_inputs(wl)
    _, _, (_, _, _, res) = run(wl, inp, 1)
    o = oracle_newton(wl, inp, 1)
    r = np_(res)
    print(f"residual gpu {r}, oracle {o['res']}")
    assert o["res"][1] > 100 * o["res"][0]
    assert r[1] > 100 * r[0]
    assert abs(r[0] - o["res"][0]) <= 1e-5


def test_newton_workload_full_size():
    """The Newton workload at full size (B = 1, T = 16384, four value heads,
    K = 64, V = 16, shared q/k): after three iterations the readout matches the
    oracle's sequential forward and the sequential kernel, and the residual has
    fallen to the fp32 floor."""
    wl = NEWTON_WORKLOADS["newton_k64_v16"]
    inp = make_inputs(wl)
    d, f, (y, HT, _, res) = run(wl, inp, 3)
    y_seq, HT_seq, _ = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"])
    torch.cuda.synchronize()
    fo = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
    o = oracle.forward(inp.k, inp.v, inp.q, fo, inp.W, inp.w_r)
    e_or = max(maxerr(np_(y), o["y"]), maxerr(np_(HT), o["HT"]))
    e_seq = max(maxerr(np_(y), np_(y_seq)), maxerr(np_(HT), np_(HT_seq)))
    print(f"full size: vs oracle {e_or:.1e}, vs sequential kernel {e_seq:.1e}, residual {np_(res)}")
    assert e_or <= TOL and e_seq <= TOL
    assert float(np_(res)[-1]) < 1e-5


@pytest.mark.parametrize("B,T,N", [(0, 5, 2), (2, 0, 2), (2, 5, 0)])
def test_newton_empty(B, T, N):
    dev = "cuda:0"
    k = torch.zeros((B, T, N, 20), device=dev)
    v = torch.zeros((B, T, N, 16), device=dev)
    f = torch.zeros((B, T, N), device=dev)
    W = torch.zeros((N, 16, 16), device=dev)
    w_r = torch.zeros((N, 16), device=dev)
    H0 = torch.rand((B, N, 20, 16), device=dev)
    y, HT, _, res = m2rnn_newton_fwd(k, v, k, f, W, w_r, H0, iters=2, want_residual=True)
    torch.cuda.synchronize()
    assert torch.equal(HT, H0)
    assert torch.equal(res, torch.zeros(3, device=dev))
    assert tuple(y.shape) == (B, T, N, 16)
